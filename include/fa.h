/*
 * fa.h - C ABI of the MI355X (gfx950) fused exact-attention library (libfa.so).
 *
 * The operation is exact attention O = softmax(scale * Q K^T [+ causal mask]) V
 * with its per-row logsumexp L = m + ln(l), computed by a fused, tiled forward
 * pass that never writes the N x N score or probability matrix to memory
 * (the three steps and the single fused kernel: 91haoming.cn FlashAttention
 * v1-v3 article, "FlashAttention v1 / attention implementation improvements";
 * L kept instead of (m, l): same article, "FlashAttention v2 / forward pass
 * improvements").
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers (HBM) unless stated otherwise; the caller
 *     owns every buffer. The library allocates nothing and never synchronises:
 *     all work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream), so results are ready once the stream is. Kernels
 *     launch on the calling thread's current HIP device: the buffers and the
 *     stream must belong to it.
 *   - Tensors are dense row-major: q/k/v/o [B, H, N, d], lse [B, H, N] fp32.
 *   - Natural logarithms; L is in the units of the scaled scores.
 *   - causal is 0 or 1 (FA_ERR_UNSUPPORTED otherwise); causal = 1: key j is
 *     visible to query i iff j <= i (top-left aligned, diagonal visible;
 *     queries and keys have the same length N).
 *   - Arguments are checked on the host before anything is launched. A failed
 *     check returns its status and has no side effect. A launch failure
 *     returns FA_ERR_HIP. Device-side contracts (block_table entries, ctx_lens)
 *     are the caller's to keep and are not checked by the attention calls;
 *     fa_check_paged_tables checks them on the device when asked.
 *   - Stateless and re-entrant; calls on different streams may overlap.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL_PTR = 1,     /* a required pointer is NULL */
    FA_ERR_BAD_SHAPE = 2,    /* a size is <= 0 or out of the supported range */
    FA_ERR_UNSUPPORTED = 3,  /* head size / page size / flag value not supported */
    FA_ERR_WORKSPACE = 4,    /* workspace too small */
    FA_ERR_HIP = 5,          /* the HIP runtime reported an error at launch */
    FA_ERR_NO_PAGES = 6,     /* block manager: no free page left */
    FA_ERR_STATE = 7,        /* block manager: invalid state, or the sequence is
                                absent / already present */
    FA_ERR_SCRATCH_LIMIT = 8 /* the call needs more workspace than the library's
                                static buffer holds (fa_paged_decode_noalloc) */
} fa_status;

/*
 * Fused attention forward, bf16 in / bf16 out (fp32 accumulation).
 * q, k, v: bf16 [B, H, N, d]; o: bf16 [B, H, N, d] (rounded to nearest even);
 * lse: fp32 [B, H, N] (may be NULL to skip it).
 * d in {64, 128}; B, H, N >= 1 with B*H*N*d < 2^31.
 * q, k and v must be finite (the kernel is built without NaN and infinity
 * semantics; a NaN or infinite input leaves O and L undefined), and the
 * weighted sums must stay in fp32 range: |v| < 2^64.
 * Tiling (row blocks of Q in parallel, K/V tiles streamed through on-chip
 * memory, online softmax with one final 1/l): "FlashAttention系列优化",
 * FlashAttentionV2 section and its equations.
 */
fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int H, int N, int d, float scale, int causal, void *stream);

/*
 * Same operation in fp32 (fp32 in, fp32 out, fp32 arithmetic), any 1 <= d <= 128.
 * The correctness path used for the worked example of "FlashAttention系列优化"
 * (16 x 8, scale 1).
 */
fa_status fa_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                     int B, int H, int N, int d, float scale, int causal, void *stream);

/*
 * FP8 attention forward with per-block scales (FlashAttention-3 block
 * quantisation: "FlashAttention系列优化", FlashAttentionV3 / FP低精度).
 * q8, k8, v8: OCP E4M3FN bytes [B, H, N, d]; q_scale, k_scale, v_scale: fp32
 * [B, H, ceil(N/128)], one per (batch, head, 128-token block); the value of an
 * element is decode(x8) * scale of its block. o: bf16 [B, H, N, d];
 * lse: fp32 [B, H, N] or NULL. d in {64, 128}. Codes are finite (no 0x7f / 0xff)
 * and scales finite and >= 0; a q_scale, k_scale or v_scale entry below
 * 2^-100 (zero included) acts as 2^-100, which keeps the score multiplier
 * positive and moves O by far less than a bf16 ulp. Q.K^T runs on fp8 MFMA;
 * P.V runs on bf16 MFMA with V widened exactly from E4M3 to bf16.
 */
fa_status fa_fwd_fp8(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8,
                     const float *q_scale, const float *k_scale, const float *v_scale,
                     void *o, float *lse, int B, int H, int N, int d,
                     float scale, int causal, void *stream);

/*
 * Fused incoherent processing and FP8 block quantisation: the producer of
 * fa_fwd_fp8's inputs (FlashAttention-3 FP8: "FlashAttention系列优化",
 * FlashAttentionV3 / FP低精度, where Q and K are multiplied by a random
 * orthogonal matrix before block quantisation so that outliers spread; the
 * scores (QR)(KR)^T = QK^T do not change).
 *   x: bf16 [B, H, N, d], device; rot: bf16 [d, d] row-major R, or NULL for
 *     no rotation (V, or Q and K without incoherent processing);
 *   codes: uint8 [B, H, N, d], OCP E4M3FN; scales: fp32 [B, H, ceil(N/128)].
 *   With y = x R (fp32 sums of exact bf16 products), for each 128-token block
 *   of each (b, h): scale = max |y| / 448 over the block (1 if that is 0) and
 *   code = E4M3FN(clamp(y / scale, -448, 448)), rounded to nearest even.
 *   The last block of a row may be short; it is scaled on its own tokens.
 * d == 128; x, rot and codes 16-byte aligned, scales 4-byte aligned
 * (FA_ERR_UNSUPPORTED otherwise); x must be finite. Device pointers; the
 * call is asynchronous on stream.
 */
fa_status fa_quantize_fp8(const void *x, const void *rot, uint8_t *codes, float *scales, int B, int H,
                          int N, int d, void *stream);

/*
 * The three inputs of fa_fwd_fp8 in one launch: Q and K multiplied by rot
 * (the one R that leaves QK^T unchanged; NULL for no rotation), V not
 * rotated, each block-quantised as fa_quantize_fp8 does (same pages). The
 * codes and scales are bit for bit those of three fa_quantize_fp8 calls
 * (q with rot, k with rot, v with NULL); one grid covers all three, so the
 * start and tail of two launches are saved.
 *   q, k, v: bf16 [B, H, N, d], device; rot: bf16 [d, d] or NULL;
 *   q_codes, k_codes, v_codes: uint8 [B, H, N, d]; q_scales, k_scales,
 *   v_scales: fp32 [B, H, ceil(N/128)]. Outputs must not overlap the inputs
 *   or each other.
 * Errors and requirements as for fa_quantize_fp8 (FA_ERR_NULL_PTR for any
 * NULL pointer other than rot). Asynchronous on stream.
 */
fa_status fa_quantize_fp8_qkv(const void *q, const void *k, const void *v, const void *rot, uint8_t *q_codes,
                              uint8_t *k_codes, uint8_t *v_codes, float *q_scales, float *k_scales,
                              float *v_scales, int B, int H, int N, int d, void *stream);

/*
 * Block-sparse attention forward with optional dropout, bf16 (d == 128).
 * Block-sparse FlashAttention (91haoming.cn FlashAttention v1-v3 article, v1
 * results): the fused tile loop runs only over the (query block, key block)
 * pairs that block_mask keeps; blocks are 128 x 128 tokens.
 *   block_mask: device uint8 [nb, nb], nb = ceil(N / 128), shared by every
 *     batch and head; entry [i][j] != 0 keeps key block j for query block i.
 *     With causal = 1, keys after the query are masked as well. A query with
 *     no kept key gets O = 0 and L = -inf.
 *   dropout_p in [0, 1): each softmax weight P_ij is kept with probability
 *     1 - dropout_p and scaled by 1 / (1 - dropout_p) (the "masking and
 *     dropout" fused into the kernel, same article); L and the normaliser are
 *     those before dropout. The decision uses Philox4x32-10 (Salmon et al.,
 *     SC 2011) with key (seed & 0xffffffff, seed >> 32) and counter
 *     (j / 4, i, b * H + h, 0): P_ij is dropped iff word j % 4 of the output
 *     is below floor(dropout_p * 2^32).
 * Other arguments as for fa_fwd; N <= 131072.
 */
fa_status fa_fwd_block_sparse(const void *q, const void *k, const void *v, const uint8_t *block_mask,
                              void *o, float *lse, int B, int H, int N, int d, float scale, int causal,
                              float dropout_p, uint64_t seed, void *stream);

/*
 * Bytes of device workspace fa_bwd needs (two fp32 values per row: -L_i/scale
 * and -D_i with D_i = dO_i . O_i; B * H * N * 8). Returns 0 for unsupported
 * sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Attention backward for fa_fwd, bf16 in / bf16 out (fp32 accumulation):
 * gradients of a loss that reaches the attention through O only.
 * Recomputation (FlashAttention v1 backward and the v2 "keep only L" change:
 * 91haoming.cn FlashAttention v1-v3 article; backward part of "Flash
 * Attention 再学习"): the tiles of P are rebuilt on chip from Q, K and the
 * logsumexp L of the forward pass; work is parallel over key blocks (each owns
 * its dK, dV) and, for dQ, over query blocks, without atomics.
 *   q, k, v, o, dout: bf16 [B, H, N, d] (o: the forward output);
 *   lse: fp32 [B, H, N], the forward pass's L (natural log);
 *   dq, dk, dv: bf16 [B, H, N, d], written (not accumulated);
 *   workspace: device memory of at least fa_bwd_workspace_bytes(B, H, N, d)
 *   bytes; contents on entry do not matter.
 * d in {64, 128}; the other sizes, scale and causal are as for fa_fwd.
 */
fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 const void *dout, void *dq, void *dk, void *dv, int B, int H, int N, int d,
                 float scale, int causal, void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * Bytes of device workspace fa_paged_decode needs for these sizes (the split
 * partials (m, l, unscaled O) of every (sequence, head, KV chunk of 32
 * pages), then per (sequence, chunk) a 64-bit hash, a partner index and a
 * pair-list slot, and a hash table of chunk classes with twice as many slots
 * as chunks (rounded up to a power of two), used to read chunks shared
 * between sequences once). Returns 0 for unsupported sizes.
 */
size_t fa_paged_decode_workspace_bytes(int num_seqs, int H, int d, int page_size,
                                       int max_blocks_per_seq);

/*
 * Decode attention over a paged KV cache (PagedAttention block table:
 * "FlashAttention系列优化", PagedAttention section), one query token per
 * sequence, split over KV chunks and merged with the same rescale identity as
 * the FlashAttention-2 accumulator.
 *   q:        bf16 [num_seqs, H, d]
 *   kcache,
 *   vcache:   bf16 [num_pages, H, page_size, d]; token t of sequence s lives in
 *             page block_table[s][t / page_size], slot t % page_size
 *   block_table: int32 [num_seqs, max_blocks_per_seq]; entries for the first
 *             ceil(ctx_lens[s] / page_size) blocks must be in [0, num_pages);
 *             the rest are ignored (pad with -1). Pages may be shared.
 *   ctx_lens: int32 [num_seqs], each in [1, max_blocks_per_seq * page_size]
 *             (0 gives O = 0 and L = -inf). Slots past the context in the last
 *             page may be loaded (they lie inside the page) but never
 *             contribute, whatever they hold.
 *   o:        bf16 [num_seqs, H, d];  lse: fp32 [num_seqs, H] or NULL.
 *   workspace: device memory of at least fa_paged_decode_workspace_bytes(...)
 *             bytes; contents on entry do not matter.
 * d == 128, page_size == 16, num_seqs and H <= 65535, and at most 2^29
 * chunks of 32 blocks: num_seqs * ceil(max_blocks_per_seq / 32) <= 2^29 (e.g.
 * 65535 sequences of up to 262144 blocks); FA_ERR_BAD_SHAPE otherwise, and
 * fa_paged_decode_workspace_bytes returns 0. ctx_lens and block_table are read
 * only on the device (no host synchronisation).
 */
fa_status fa_paged_decode(const void *q, const void *kcache, const void *vcache,
                          const int32_t *block_table, const int32_t *ctx_lens,
                          void *o, float *lse, int num_seqs, int H, int d,
                          int page_size, int max_blocks_per_seq, int num_pages,
                          float scale, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * fa_paged_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments, kernels and results as fa_paged_decode, but the
 * workspace is a static device buffer inside the library
 * (fa_noalloc_scratch_bytes() = 80 MiB per device, held from the time the
 * library's code is loaded on a device until the process ends). No call
 * allocates or frees memory.
 * Sizes whose fa_paged_decode_workspace_bytes(...) exceeds that buffer return
 * FA_ERR_SCRATCH_LIMIT before anything is launched. That bound is about
 * num_seqs * H * ceil(max_blocks_per_seq / 32) <= 161000 (for example 64
 * sequences x 32 heads with max_blocks_per_seq up to 2496, i.e. contexts up to
 * 39936 tokens).
 * Every call on one device shares that device's buffer: calls that can overlap
 * on one device (different streams, or several host threads) race and must be
 * ordered by the caller; calls on one stream are ordered by the stream. The
 * buffer keeps the last call's contents; each call writes every part of it
 * that it reads, so nothing needs clearing.
 */
size_t fa_noalloc_scratch_bytes(void);
fa_status fa_paged_decode_noalloc(const void *q, const void *kcache, const void *vcache,
                                  const int32_t *block_table, const int32_t *ctx_lens,
                                  void *o, float *lse, int num_seqs, int H, int d,
                                  int page_size, int max_blocks_per_seq, int num_pages,
                                  float scale, void *stream);

/*
 * Paged (chunked) prefill: the n_new newest tokens of each sequence attend to
 * its paged KV cache (PagedAttention block table, "FlashAttention系列优化";
 * the tile loop of the FlashAttention-2 forward of the same page). Query i of
 * sequence s is the token at position ctx_lens[s] - n_new + i and sees cached
 * tokens 0 .. that position (causal); its own K/V must already be in the
 * cache. A query whose position is negative sees nothing (O = 0, L = -inf).
 *   q:        bf16 [num_seqs, H, n_new, d]
 *   kcache, vcache, block_table, ctx_lens: as for fa_paged_decode
 *   o:        bf16 [num_seqs, H, n_new, d];  lse: fp32 [num_seqs, H, n_new] or NULL
 * d == 128, page_size == 16, num_seqs * H <= 65535.
 */
fa_status fa_paged_prefill(const void *q, const void *kcache, const void *vcache,
                           const int32_t *block_table, const int32_t *ctx_lens, void *o, float *lse,
                           int num_seqs, int H, int n_new, int d, int page_size,
                           int max_blocks_per_seq, int num_pages, float scale, void *stream);

/*
 * Paged KV block manager (PagedAttention, "FlashAttention系列优化": logical
 * blocks of a sequence map to physical pages through a block table; pages are
 * taken on demand; sequences share pages with reference counts and
 * copy-on-write). Host-side bookkeeping only: the state lives in host memory
 * the caller provides (fa_bm_state_bytes), the library allocates nothing, and
 * the only device work is fa_copy_pages. A failed call returns its status and
 * changes nothing. Not thread-safe for one state; separate states are
 * independent.
 *   fa_bm_init:         empty pool of num_pages pages of page_size tokens for
 *                       sequence ids 0..max_seqs-1 of up to max_blocks_per_seq
 *                       blocks each
 *   fa_bm_add_seq:      a new sequence of num_tokens tokens on fresh pages
 *   fa_bm_fork:         child maps every block of parent (refcounts + 1)
 *   fa_bm_append_token: reserve the slot of one more token of seq: a fresh page
 *                       when the token starts a block; when its block's page is
 *                       shared, seq gets a private page and (*cow_src,
 *                       *cow_dst) name the page to copy (fa_copy_pages) before
 *                       the token's K/V are written; otherwise both are -1
 *   fa_bm_free_seq:     drop seq's references; pages reaching 0 are free again
 *   fa_bm_block_table:  host block_table [max_seqs, max_blocks_per_seq] (-1
 *                       padded) and ctx_lens [max_seqs] (0 for absent ids), the
 *                       arguments of fa_paged_decode / fa_paged_prefill once
 *                       copied to the device
 */
size_t fa_bm_state_bytes(int num_pages, int max_seqs, int max_blocks_per_seq);
fa_status fa_bm_init(void *state, size_t state_bytes, int num_pages, int max_seqs,
                     int max_blocks_per_seq, int page_size);
fa_status fa_bm_add_seq(void *state, int seq, int num_tokens);
fa_status fa_bm_fork(void *state, int parent, int child);
fa_status fa_bm_append_token(void *state, int seq, int32_t *cow_src, int32_t *cow_dst);
fa_status fa_bm_free_seq(void *state, int seq);
int fa_bm_num_free_pages(const void *state);          /* -1 for an invalid state */
int fa_bm_seq_len(const void *state, int seq);        /* -1 for an absent sequence */
int fa_bm_page_refcount(const void *state, int page); /* -1 for a bad page id */
fa_status fa_bm_block_table(const void *state, int32_t *block_table, int32_t *ctx_lens);

/*
 * Copy n whole pages (every head, page_size tokens, d channels, bf16) of both
 * caches [num_pages, H, page_size, d]: page src[i] -> page dst[i]. src, dst:
 * device int32 [n], ids in [0, num_pages) (not checked on the device), no dst
 * repeated and no dst among the src. The copies of copy-on-write.
 */
fa_status fa_copy_pages(void *kcache, void *vcache, const int32_t *src, const int32_t *dst, int n,
                        int num_pages, int H, int d, int page_size, void *stream);

/*
 * Debug check of the paged calls' device-side contract (PagedAttention block
 * table, "FlashAttention系列优化"): an entry outside the page pool makes
 * fa_paged_decode / fa_paged_prefill read outside the caches, so a caller that
 * builds tables itself can run this first, on the same stream.
 *   block_table: device int32 [num_seqs, max_blocks_per_seq]
 *   ctx_lens:    device int32 [num_seqs]
 *   result:      device int32 [2], written by the call (contents on entry do
 *                not matter): result[0] = number of sequences s whose
 *                ctx_lens[s] is outside [0, max_blocks_per_seq * page_size]
 *                or one of whose first ceil(ctx_lens[s] / page_size) entries
 *                is outside [0, num_pages); result[1] = the smallest such s,
 *                or -1 when there is none. Entries past a sequence's used
 *                blocks are not read.
 * Any page_size >= 1. Pointers 4-byte aligned (FA_ERR_UNSUPPORTED otherwise).
 * Two kernel launches, no host synchronisation and no memset (so it may be
 * recorded into a HIP graph); the caller reads result once the stream is done.
 */
fa_status fa_check_paged_tables(const int32_t *block_table, const int32_t *ctx_lens, int num_seqs,
                                int max_blocks_per_seq, int page_size, int num_pages, int32_t *result,
                                void *stream);

/*
 * Measurement helper, not part of the attention path: reads bytes (a
 * multiple of 16, > 0) at the device pointer src once, as a plain streaming
 * kernel (one contiguous slab per workgroup), and XORs every 32-bit word it
 * read into the device word *sink (which the caller sets beforehand; the
 * result only keeps the loads alive, and shows that each word was read once
 * when checked against the host). Timed by the
 * caller, it gives the HBM read rate a trivial kernel reaches on this GPU,
 * the practical ceiling beside the spec peak for a kernel that only streams
 * pages once (the paged decode). src 16-byte aligned, sink 4-byte aligned
 * (FA_ERR_UNSUPPORTED otherwise).
 */
fa_status fa_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Human-readable name of a status (static string, never NULL). */
const char *fa_status_str(fa_status s);

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
