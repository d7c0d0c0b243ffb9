// C ABI of libfa.so: argument checks on the host, then one launcher per entry
// point. Nothing here allocates, synchronises or reads device memory.
#include <math.h>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

constexpr long long kMaxElems = (1LL << 31) - 1;

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

bool bad_scale(float scale) { return !(isfinite(scale) && scale > 0.f); }

fa_status check_dense(const void *q, const void *k, const void *v, const void *o, int B, int H,
                      int N, int d, float scale, int causal)
{
    if (!q || !k || !v || !o) return FA_ERR_NULL_PTR;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_BAD_SHAPE;
    if ((long long)B * H * N * d > kMaxElems) return FA_ERR_BAD_SHAPE;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    if (bad_scale(scale)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                 int N, int d, float scale, int causal, void *stream)
{
    fa_status st = check_dense(q, k, v, o, B, H, N, d, scale, causal);
    if (st != FA_OK) return st;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_fwd_bf16(q, k, v, o, lse, B, H, N, d, scale, causal,
                                        static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, int B,
                     int H, int N, int d, float scale, int causal, void *stream)
{
    fa_status st = check_dense(q, k, v, o, B, H, N, d, scale, causal);
    if (st != FA_OK) return st;
    if (d > 128) return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal,
                                       static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_fp8(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8, const float *q_scale,
                     const float *k_scale, const float *v_scale, void *o, float *lse, int B, int H,
                     int N, int d, float scale, int causal, void *stream)
{
    fa_status st = check_dense(q8, k8, v8, o, B, H, N, d, scale, causal);
    if (st != FA_OK) return st;
    if (!q_scale || !k_scale || !v_scale) return FA_ERR_NULL_PTR;
    if (d != 128 && d != 64) return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, N, d,
                                       scale, causal, static_cast<hipStream_t>(stream)));
}

fa_status fa_quantize_fp8(const void *x, const void *rot, uint8_t *codes, float *scales, int B, int H,
                          int N, int d, void *stream)
{
    if (!x || !codes || !scales) return FA_ERR_NULL_PTR;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_BAD_SHAPE;
    if ((long long)B * H * N * d > kMaxElems) return FA_ERR_BAD_SHAPE;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    const uintptr_t mis = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(rot) |
                          reinterpret_cast<uintptr_t>(codes);
    if ((mis & 15) || (reinterpret_cast<uintptr_t>(scales) & 3)) return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_fp8_quantize(x, rot, codes, scales, B, H, N, static_cast<hipStream_t>(stream)));
}

fa_status fa_quantize_fp8_qkv(const void *q, const void *k, const void *v, const void *rot, uint8_t *q_codes,
                              uint8_t *k_codes, uint8_t *v_codes, float *q_scales, float *k_scales, float *v_scales,
                              int B, int H, int N, int d, void *stream)
{
    if (!q || !k || !v || !q_codes || !k_codes || !v_codes || !q_scales || !k_scales || !v_scales)
        return FA_ERR_NULL_PTR;
    if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_BAD_SHAPE;
    if ((long long)B * H * N * d > kMaxElems) return FA_ERR_BAD_SHAPE;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(rot) |
                          reinterpret_cast<uintptr_t>(q_codes) | reinterpret_cast<uintptr_t>(k_codes) |
                          reinterpret_cast<uintptr_t>(v_codes);
    const uintptr_t mis_s = reinterpret_cast<uintptr_t>(q_scales) | reinterpret_cast<uintptr_t>(k_scales) |
                            reinterpret_cast<uintptr_t>(v_scales);
    if ((mis & 15) || (mis_s & 3)) return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_fp8_quantize_qkv(q, k, v, rot, q_codes, k_codes, v_codes, q_scales, k_scales,
                                                v_scales, B, H, N, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_block_sparse(const void *q, const void *k, const void *v, const uint8_t *block_mask,
                              void *o, float *lse, int B, int H, int N, int d, float scale, int causal,
                              float dropout_p, uint64_t seed, void *stream)
{
    fa_status st = check_dense(q, k, v, o, B, H, N, d, scale, causal);
    if (st != FA_OK) return st;
    if (!block_mask) return FA_ERR_NULL_PTR;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    if (N > 131072) return FA_ERR_BAD_SHAPE;
    if (!(dropout_p >= 0.f && dropout_p < 1.f)) return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_fwd_block_sparse(q, k, v, block_mask, o, lse, B, H, N, scale, causal, dropout_p,
                                                seed, static_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d)
{
    if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
    if ((long long)B * H * N * d > kMaxElems) return 0;
    return fa::bwd_workspace_bytes(B, H, N);
}

fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 const void *dout, void *dq, void *dk, void *dv, int B, int H, int N, int d,
                 float scale, int causal, void *workspace, size_t workspace_bytes, void *stream)
{
    fa_status st = check_dense(q, k, v, o, B, H, N, d, scale, causal);
    if (st != FA_OK) return st;
    if (!lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_NULL_PTR;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (workspace_bytes < fa::bwd_workspace_bytes(B, H, N)) return FA_ERR_WORKSPACE;
    return from_hip(fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                                        static_cast<float *>(workspace),
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// The decode's chunk count num_seqs * ceil(max_blocks / 32) and its hash table
// (a power of two of at least twice that) index in 32-bit ints: at most 2^29
// chunks (65535 sequences of up to 262144 blocks = 4.2M tokens each).
static bool decode_chunks_ok(int num_seqs, int max_blocks_per_seq)
{
    return (long long)num_seqs * fa::decode_max_splits(max_blocks_per_seq) <= (1LL << 29);
}

extern "C" {

size_t fa_paged_decode_workspace_bytes(int num_seqs, int H, int d, int page_size,
                                       int max_blocks_per_seq)
{
    if (num_seqs <= 0 || H <= 0 || max_blocks_per_seq <= 0) return 0;
    if (d != 128 || page_size != 16) return 0;
    if (!decode_chunks_ok(num_seqs, max_blocks_per_seq)) return 0;
    return fa::decode_workspace_bytes(num_seqs, H, max_blocks_per_seq);
}

static fa_status check_paged_decode(const void *q, const void *kcache, const void *vcache,
                                    const int32_t *block_table, const int32_t *ctx_lens, const void *o,
                                    int num_seqs, int H, int d, int page_size, int max_blocks_per_seq,
                                    int num_pages, float scale)
{
    if (!q || !kcache || !vcache || !block_table || !ctx_lens || !o) return FA_ERR_NULL_PTR;
    if (num_seqs <= 0 || H <= 0 || d <= 0 || page_size <= 0 || max_blocks_per_seq <= 0 ||
        num_pages <= 0)
        return FA_ERR_BAD_SHAPE;
    if (d != 128 || page_size != 16) return FA_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || H > 65535) return FA_ERR_BAD_SHAPE;
    if ((long long)max_blocks_per_seq * page_size > kMaxElems) return FA_ERR_BAD_SHAPE;
    if (!decode_chunks_ok(num_seqs, max_blocks_per_seq)) return FA_ERR_BAD_SHAPE;
    if (bad_scale(scale)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status fa_paged_decode(const void *q, const void *kcache, const void *vcache,
                          const int32_t *block_table, const int32_t *ctx_lens, void *o, float *lse,
                          int num_seqs, int H, int d, int page_size, int max_blocks_per_seq,
                          int num_pages, float scale, void *workspace, size_t workspace_bytes,
                          void *stream)
{
    fa_status st = check_paged_decode(q, kcache, vcache, block_table, ctx_lens, o, num_seqs, H, d, page_size,
                                      max_blocks_per_seq, num_pages, scale);
    if (st != FA_OK) return st;
    if (!workspace) return FA_ERR_NULL_PTR;
    if (workspace_bytes < fa_paged_decode_workspace_bytes(num_seqs, H, d, page_size,
                                                          max_blocks_per_seq))
        return FA_ERR_WORKSPACE;
    return from_hip(fa::launch_paged_decode(q, kcache, vcache, block_table, ctx_lens, o, lse,
                                            num_seqs, H, d, page_size, max_blocks_per_seq, scale,
                                            static_cast<float *>(workspace),
                                            static_cast<hipStream_t>(stream)));
}

size_t fa_noalloc_scratch_bytes(void) { return fa::kNoallocScratchBytes; }

fa_status fa_paged_decode_noalloc(const void *q, const void *kcache, const void *vcache,
                                  const int32_t *block_table, const int32_t *ctx_lens, void *o, float *lse,
                                  int num_seqs, int H, int d, int page_size, int max_blocks_per_seq,
                                  int num_pages, float scale, void *stream)
{
    fa_status st = check_paged_decode(q, kcache, vcache, block_table, ctx_lens, o, num_seqs, H, d, page_size,
                                      max_blocks_per_seq, num_pages, scale);
    if (st != FA_OK) return st;
    if (fa_paged_decode_workspace_bytes(num_seqs, H, d, page_size, max_blocks_per_seq) > fa::kNoallocScratchBytes)
        return FA_ERR_SCRATCH_LIMIT;
    return from_hip(fa::launch_paged_decode_noalloc(q, kcache, vcache, block_table, ctx_lens, o, lse, num_seqs,
                                                    H, d, page_size, max_blocks_per_seq, scale,
                                                    static_cast<hipStream_t>(stream)));
}

fa_status fa_paged_prefill(const void *q, const void *kcache, const void *vcache,
                           const int32_t *block_table, const int32_t *ctx_lens, void *o, float *lse,
                           int num_seqs, int H, int n_new, int d, int page_size,
                           int max_blocks_per_seq, int num_pages, float scale, void *stream)
{
    if (!q || !kcache || !vcache || !block_table || !ctx_lens || !o) return FA_ERR_NULL_PTR;
    if (num_seqs <= 0 || H <= 0 || n_new <= 0 || d <= 0 || page_size <= 0 || max_blocks_per_seq <= 0 ||
        num_pages <= 0)
        return FA_ERR_BAD_SHAPE;
    if (d != 128 || page_size != 16) return FA_ERR_UNSUPPORTED;
    if ((long long)num_seqs * H > 65535) return FA_ERR_BAD_SHAPE;
    if ((long long)num_seqs * H * n_new * d > kMaxElems) return FA_ERR_BAD_SHAPE;
    if ((long long)max_blocks_per_seq * page_size > kMaxElems) return FA_ERR_BAD_SHAPE;
    if (bad_scale(scale)) return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_paged_prefill_mfma(q, kcache, vcache, block_table, ctx_lens, o, lse, num_seqs, H,
                                                  n_new, max_blocks_per_seq, scale,
                                                  static_cast<hipStream_t>(stream)));
}

const char *fa_status_str(fa_status s)
{
    switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL_PTR: return "FA_ERR_NULL_PTR: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE: a size is non-positive or too large";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head size, page size, flag or scale not supported";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
    case FA_ERR_NO_PAGES: return "FA_ERR_NO_PAGES: the block manager has no free page";
    case FA_ERR_STATE: return "FA_ERR_STATE: invalid block-manager state or sequence id in the wrong state";
    case FA_ERR_SCRATCH_LIMIT:
        return "FA_ERR_SCRATCH_LIMIT: the sizes need more workspace than the library's static buffer holds";
    }
    return "unknown fa_status";
}

fa_status fa_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream)
{
    if (!src || !sink) return FA_ERR_NULL_PTR;
    if (bytes == 0) return FA_ERR_BAD_SHAPE;
    if (bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)sink & 3)) return FA_ERR_UNSUPPORTED;
    return from_hip(fa::launch_read_probe(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

int fa_version(void) { return 100; }

}  // extern "C"
