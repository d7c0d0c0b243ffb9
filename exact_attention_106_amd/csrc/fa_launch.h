// Internal launchers (host side). Arguments are already validated by the C ABI
// layer; each launcher only computes the grid and enqueues kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                          int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

hipError_t launch_fwd_fp8(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8,
                          const float *qs, const float *ks, const float *vs, void *o, float *lse,
                          int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

// Backward workspace: per row -L_i / scale, then per row -D_i (D_i = dO_i . O_i), fp32.
inline size_t bwd_workspace_bytes(int B, int H, int N) { return 2 * (size_t)B * H * N * sizeof(float); }

hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                           const float *lse, const void *dout, void *dq, void *dk, void *dv, int B,
                           int H, int N, int d, float scale, int causal, float *workspace,
                           hipStream_t stream);

// Pages per KV chunk (split) of the paged decode.
constexpr int kDecodePagesPerSplit = 32;

inline int decode_max_splits(int max_blocks_per_seq) {
    return (max_blocks_per_seq + kDecodePagesPerSplit - 1) / kDecodePagesPerSplit;
}

// Floats per split partial: m, l, then d unscaled output values.
inline size_t decode_partial_floats(int d) { return (size_t)d + 2; }

// Workspace: the partials of every (sequence, head, chunk), d = 128; per
// (sequence, chunk) a 64-bit hash; the hash table of chunk classes (T 64-bit
// slots); per (sequence, chunk) a partner index and a pair-list slot; the
// table's T parking slots; the pair-list length.
inline size_t decode_partials_floats(int num_seqs, int H, int max_blocks_per_seq) {
    return (size_t)num_seqs * H * decode_max_splits(max_blocks_per_seq) * decode_partial_floats(128);
}
// slots of the chunk-class hash table: a power of two, at least twice the chunks
inline int decode_table_slots(int num_seqs, int max_blocks_per_seq) {
    const size_t need = 2 * (size_t)num_seqs * decode_max_splits(max_blocks_per_seq);
    size_t t = 64;
    while (t < need) t <<= 1;
    return (int)t;
}
inline size_t decode_workspace_bytes(int num_seqs, int H, int max_blocks_per_seq) {
    const size_t n_chunks = (size_t)num_seqs * decode_max_splits(max_blocks_per_seq);
    const size_t T = (size_t)decode_table_slots(num_seqs, max_blocks_per_seq);
    return decode_partials_floats(num_seqs, H, max_blocks_per_seq) * sizeof(float) +
           n_chunks * (sizeof(uint64_t) + 2 * sizeof(int)) + T * (sizeof(uint64_t) + sizeof(int)) + sizeof(int);
}

// Plain streaming read of bytes (a multiple of 16) at src; XOR of the data into *sink.
hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

hipError_t launch_fp8_quantize(const void *x, const void *rot, uint8_t *codes, float *scales, int B, int H,
                               int N, hipStream_t stream);
// The same for Q, K (rotated when rot is given) and V (never rotated) in one launch.
hipError_t launch_fp8_quantize_qkv(const void *q, const void *k, const void *v, const void *rot, uint8_t *q_codes,
                                   uint8_t *k_codes, uint8_t *v_codes, float *q_scales, float *k_scales,
                                   float *v_scales, int B, int H, int N, hipStream_t stream);

hipError_t launch_fwd_block_sparse(const void *q, const void *k, const void *v, const uint8_t *block_mask,
                                   void *o, float *lse, int B, int H, int N, float scale, int causal,
                                   float dropout_p, uint64_t seed, hipStream_t stream);

hipError_t launch_paged_prefill_mfma(const void *q, const void *kcache, const void *vcache,
                                     const int32_t *block_table, const int32_t *ctx_lens, void *o, float *lse,
                                     int num_seqs, int H, int n_new, int max_blocks_per_seq, float scale,
                                     hipStream_t stream);

hipError_t launch_paged_decode(const void *q, const void *kcache, const void *vcache,
                               const int32_t *block_table, const int32_t *ctx_lens, void *o,
                               float *lse, int num_seqs, int H, int d, int page_size,
                               int max_blocks_per_seq, float scale, float *workspace,
                               hipStream_t stream);

// Size of the static device buffer that serves as the paged decode's
// workspace in the entry point that allocates nothing (one per device).
constexpr size_t kNoallocScratchBytes = (size_t)80 << 20;

// The paged decode on the current device with its workspace in that static
// buffer. The caller has checked decode_workspace_bytes(...) <= kNoallocScratchBytes.
hipError_t launch_paged_decode_noalloc(const void *q, const void *kcache, const void *vcache,
                                       const int32_t *block_table, const int32_t *ctx_lens, void *o,
                                       float *lse, int num_seqs, int H, int d, int page_size,
                                       int max_blocks_per_seq, float scale, hipStream_t stream);

}  // namespace fa
