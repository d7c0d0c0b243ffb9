// Paged (chunked) prefill through the block table: the paged instantiation of the kernel in fwd_prefill.h.
#include "fwd_prefill.h"

namespace fa {

// chunked prefill through the block table: the n_new newest tokens of each
// sequence (q [S, H, n_new, 128]) against its paged cache [pages, H, 16, 128]
hipError_t launch_paged_prefill_mfma(const void *q, const void *kcache, const void *vcache,
                                     const int32_t *block_table, const int32_t *ctx_lens, void *o, float *lse,
                                     int num_seqs, int H, int n_new, int max_blocks_per_seq, float scale,
                                     hipStream_t stream)
{
    const int n_rb = (n_new + kBR - 1) / kBR;
    const int BH = num_seqs * H;
    const dim3 grid((unsigned)((size_t)BH * n_rb));
    const PagedArgs pg{block_table, ctx_lens, (uint64_t)H * 16 * 128 * 2, max_blocks_per_seq, H};
    hipLaunchKernelGGL((fwd_kernel3<128, true, false, true>), grid, dim3(kThreads3), 0, stream,
                       static_cast<const uint8_t *>(q), static_cast<const uint8_t *>(kcache),
                       static_cast<const uint8_t *>(vcache), nullptr, nullptr, nullptr, static_cast<uint16_t *>(o),
                       lse, n_new, BH, n_rb, scale * kLog2e, pg);
    return hipGetLastError();
}

}  // namespace fa
