// Fused attention forward, bf16 d = 128 (and the d dispatch): instantiations of the kernel in fwd_prefill.h.
#include "fwd_prefill.h"

namespace fa {

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                           int H, int N, int d, float scale, int causal, hipStream_t stream)
{
    if (d == 64) return launch_fwd_bf16_d64(q, k, v, o, lse, B, H, N, scale, causal, stream);
    return causal ? launch_t<128, true, false>(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, scale, stream)
                  : launch_t<128, false, false>(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
