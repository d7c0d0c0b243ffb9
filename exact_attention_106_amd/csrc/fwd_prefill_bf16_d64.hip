// Fused attention forward, bf16 d = 64: instantiations of the kernel in fwd_prefill.h.
#include "fwd_prefill.h"

namespace fa {

hipError_t launch_fwd_bf16_d64(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                               int N, float scale, int causal, hipStream_t stream)
{
    return causal ? launch_t<64, true, false>(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, scale, stream)
                  : launch_t<64, false, false>(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
