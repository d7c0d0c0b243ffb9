// Fused attention forward, FP8 E4M3 with per-block scales, d = 64:
// instantiations of the kernel in fwd_prefill.h.
#include "fwd_prefill.h"

namespace fa {

hipError_t launch_fwd_fp8_d64(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8, const float *qs,
                              const float *ks, const float *vs, void *o, float *lse, int B, int H, int N,
                              float scale, int causal, hipStream_t stream)
{
    return causal ? launch_t<64, true, true>(q8, k8, v8, qs, ks, vs, o, lse, B, H, N, scale, stream)
                  : launch_t<64, false, true>(q8, k8, v8, qs, ks, vs, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
