// Fused attention forward, FP8 E4M3 with per-block scales, d = 128 (and the d
// dispatch): instantiations of the kernel in fwd_prefill.h.
#include "fwd_prefill.h"

namespace fa {

hipError_t launch_fwd_fp8(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8, const float *qs,
                          const float *ks, const float *vs, void *o, float *lse, int B, int H, int N,
                          int d, float scale, int causal, hipStream_t stream)
{
    if (d == 64) return launch_fwd_fp8_d64(q8, k8, v8, qs, ks, vs, o, lse, B, H, N, scale, causal, stream);
    return causal ? launch_t<128, true, true>(q8, k8, v8, qs, ks, vs, o, lse, B, H, N, scale, stream)
                  : launch_t<128, false, true>(q8, k8, v8, qs, ks, vs, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
