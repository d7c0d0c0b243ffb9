// fp32 fused attention forward (correctness path, any 1 <= d <= 128).
//
// One wave per block of 64 query rows, one lane per row. K/V tiles of 16 keys
// are staged in LDS (zero-padded to a power-of-two head size), each lane keeps
// its query row, its unscaled output row and its running (max, sum) in
// registers and applies the online-softmax update once per tile; the output is
// normalised once at the end (FlashAttention-2 form of the update,
// "FlashAttention系列优化", FlashAttentionV2 equations). Scores are kept in
// base 2: t = s * scale * log2(e), so 2^(t - m) = e^(s*scale - m ln 2).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kRows = 64;
constexpr int kKeys = 16;

template <int DP>
__global__ __launch_bounds__(64, 1) void fwd_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    float *__restrict__ o, float *__restrict__ lse, int N, int d, int n_rb, float c, int causal)
{
    __shared__ float ks[kKeys][DP];
    __shared__ float vs[kKeys][DP];

    const int lane = threadIdx.x;
    const int rb = blockIdx.x % n_rb;
    const size_t bh = blockIdx.x / n_rb;
    const int row = rb * kRows + lane;
    const float *qh = q + bh * (size_t)N * d;
    const float *kh = k + bh * (size_t)N * d;
    const float *vh = v + bh * (size_t)N * d;

    float qr[DP];
#pragma unroll
    for (int cc = 0; cc < DP; ++cc) qr[cc] = (row < N && cc < d) ? qh[(size_t)row * d + cc] : 0.f;
    float acc[DP];
#pragma unroll
    for (int cc = 0; cc < DP; ++cc) acc[cc] = 0.f;
    float m = neg_inf(), l = 0.f;

    // causal: the block's last query is rb*64+63, so later keys are never visible
    const int kend = causal ? min(N, rb * kRows + kRows) : N;
    for (int j0 = 0; j0 < kend; j0 += kKeys) {
        __syncthreads();
        for (int e = lane; e < kKeys * DP; e += 64) {
            const int r = e / DP, cc = e % DP, key = j0 + r;
            const bool ok = key < N && cc < d;
            ks[r][cc] = ok ? kh[(size_t)key * d + cc] : 0.f;
            vs[r][cc] = ok ? vh[(size_t)key * d + cc] : 0.f;
        }
        __syncthreads();

        float t[kKeys];
        float mx = neg_inf();
#pragma unroll
        for (int r = 0; r < kKeys; ++r) {
            float dot = 0.f;
#pragma unroll
            for (int cc = 0; cc < DP; ++cc) dot = fmaf(qr[cc], ks[r][cc], dot);
            const int key = j0 + r;
            const bool vis = key < N && (!causal || key <= row);
            t[r] = vis ? dot * c : neg_inf();
            mx = fmaxf(mx, t[r]);
        }
        const float m_new = fmaxf(m, mx);
        if (m_new == neg_inf()) continue;  // nothing visible to this row yet
        const float alpha = exp2_hw(m - m_new);
        l *= alpha;
#pragma unroll
        for (int cc = 0; cc < DP; ++cc) acc[cc] *= alpha;
#pragma unroll
        for (int r = 0; r < kKeys; ++r) {
            const float p = exp2_hw(t[r] - m_new);
            l += p;
#pragma unroll
            for (int cc = 0; cc < DP; ++cc) acc[cc] = fmaf(p, vs[r][cc], acc[cc]);
        }
        m = m_new;
    }

    if (row < N) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *orow = o + (bh * (size_t)N + row) * d;
#pragma unroll
        for (int cc = 0; cc < DP; ++cc)
            if (cc < d) orow[cc] = acc[cc] * inv;
        if (lse) lse[bh * (size_t)N + row] = l > 0.f ? (m + log2f(l)) * kLn2 : neg_inf();
    }
}

template <int DP>
hipError_t launch_dp(const float *q, const float *k, const float *v, float *o, float *lse,
                     int B, int H, int N, int d, float scale, int causal, hipStream_t stream)
{
    const int n_rb = (N + kRows - 1) / kRows;
    const dim3 grid((unsigned)((size_t)B * H * n_rb));
    hipLaunchKernelGGL(fwd_f32_kernel<DP>, grid, dim3(64), 0, stream, q, k, v, o, lse, N, d, n_rb,
                       scale * kLog2e, causal);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                          int B, int H, int N, int d, float scale, int causal, hipStream_t stream)
{
    if (d <= 16) return launch_dp<16>(q, k, v, o, lse, B, H, N, d, scale, causal, stream);
    if (d <= 32) return launch_dp<32>(q, k, v, o, lse, B, H, N, d, scale, causal, stream);
    if (d <= 64) return launch_dp<64>(q, k, v, o, lse, B, H, N, d, scale, causal, stream);
    return launch_dp<128>(q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

}  // namespace fa
