// FP8 (OCP E4M3FN) fused attention forward on gfx950, d = 128, with one fp32
// scale per (batch, head, 128-token block) for each of Q, K and V
// (FlashAttention-3 block quantisation, "FlashAttention系列优化",
// FlashAttentionV3 / FP低精度).
//
// Same decomposition as the bf16 kernel (128-query row block per workgroup,
// 4 waves x 32 queries, 64-key tiles through a 2-stage LDS ring, S^T
// orientation so the softmax reductions stay in-lane). Differences:
//   * S^T = K8 Q8^T on v_mfma_f32_32x32x16_fp8_fp8 with fp32 accumulation:
//     the products of E4M3 values are exact, so the scores carry only fp32
//     summation error. Row blocks (128) line up with the scale blocks and a
//     64-key tile lies inside one scale block, so the dequantisation is one
//     scalar per tile folded into the softmax multiplier:
//     t = s8 * (sq * sk * scale * log2 e).
//   * P.V runs on bf16 MFMA: V is widened E4M3 -> bf16 (exact) while it is
//     transposed into LDS (the in-kernel layout change that the FlashAttention-3
//     FP8 description needs for the second GEMM), and the tile's V scale is
//     folded into P before P is rounded to bf16. P itself is not quantised to
//     E4M3: with V outliers of tens, a 3-bit mantissa on P alone would exceed
//     the accuracy this path is held to.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBR = 128;
constexpr int kBC = 64;
constexpr int kThreads = 256;
constexpr int kD = 128;
constexpr int kScaleBlock = 128;

constexpr int KS8 = kD + 16;                  // bytes per K8 row in LDS (+16 B pad)
constexpr int K8_BYTES = kBC * KS8;           // 9216
constexpr int VS = kBC + 8;                   // V^T row stride (bf16 elements)
constexpr int VT_BYTES = kD * VS * 2;         // 18432
constexpr int STAGE_BYTES = K8_BYTES + VT_BYTES;
constexpr int K8_LOADS = kBC * (kD / 16) / kThreads;   // 2 x 16 B per thread
constexpr int V8_UNITS = (kBC / 4) * (kD / 16);        // 4 keys x 16 channels -> 128 units

__device__ __forceinline__ int vt_slot_of_group(int g) { return ((g & 1) << 1) | (g >> 1); }

// two E4M3 bytes (selected 16-bit half of w) -> two bf16 in one dword, exact
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
    const f32x2 f = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_fp8_kernel(
    const uint8_t *__restrict__ Q8, const uint8_t *__restrict__ K8, const uint8_t *__restrict__ V8,
    const float *__restrict__ QS, const float *__restrict__ KS, const float *__restrict__ VSc,
    uint16_t *__restrict__ O, float *__restrict__ LSE, int N, int BH, int n_rb, float c0)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int rank = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    const int rb = CAUSAL ? (n_rb - 1 - rank) : rank;
    const size_t head = (size_t)bh * N * kD;
    const int nsb = (N + kScaleBlock - 1) / kScaleBlock;
    const float *qs_h = QS + (size_t)bh * nsb;
    const float *ks_h = KS + (size_t)bh * nsb;
    const float *vs_h = VSc + (size_t)bh * nsb;
    const uint8_t *Qh = Q8 + head;
    const uint8_t *Kh = K8 + head;
    const uint8_t *Vh = V8 + head;

    const int q0 = rb * kBR;
    const int qw = q0 + w * 32;
    const int my_q = qw + l32;
    const float cq = c0 * qs_h[rb];

    // Q fragments: 8 bytes (channels 16 kc + 8 hf .. +7) per 16-channel chunk
    long qf[kD / 16];
#pragma unroll
    for (int kc = 0; kc < kD / 16; ++kc)
        qf[kc] = my_q < N ? *reinterpret_cast<const long *>(Qh + (size_t)my_q * kD + 16 * kc + 8 * hf) : 0L;

    const int kend = CAUSAL ? min(N, q0 + kBR) : N;
    const int n_tiles = (kend + kBC - 1) / kBC;

    u32x4 kreg[K8_LOADS];
    u32x4 vreg[4];
    const bool v_unit = tid < V8_UNITS;
    const int v_kg = tid / (kD / 16);
    const int v_dg = tid % (kD / 16);

    auto load_tile = [&](int j) {
        const int k0 = j * kBC;
#pragma unroll
        for (int i = 0; i < K8_LOADS; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / (kD / 16), ch = idx % (kD / 16);
            const int key = k0 + r;
            kreg[i] = key < N ? *reinterpret_cast<const u32x4 *>(Kh + (size_t)key * kD + ch * 16) : u32x4{};
        }
        if (v_unit) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + v_kg * 4 + r;
                vreg[r] = key < N ? *reinterpret_cast<const u32x4 *>(Vh + (size_t)key * kD + v_dg * 16) : u32x4{};
            }
        }
    };

    auto store_tile = [&](int stage) {
        uint8_t *sk = smem + stage * STAGE_BYTES;
        uint16_t *sv = reinterpret_cast<uint16_t *>(sk + K8_BYTES);
#pragma unroll
        for (int i = 0; i < K8_LOADS; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / (kD / 16), ch = idx % (kD / 16);
            *reinterpret_cast<u32x4 *>(sk + r * KS8 + ch * 16) = kreg[i];
        }
        if (v_unit) {
            const int col = 16 * (v_kg >> 2) + 4 * vt_slot_of_group(v_kg & 3);
#pragma unroll
            for (int p = 0; p < 8; ++p) {   // channel pair (2p, 2p+1) of the 16
                uint32_t b[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) b[r] = e4m3x2_to_bf16x2(vreg[r][p >> 1], (p & 1) != 0);
                u32x2 even, odd;
                even[0] = (b[0] & 0xffffu) | (b[1] << 16);
                even[1] = (b[2] & 0xffffu) | (b[3] << 16);
                odd[0] = (b[0] >> 16) | (b[1] & 0xffff0000u);
                odd[1] = (b[2] >> 16) | (b[3] & 0xffff0000u);
                const int dch = v_dg * 16 + 2 * p;
                *reinterpret_cast<u32x2 *>(sv + dch * VS + col) = even;
                *reinterpret_cast<u32x2 *>(sv + (dch + 1) * VS + col) = odd;
            }
        }
    };

    f32x16 oacc[kD / 32];
#pragma unroll
    for (int t = 0; t < kD / 32; ++t) oacc[t] = f32x16{};
    float m = neg_inf();
    float lsum = 0.f;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const int stage = j & 1;
        const bool has_next = j + 1 < n_tiles;
        if (has_next) load_tile(j + 1);

        const int k0 = j * kBC;
        const bool active = !CAUSAL || k0 <= qw + 31;
        if (active) {
            const uint8_t *sk = smem + stage * STAGE_BYTES;
            const uint16_t *sv = reinterpret_cast<const uint16_t *>(sk + K8_BYTES);
            const float c = cq * ks_h[k0 / kScaleBlock];
            const float sv_scale = vs_h[k0 / kScaleBlock];

            f32x16 sacc[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                sacc[kt] = f32x16{};
#pragma unroll
                for (int kc = 0; kc < kD / 16; ++kc) {
                    const long a = *reinterpret_cast<const long *>(sk + (kt * 32 + l32) * KS8 + 16 * kc + 8 * hf);
                    sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, qf[kc], sacc[kt], 0, 0, 0);
                }
            }

            const bool need_mask = (k0 + kBC > N) || (CAUSAL && k0 + kBC - 1 > qw);
            if (need_mask) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = k0 + kt * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                        const bool vis = key < N && (!CAUSAL || key <= my_q);
                        if (!vis) sacc[kt][i] = neg_inf();
                    }
            }

            float mx = neg_inf();
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
            mx = xor32_max(mx);
            const float m_new = fmaxf(m, mx * c);
            const float m_use = m_new == neg_inf() ? 0.f : m_new;
            const float alpha = exp2_hw(m - m_use);
            m = m_new;

            float rs = 0.f;
            bf16x8 pf[4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = exp2_hw(fmaf(sacc[kt][i], c, -m_use));
                    rs += p;
                    pf[kt * 2 + (i >> 3)][i & 7] = (__bf16)(p * sv_scale);
                }
            lsum = fmaf(lsum, alpha, rs);
#pragma unroll
            for (int t = 0; t < kD / 32; ++t) oacc[t] *= alpha;

#pragma unroll
            for (int t = 0; t < kD / 32; ++t)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sv + (t * 32 + l32) * VS + 16 * ch + 8 * hf);
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ch], oacc[t], 0, 0, 0);
                }
        }

        if (has_next) store_tile(stage ^ 1);
        __syncthreads();
    }

    const float lt = xor32_sum(lsum);
    if (my_q < N) {
        const float inv = 1.f / lt;
        uint16_t *orow = O + head + (size_t)my_q * kD;
#pragma unroll
        for (int t = 0; t < kD / 32; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 packed;
                packed[0] = pack_bf16x2(oacc[t][4 * g + 0] * inv, oacc[t][4 * g + 1] * inv);
                packed[1] = pack_bf16x2(oacc[t][4 * g + 2] * inv, oacc[t][4 * g + 3] * inv);
                *reinterpret_cast<u32x2 *>(orow + t * 32 + 8 * g + 4 * hf) = packed;
            }
        if (LSE && hf == 0) LSE[(size_t)bh * N + my_q] = (m + __log2f(lt)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd_fp8(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8, const float *qs,
                          const float *ks, const float *vs, void *o, float *lse, int B, int H, int N,
                          int d, float scale, int causal, hipStream_t stream)
{
    (void)d;
    const int n_rb = (N + kBR - 1) / kBR;
    const int BH = B * H;
    const dim3 grid((unsigned)((size_t)BH * n_rb));
    const float c0 = scale * kLog2e;
    if (causal)
        hipLaunchKernelGGL(fwd_fp8_kernel<true>, grid, dim3(kThreads), 0, stream, q8, k8, v8, qs, ks, vs,
                           static_cast<uint16_t *>(o), lse, N, BH, n_rb, c0);
    else
        hipLaunchKernelGGL(fwd_fp8_kernel<false>, grid, dim3(kThreads), 0, stream, q8, k8, v8, qs, ks, vs,
                           static_cast<uint16_t *>(o), lse, N, BH, n_rb, c0);
    return hipGetLastError();
}

}  // namespace fa
