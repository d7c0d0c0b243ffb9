// bf16 fused attention forward on gfx950 MFMA (d = 64 or 128).
//
// Work decomposition (FlashAttention-2 parallelisation, 91haoming.cn article,
// "FlashAttention v2 / parallelisation improvements"; "Flash Attention 再学习",
// thread-block and warp sections):
//   * one workgroup per (batch*head, row block of 128 queries), no
//     communication between workgroups; causal grids are issued heaviest row
//     block first;
//   * 4 waves per workgroup, each owning 32 query rows (split-Q): a wave's
//     rows never need another wave's results;
//   * K/V tiles of 64 keys stream through a 2-stage LDS ring; the next tile is
//     fetched from HBM into registers while the current one is consumed.
//
// MFMA orientation. Each wave computes S^T = K_j Q_i^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 channels from LDS, B = the wave's
// 32 queries held in registers). In the 32x32 accumulator layout a lane holds
// one column (one query) and 16 rows (keys), so the row max and row sum of the
// online softmax are in-lane reductions plus one exchange between the two wave
// halves. The same registers, rounded to bf16, are directly the B operand of
// O^T += V_j^T P^T (A = 32 channels x 16 keys of V^T from LDS); the per-query
// rescale factor is then a per-lane scalar. V is transposed once per tile on
// its way into LDS, with the keys of each 16-key chunk stored in the order the
// P registers hold them (bits 2 and 3 of the key index swapped), which turns
// the A-operand fetch into one 16-byte LDS read.
//
// Online softmax (pseudocode of the FlashAttentionV1 section and the V2
// equations of "FlashAttention系列优化"): running max m and unscaled running
// sum l per query, unscaled O accumulator rescaled by 2^(m_old - m_new), one
// final 1/l, L = (m + log2 l) ln 2. Scores are handled in base 2
// (t = s * scale * log2 e).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBR = 128;      // query rows per workgroup
constexpr int kBC = 64;       // keys per tile
constexpr int kThreads = 256; // 4 waves

template <int D>
struct Bf16Layout {
    static constexpr int KS = D + 8;            // K tile row stride (elements): +16 B pad
    static constexpr int VS = kBC + 8;          // V^T tile row stride (elements): +16 B pad
    static constexpr int K_ELEMS = kBC * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int CPR = D / 8;           // 16-byte chunks per K row
    static constexpr int K_LOADS = kBC * CPR / kThreads;
    static constexpr int V_UNITS = (kBC / 4) * (D / 8);  // 4 keys x 8 channels each
};

// position of key r (0..15) inside its 16-key chunk of the V^T tile
__device__ __forceinline__ int vt_slot_of_group(int g) {  // g = key group of 4 (0..3)
    return ((g & 1) << 1) | (g >> 1);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ O, float *__restrict__ LSE, int N, int BH, int n_rb, float c)
{
    using L = Bf16Layout<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int rank = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    const int rb = CAUSAL ? (n_rb - 1 - rank) : rank;
    const size_t head = (size_t)bh * N * D;
    const uint16_t *Qh = Q + head;
    const uint16_t *Kh = K + head;
    const uint16_t *Vh = V + head;

    const int q0 = rb * kBR;
    const int qw = q0 + w * 32;
    const int my_q = qw + l32;

    // Q fragments: B operand, lane (query l32, channel group hf)
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
        if (my_q < N)
            qf[kc] = *reinterpret_cast<const bf16x8 *>(Qh + (size_t)my_q * D + 16 * kc + 8 * hf);
        else
            qf[kc] = bf16x8{};
    }

    const int kend = CAUSAL ? min(N, q0 + kBR) : N;
    const int n_tiles = (kend + kBC - 1) / kBC;

    // register staging of one K/V tile
    u32x4 kreg[L::K_LOADS];
    u32x4 vreg[4];
    const bool v_unit = tid < L::V_UNITS;
    const int v_kg = tid / (D / 8);   // key group (4 keys)
    const int v_dg = tid % (D / 8);   // channel group (8 channels)

    auto load_tile = [&](int j) {
        const int k0 = j * kBC;
#pragma unroll
        for (int i = 0; i < L::K_LOADS; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / L::CPR, ch = idx % L::CPR;
            const int key = k0 + r;
            kreg[i] = key < N ? *reinterpret_cast<const u32x4 *>(Kh + (size_t)key * D + ch * 8) : u32x4{};
        }
        if (v_unit) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = k0 + v_kg * 4 + r;
                vreg[r] = key < N ? *reinterpret_cast<const u32x4 *>(Vh + (size_t)key * D + v_dg * 8) : u32x4{};
            }
        }
    };

    auto store_tile = [&](int stage) {
        uint16_t *sk = smem + stage * L::STAGE;
        uint16_t *sv = sk + L::K_ELEMS;
#pragma unroll
        for (int i = 0; i < L::K_LOADS; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / L::CPR, ch = idx % L::CPR;
            *reinterpret_cast<u32x4 *>(sk + r * L::KS + ch * 8) = kreg[i];
        }
        if (v_unit) {
            // 4 keys x 8 channels -> 8 rows (channels) of 4 keys
            const int col = 16 * (v_kg >> 2) + 4 * vt_slot_of_group(v_kg & 3);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t a0 = vreg[0][p], a1 = vreg[1][p], a2 = vreg[2][p], a3 = vreg[3][p];
                u32x2 even, odd;
                even[0] = (a0 & 0xffffu) | (a1 << 16);
                even[1] = (a2 & 0xffffu) | (a3 << 16);
                odd[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                odd[1] = (a2 >> 16) | (a3 & 0xffff0000u);
                const int dch = v_dg * 8 + 2 * p;
                *reinterpret_cast<u32x2 *>(sv + dch * L::VS + col) = even;
                *reinterpret_cast<u32x2 *>(sv + (dch + 1) * L::VS + col) = odd;
            }
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
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
            const uint16_t *sk = smem + stage * L::STAGE;
            const uint16_t *sv = sk + L::K_ELEMS;

            // S^T = K_j Q^T : two 32-key sub-tiles
            f32x16 sacc[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                sacc[kt] = f32x16{};
#pragma unroll
                for (int kc = 0; kc < D / 16; ++kc) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sk + (kt * 32 + l32) * L::KS + 16 * kc + 8 * hf);
                    sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], sacc[kt], 0, 0, 0);
                }
            }

            // mask keys past N and (causal) keys after the query
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

            // online softmax update (base 2)
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
                    pf[kt * 2 + (i >> 3)][i & 7] = (__bf16)p;
                }
            lsum = fmaf(lsum, alpha, rs);
#pragma unroll
            for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;

            // O^T += V^T P^T : 16-key chunks
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sv + (t * 32 + l32) * L::VS + 16 * ch + 8 * hf);
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ch], oacc[t], 0, 0, 0);
                }
        }

        if (has_next) store_tile(stage ^ 1);
        __syncthreads();
    }

    // epilogue: O = O~ / l ; L = (m + log2 l) ln 2
    const float lt = xor32_sum(lsum);
    if (my_q < N) {
        const float inv = 1.f / lt;
        uint16_t *orow = O + head + (size_t)my_q * D;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
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

template <int D, bool CAUSAL>
hipError_t launch_t(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                    int N, float scale, hipStream_t stream)
{
    const int n_rb = (N + kBR - 1) / kBR;
    const int BH = B * H;
    const dim3 grid((unsigned)((size_t)BH * n_rb));
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), static_cast<uint16_t *>(o), lse, N, BH, n_rb,
                       scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                           int H, int N, int d, float scale, int causal, hipStream_t stream)
{
    if (d == 64)
        return causal ? launch_t<64, true>(q, k, v, o, lse, B, H, N, scale, stream)
                      : launch_t<64, false>(q, k, v, o, lse, B, H, N, scale, stream);
    return causal ? launch_t<128, true>(q, k, v, o, lse, B, H, N, scale, stream)
                  : launch_t<128, false>(q, k, v, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
