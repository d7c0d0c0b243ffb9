// Fused attention forward on gfx950 MFMA: bf16 (d = 64, 128) and FP8 E4M3
// with per-block scales (d = 128), one kernel template for both.
//
// Work decomposition (FlashAttention-2 parallelisation, 91haoming.cn article,
// "FlashAttention v2 / parallelisation improvements"; "Flash Attention 再学习",
// thread-block and warp sections):
//   * one workgroup per (batch*head, row block of 128 queries), no
//     communication between workgroups; causal grids are issued heaviest row
//     block first;
//   * 4 waves per workgroup, each owning 32 query rows (split-Q);
//   * K/V tiles of 64 keys stream through a 2-stage LDS ring; the next tile is
//     fetched from HBM (buffer loads, which return zeros past row N - 1) into
//     registers while the current one is consumed.
//
// MFMA orientation. Each wave computes S^T = K_j Q_i^T (A = 32 keys x 16
// channels from LDS, B = the wave's 32 queries held in registers). In the
// 32x32 accumulator layout a lane holds one query and 16 keys, so the row max
// and sum of the online softmax are in-lane reductions plus one exchange
// between the wave halves (v_permlane32_swap). The same registers, rounded to
// bf16, are directly the B operand of O^T += V_j^T P^T. V stays row-major in
// LDS and the A operand V^T is read with ds_read_b64_tr_b16, whose lane
// transpose delivers 4 keys of one channel per lane; the keys a lane reads are
// the ones its P registers hold (keys are a summation index, so only the
// pairing matters).
//
// Online softmax (pseudocode of the FlashAttentionV1 section and the V2
// equations of "FlashAttention系列优化"): running reference max m, unscaled
// sums, unscaled O accumulator, one final division, L = (m + log2 l) ln 2, in
// base 2 (t = s * scale * log2 e). The reference max only moves when a row max
// exceeds it by more than kRescaleSlack. O is divided by the sum of the
// bf16-rounded weights that the P.V MFMA actually used; L uses the fp32 sum.
//
// FP8 (FlashAttention-3 block quantisation, "FlashAttention系列优化",
// FlashAttentionV3 / FP低精度): S^T = K8 Q8^T on v_mfma_f32_32x32x16_fp8_fp8
// (products of E4M3 values are exact); row blocks (128) coincide with the
// scale blocks and a 64-key tile lies in one scale block, so dequantisation is
// one scalar per tile folded into the softmax multiplier. V is widened
// E4M3 -> bf16 (exact) on its way into LDS and P.V runs on bf16 MFMA with the
// tile's V scale folded into P. P is not quantised to E4M3: with V outliers of
// tens, a 3-bit mantissa on P would exceed this path's accuracy bound.
#include "fa_device.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kBR = 128;       // query rows per workgroup
constexpr int kBC = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kScaleBlock = 128;

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D, bool FP8>
struct Layout {
    static constexpr int KROW = FP8 ? D : 2 * D;   // bytes of one K / V row in HBM
    static constexpr int KS = KROW + 16;           // LDS K row stride: +16 B keeps MFMA reads conflict-free
    static constexpr int VS = 2 * D + 64;          // LDS V row stride (bf16): +64 B keeps transpose reads conflict-free
    static constexpr int K_BYTES = kBC * KS;
    static constexpr int V_BYTES = kBC * VS;
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int CPR = KROW / 16;          // 16-byte chunks per row
    static constexpr int LOADS = kBC * CPR / kThreads;
};

// two E4M3 bytes (selected 16-bit half of w) -> two bf16 in one dword, exact
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
    const f32x2 f = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
}

__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(const_cast<uint8_t *>(p)));
}

template <int D, bool CAUSAL, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(
    const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K, const uint8_t *__restrict__ V,
    const float *__restrict__ QS, const float *__restrict__ KSc, const float *__restrict__ VSc,
    uint16_t *__restrict__ O, float *__restrict__ LSE, int N, int BH, int n_rb, float c0)
{
    using L = Layout<D, FP8>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int rank = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    const int rb = CAUSAL ? (n_rb - 1 - rank) : rank;
    const size_t head_bytes_off = (size_t)bh * N * L::KROW;
    const uint32_t head_bytes = (uint32_t)N * L::KROW;
    // loads past row N - 1 of this head return zeros
    const auto rq = make_rsrc(Q + head_bytes_off, head_bytes);
    const auto rk = make_rsrc(K + head_bytes_off, head_bytes);
    const auto rv = make_rsrc(V + head_bytes_off, head_bytes);

    const int q0 = rb * kBR;
    const int qw = q0 + w * 32;
    const int my_q = qw + l32;

    float c = c0;
    const float *ks_h = nullptr, *vs_h = nullptr;
    if constexpr (FP8) {
        const int nsb = (N + kScaleBlock - 1) / kScaleBlock;
        c = c0 * QS[(size_t)bh * nsb + rb];
        ks_h = KSc + (size_t)bh * nsb;
        vs_h = VSc + (size_t)bh * nsb;
    }

    // Q fragments: B operand, lane (query l32, channel group hf) of each 16-channel chunk
    typedef typename std::conditional<FP8, long, bf16x8>::type QFrag;
    QFrag qf[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
        if constexpr (FP8)
            qf[kc] = __builtin_bit_cast(long, buf_load8(rq, (uint32_t)(my_q * D + 16 * kc + 8 * hf)));
        else
            qf[kc] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(my_q * D + 16 * kc + 8 * hf) * 2));
    }

    const int kend = CAUSAL ? min(N, q0 + kBR) : N;
    const int n_tiles = (kend + kBC - 1) / kBC;

    // register staging of one K/V tile: chunk idx = tid + i*256 is (row idx / CPR, chunk idx % CPR)
    u32x4 kreg[L::LOADS];
    u32x4 vreg[L::LOADS];
    auto load_tile = [&](int j) {
        const uint32_t base = (uint32_t)(j * kBC) * L::KROW;
#pragma unroll
        for (int i = 0; i < L::LOADS; ++i) {
            const uint32_t off = base + (uint32_t)(tid + i * kThreads) * 16;
            kreg[i] = buf_load16(rk, off);
            vreg[i] = buf_load16(rv, off);
        }
    };
    auto store_tile = [&](int stage) {
        uint8_t *sk = smem + stage * L::STAGE;
        uint8_t *sv = sk + L::K_BYTES;
#pragma unroll
        for (int i = 0; i < L::LOADS; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / L::CPR, ch = idx % L::CPR;
            *reinterpret_cast<u32x4 *>(sk + r * L::KS + ch * 16) = kreg[i];
            if constexpr (FP8) {
                // 16 E4M3 channels -> 16 bf16 (32 bytes)
                u32x4 lo, hi;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    lo[2 * e] = e4m3x2_to_bf16x2(vreg[i][e], false);
                    lo[2 * e + 1] = e4m3x2_to_bf16x2(vreg[i][e], true);
                    hi[2 * e] = e4m3x2_to_bf16x2(vreg[i][2 + e], false);
                    hi[2 * e + 1] = e4m3x2_to_bf16x2(vreg[i][2 + e], true);
                }
                *reinterpret_cast<u32x4 *>(sv + r * L::VS + ch * 32) = lo;
                *reinterpret_cast<u32x4 *>(sv + r * L::VS + ch * 32 + 16) = hi;
            } else {
                *reinterpret_cast<u32x4 *>(sv + r * L::VS + ch * 16) = vreg[i];
            }
        }
    };

    // transpose-read base of this lane: 16-lane group G supplies 4 keys x 16
    // channels; lane s = 4e + j of the group points at key 4 (G / 2) + e,
    // channels 16 (G % 2) + 4 j .. +3
    const int tr_G = lane >> 4, tr_s = lane & 15;
    const int tr_base = (4 * (tr_G >> 1) + (tr_s >> 2)) * L::VS + (16 * (tr_G & 1) + 4 * (tr_s & 3)) * 2;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
    float m = neg_inf();  // reference max (base 2), moved only by more than kRescaleSlack
    float lsum = 0.f;     // this lane's share of l (fp32 weights)
    float lsumb = 0.f;    // same, over the bf16-rounded weights the P.V product uses

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
            const uint8_t *sk = smem + stage * L::STAGE;
            const uint8_t *sv = sk + L::K_BYTES;
            float ct = c, pscale = 1.f, inv_pscale = 1.f;
            if constexpr (FP8) {
                ct = c * ks_h[k0 / kScaleBlock];
                pscale = vs_h[k0 / kScaleBlock];
                inv_pscale = 1.f / pscale;
            }

            // S^T = K_j Q^T : two 32-key sub-tiles
            f32x16 sacc[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                sacc[kt] = f32x16{};
#pragma unroll
                for (int kc = 0; kc < D / 16; ++kc) {
                    if constexpr (FP8) {
                        const long a = *reinterpret_cast<const long *>(sk + (kt * 32 + l32) * L::KS + 16 * kc + 8 * hf);
                        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, qf[kc], sacc[kt], 0, 0, 0);
                    } else {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sk + (kt * 32 + l32) * L::KS + (16 * kc + 8 * hf) * 2);
                        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], sacc[kt], 0, 0, 0);
                    }
                }
            }

            // mask keys past N and (causal) keys after the query: register i of
            // sub-tile kt holds key k0 + 4 hf + kt*32 + 8 (i/4) + i%4
            const bool need_mask = (k0 + kBC > N) || (CAUSAL && k0 + kBC - 1 > qw);
            if (need_mask) {
                const int lim = (CAUSAL ? min(my_q, N - 1) : N - 1) - (k0 + 4 * hf);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (kt * 32 + 8 * (i >> 2) + (i & 3) > lim) sacc[kt][i] = neg_inf();
            }

            // online softmax (base 2) with a lazily moved reference max
            float mx = neg_inf();
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
            const float mxc = other_half_max(mx) * ct;
            const bool move = mxc > m + kRescaleSlack;
            if (__builtin_amdgcn_ballot_w64(move)) {
                const float m_new = move ? mxc : m;
                const float alpha = exp2_hw(m - m_new);
                lsum *= alpha;
                lsumb *= alpha;
#pragma unroll
                for (int t = 0; t < D / 32; ++t) oacc[t] *= alpha;
                m = m_new;
            }
            const float m_use = m == neg_inf() ? 0.f : m;

            float rs = 0.f, rsb = 0.f;
            bf16x8 pf[4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = exp2_hw(fmaf(sacc[kt][i], ct, -m_use));
                    rs += p;
                    pf[kt * 2 + (i >> 3)][i & 7] = (__bf16)(FP8 ? p * pscale : p);
                }
            typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
            const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                rsb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[ch], pf[ch], 0, 1), ones, rsb, false);
                rsb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[ch], pf[ch], 2, 3), ones, rsb, false);
                rsb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[ch], pf[ch], 4, 5), ones, rsb, false);
                rsb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[ch], pf[ch], 6, 7), ones, rsb, false);
            }
            lsum += rs;
            lsumb = FP8 ? fmaf(rsb, inv_pscale, lsumb) : lsumb + rsb;

            // O^T += V^T P^T : 16-key chunks; A operand = two transpose reads
            // (keys 16ch + 4 hf + 0..3 and 16ch + 8 + 4 hf + 0..3)
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const uint8_t *p0 = sv + tr_base + (16 * ch) * L::VS + 64 * t;
                    const s16x4 lo = lds_read_tr16(p0);
                    const s16x4 hi = lds_read_tr16(p0 + 8 * L::VS);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ch], oacc[t], 0, 0, 0);
                }
        }

        if (has_next) store_tile(stage ^ 1);
        __syncthreads();
    }

    // epilogue: O = O~ / l_bf16 ; L = (m + log2 l) ln 2
    const float lt = other_half_sum(lsum);
    const float ltb = other_half_sum(lsumb);
    if (my_q < N) {
        const float inv = 1.f / ltb;
        uint16_t *orow = O + ((size_t)bh * N + my_q) * D;
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

template <int D, bool CAUSAL, bool FP8>
hipError_t launch_t(const void *q, const void *k, const void *v, const float *qs, const float *ks,
                    const float *vs, void *o, float *lse, int B, int H, int N, float scale,
                    hipStream_t stream)
{
    const int n_rb = (N + kBR - 1) / kBR;
    const int BH = B * H;
    const dim3 grid((unsigned)((size_t)BH * n_rb));
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, FP8>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint8_t *>(q), static_cast<const uint8_t *>(k),
                       static_cast<const uint8_t *>(v), qs, ks, vs, static_cast<uint16_t *>(o), lse, N,
                       BH, n_rb, scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                           int H, int N, int d, float scale, int causal, hipStream_t stream)
{
    if (d == 64)
        return causal ? launch_t<64, true, false>(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, scale, stream)
                      : launch_t<64, false, false>(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, scale, stream);
    return causal ? launch_t<128, true, false>(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, scale, stream)
                  : launch_t<128, false, false>(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, scale, stream);
}

hipError_t launch_fwd_fp8(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8, const float *qs,
                          const float *ks, const float *vs, void *o, float *lse, int B, int H, int N,
                          int d, float scale, int causal, hipStream_t stream)
{
    (void)d;
    return causal ? launch_t<128, true, true>(q8, k8, v8, qs, ks, vs, o, lse, B, H, N, scale, stream)
                  : launch_t<128, false, true>(q8, k8, v8, qs, ks, vs, o, lse, B, H, N, scale, stream);
}

}  // namespace fa
