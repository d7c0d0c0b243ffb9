// Fused incoherent processing + FP8 block quantisation on gfx950.
//
// FlashAttention-3 FP8 ("FlashAttention系列优化", FlashAttentionV3 / FP低精度;
// 91haoming.cn FlashAttention v1-v3 article, v3 FP8 part): scales are kept per
// block of tokens, and incoherent processing multiplies Q and K by one random
// orthogonal matrix R first, which spreads outlier channels over all channels
// while (QR)(KR)^T = QK^T leaves the scores unchanged. One kernel does both for
// a [B, H, N, 128] bf16 tensor:
//   y = x R, bf16 MFMA with fp32 sums (y = x when no R is given: V, or Q and
//   K without incoherent processing; that variant skips the MFMA);
//   per (b, h, 128-token block): s = fp32(amax|y| / 448) (1 when amax = 0);
//   code = E4M3FN(round to nearest even of clamp(y / s, -448, 448)), with
//   the scale as stored, so that decode(code) * s is the E4M3 grid point
//   nearest to y; y / s is the correctly rounded fp32 quotient, so an exact tie
//   (possible when no rotation is applied and y = x exactly) goes to the even
//   code as the definition says.
// The MFMA computes y^T = R^T x^T, so that a lane ends with 4 consecutive
// output channels of one token and the codes leave it as packed words.
// R is read from LDS with transpose reads (ds_read_b64_tr_b16); its rows are
// stored in the order those reads deliver them, so that each lane's part of x
// is a contiguous 16-byte load. Workgroups are persistent: R is loaded once
// and the workgroup walks the token blocks grid-stride. A (b, h, block)
// lives in one workgroup, so its amax needs only an LDS reduction.
#include "fa_device.h"
#include "fa_dma.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kQzThreads = 256;
constexpr int kQzBlock = 128;   // tokens per scale block, one per loop trip
constexpr int kQzGrid = 768;    // 3 workgroups per CU (registers, and 48 KiB of LDS with R)

template <bool ROT>
__global__ __launch_bounds__(kQzThreads) void fp8_quant_kernel(const uint16_t *__restrict__ X,
                                                              const uint16_t *__restrict__ R,
                                                              uint8_t *__restrict__ codes,
                                                              float *__restrict__ scales, int N, int nb,
                                                              int total)
{
    constexpr int D = 128, ROW = 2 * D, CPR = D / 8, KC = D / 16, NT = D / 32;
    __shared__ __attribute__((aligned(16))) uint8_t sc[kQzBlock * D];  // codes of one block
    __shared__ float wmax[4];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
    const int tl = 32 * w + l32;   // token of the lane within the block

    // Input channel k = 64 g + 8 c + j (g = 0, 1; c < 8; j < 8) is MFMA k-step
    // c, lane half g, position j. The transpose read of k-step c gives lane
    // half g the LDS rows 16 c + 4 g + 0..3 and 16 c + 8 + 4 g + 0..3 in that
    // order, so R's row k goes to LDS row 16 c + 8 (j / 4) + 4 g + j % 4.
    [[maybe_unused]] uint32_t tro[2][NT];
    [[maybe_unused]] uint8_t *sr = nullptr;
    if constexpr (ROT) {
        __shared__ __attribute__((aligned(1024))) uint8_t sr_[D * ROW];   // R, rows permuted, swizzled
        sr = sr_;
        for (int idx = tid; idx < D * CPR; idx += kQzThreads) {
            const int k = idx / CPR, cc = idx % CPR;
            const int g = k >> 6, c = (k >> 3) & 7, j = k & 7;
            const int r = 16 * c + 8 * (j >> 2) + 4 * g + (j & 3);
            *reinterpret_cast<u32x4 *>(sr + r * ROW + ((cc ^ swz<CPR>(r)) << 4)) =
                *reinterpret_cast<const u32x4 *>(R + k * D + cc * 8);
        }
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
#pragma unroll
            for (int t = 0; t < NT; ++t) tro[rd][t] = tr_offset<CPR>(lane, rd, t);
        __syncthreads();
    }

    // token t0 + tl of an item, channels 64 h + 8 kc + 0..7 (the MFMA's B
    // operand x^T). Two register sets alternate: the next item's part is
    // loaded before the current one is processed, so its latency overlaps the
    // work. The loads always read an in-range address (token 0 of the tensor
    // for tokens past N or items past the end) and such values are zeroed.
    auto load_item = [&](int it, u32x4 (&dst)[KC]) __attribute__((always_inline)) {
        const int my_t = (it % nb) * kQzBlock + tl;
        const bool in = it < total && my_t < N;
        const uint16_t *xrow = X + (in ? ((size_t)(it / nb) * N + my_t) * D + 64 * h : (size_t)0);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(xrow + 8 * kc);
            dst[kc] = in ? v : u32x4{};
        }
    };
    auto process = [&](int item, const u32x4 (&xb)[KC]) __attribute__((always_inline)) {
        const int bh = item / nb, t0 = (item % nb) * kQzBlock;
        // ROT: y^T tile nt, lane = token tl, element 4 a + e = output channel
        // 32 nt + 8 a + 4 h + e. Without R, y = x as loaded (signed zeros kept).
        [[maybe_unused]] f32x16 y[NT];
        float amax = 0.f;
        if constexpr (ROT) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                y[nt] = f32x16{};
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const u32x2 a0 = lds_tr(sr + 16 * kc * ROW + tro[0][nt]);
                    const u32x2 a1 = lds_tr(sr + 16 * kc * ROW + tro[1][nt]);
                    y[nt] = mfma(u32x4{a0[0], a0[1], a1[0], a1[1]}, xb[kc], y[nt]);
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[nt][i]));
            }
        } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(xb[kc][j])), fabsf(bf16_hi(xb[kc][j]))));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        if (lane == 0) wmax[w] = amax;
        lds_barrier();   // LDS only: the next item's loads stay in flight
        const float bmax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        const float s = bmax > 0.f ? bmax / 448.f : 1.f;
        // y / s rounded correctly to fp32. For 2^-80 <= s <= 2^100 (every
        // block of ordinary data) it is refined from q0 = y * RN(1/s) with two
        // exact-residual steps, e = y - q s by fma and q + e RN(1/s) rounded
        // (Markstein's quotient refinement: a faithful q and a correctly rounded
        // reciprocal give the correctly rounded quotient; the first step makes
        // q faithful). In that range a residual can only fall below the normal
        // fp32 range when |y / s| < 2^-22, whose code is a signed zero either
        // way. Outside it, the division instruction sequence.
        const float r = 1.f / s;
        const bool refine = s >= 0x1p-80f && s <= 0x1p100f;
        auto quot = [s, r](float v, auto fc) {
            if constexpr (decltype(fc)::value) {
                const float q0 = v * r;
                const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, v), r, q0);
                const float q = __builtin_fmaf(__builtin_fmaf(-q1, s, v), r, q1);
                return __builtin_copysignf(q, v);   // -0 stays -0
            } else {
                return v / s;
            }
        };

        // codes as rows [token][channel]; the 16-byte chunk c of row r sits at
        // c ^ ((r / 2) % 8), so that the writes of 32 tokens spread over the banks
        uint8_t *srow = sc + tl * D;
        const int sw = (tl >> 1) & 7;
        auto emit = [&](auto fc) __attribute__((always_inline)) {
        auto code4 = [&](float v0, float v1, float v2, float v3) {
            const float q0 = fminf(fmaxf(quot(v0, fc), -448.f), 448.f), q1 = fminf(fmaxf(quot(v1, fc), -448.f), 448.f);
            const float q2 = fminf(fmaxf(quot(v2, fc), -448.f), 448.f), q3 = fminf(fmaxf(quot(v3, fc), -448.f), 448.f);
            const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
            return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, lo, true);
        };
        if constexpr (ROT) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int c16 = (2 * nt + (a >> 1)) ^ sw;
                    *reinterpret_cast<uint32_t *>(srow + 16 * c16 + 8 * (a & 1) + 4 * h) =
                        code4(y[nt][4 * a], y[nt][4 * a + 1], y[nt][4 * a + 2], y[nt][4 * a + 3]);
                }
        } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const u32x4 v = xb[kc];
                const int c16 = (4 * h + (kc >> 1)) ^ sw;
                *reinterpret_cast<u32x2 *>(srow + 16 * c16 + 8 * (kc & 1)) =
                    u32x2{code4(bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1])),
                          code4(bf16_lo(v[2]), bf16_hi(v[2]), bf16_lo(v[3]), bf16_hi(v[3]))};
            }
        }
        };
        if (refine) emit(std::true_type{});
        else emit(std::false_type{});
        lds_barrier();
        for (int idx = tid; idx < kQzBlock * D / 16; idx += kQzThreads) {   // 16-byte pieces
            const int r = idx / (D / 16), c = idx % (D / 16);
            if (t0 + r < N)
                // the codes are written once and not read back here: non-temporal
                // stores (measured: 28.5 -> 23.6 us per tensor with R, 24.7 ->
                // 20.1 us without; the same hint on the loads, whose 16-byte
                // pieces of a line come from 8 different instructions, made
                // them 40 % slower)
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(sc + r * D + 16 * (c ^ ((r >> 1) & 7))),
                                            reinterpret_cast<u32x4 *>(codes + ((size_t)bh * N + t0 + r) * D + c * 16));
        }
        if (tid == 0) scales[item] = s;
    };
    u32x4 xa[KC], xc[KC];
    load_item(blockIdx.x, xa);
    for (int item = blockIdx.x; item < total; item += 2 * (int)gridDim.x) {
        load_item(item + gridDim.x, xc);
        process(item, xa);
        if (item + (int)gridDim.x >= total) break;
        load_item(item + 2 * gridDim.x, xa);
        process(item + gridDim.x, xc);
    }
}

}  // namespace

hipError_t launch_fp8_quantize(const void *x, const void *rot, uint8_t *codes, float *scales, int B, int H,
                               int N, hipStream_t stream)
{
    const int nb = (N + kQzBlock - 1) / kQzBlock;
    const int total = B * H * nb;
    const int grid = total < kQzGrid ? total : kQzGrid;
    const uint16_t *xp = static_cast<const uint16_t *>(x), *rp = static_cast<const uint16_t *>(rot);
    if (rp)
        hipLaunchKernelGGL(fp8_quant_kernel<true>, dim3((unsigned)grid), dim3(kQzThreads), 0, stream, xp, rp, codes,
                           scales, N, nb, total);
    else
        hipLaunchKernelGGL(fp8_quant_kernel<false>, dim3((unsigned)grid), dim3(kQzThreads), 0, stream, xp, rp, codes,
                           scales, N, nb, total);
    return hipGetLastError();
}

}  // namespace fa
