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
// One launch can take up to three tensors of one shape (Q, K and V of the FP8
// forward): their token blocks form one list of items, the first ones
// multiplied by R and the rest not, so that one grid with one R load covers
// what would otherwise be three launches, each with its own start and tail.
#include "fa_device.h"
#include "fa_dma.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kQzThreads = 256;
constexpr int kQzBlock = 128;   // tokens per scale block, one per loop trip
constexpr int kQzGrid = 768;    // 3 workgroups per CU (registers, and 48 KiB of LDS with R)
constexpr int kRsrcFlags = 0x00020000;   // buffer descriptor word 3: raw access, reads past the size return 0
constexpr int kNonTemporal = 2;          // cache-policy operand of a buffer store: nt

// The tensors of one launch. Job j reads x[j] and writes codes[j] and
// scales[j]; jobs j < nrot are multiplied by R.
struct QzJobs {
    const uint16_t *x[3];
    uint8_t *codes[3];
    float *scales[3];
};

// Entry j of a kernel-argument array for a wave-uniform j, as selects (an
// indexed access to a by-value argument would go through private memory).
template <typename T>
__device__ __forceinline__ T pick3(const T (&a)[3], int j)
{
    return j == 0 ? a[0] : j == 1 ? a[1] : a[2];
}

// ROT: R is loaded and jobs [0, nrot) are rotated; MIXED: some jobs are not
// (both item kinds are compiled in). Items are (job, b * H + h, 128-token
// block), per = B * H * nb items per job, total = per * jobs.
template <bool ROT, bool MIXED>
// Three workgroups per CU (kQzGrid) need at most 168 registers per lane.
__global__ __launch_bounds__(kQzThreads) __attribute__((amdgpu_waves_per_eu(3))) void fp8_quant_kernel(QzJobs jobs, const uint16_t *__restrict__ R,
                                                              int nrot, int N, int nb, int per, int total)
{
    constexpr int D = 128, ROW = 2 * D, CPR = D / 8, KC = D / 16, NT = D / 32;
    __shared__ __attribute__((aligned(16))) uint8_t sc[kQzBlock * D];  // codes of one block
    __shared__ float wmax[2][4];   // per-wave maxima, double-buffered by item parity

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

    // Memory goes through buffer descriptors sized to the item's rows, so that
    // rows past N (the short last block of a (b, h)) read as zeros and their
    // stores are dropped by the hardware: no branch and no select, and the
    // compiler knows how many loads and stores are in flight, so that waiting
    // for a prefetched item does not also wait for the previous item's stores.
    auto rows_of = [&](int loc) { return min(kQzBlock, N - (loc % nb) * kQzBlock); };
    auto block_off = [&](int loc) { return ((size_t)(loc / nb) * N + (size_t)(loc % nb) * kQzBlock) * D; };
    // Token tl of an item, channels 64 h + 8 kc + 0..7 (the MFMA's B operand
    // x^T). Two register sets alternate: the next item's part is loaded before
    // the current one is processed, so its latency overlaps the work. An item
    // past the end reads zeros (a descriptor of 0 bytes).
    auto load_item = [&](int it, u32x4 (&dst)[KC]) __attribute__((always_inline)) {
        const bool live = it < total;
        const int j = live ? it / per : 0, loc = it - j * per;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(pick3(jobs.x, j) + (live ? block_off(loc) : 0)), 0, live ? rows_of(loc) * D * 2 : 0, kRsrcFlags);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            dst[kc] = __builtin_amdgcn_raw_buffer_load_b128(rs, tl * D * 2 + 128 * h + 16 * kc, 0, 0);
    };
    // M = 0: a plain item; 1: a rotated item; 2: decided per item (jobs
    // [0, nrot) rotated), with one body for both kinds so that the mixed
    // kernel needs no more registers than the rotated one.
    auto process_as = [&](int item, const u32x4 (&xb)[KC], auto modec, auto parc) __attribute__((always_inline)) {
        constexpr int M = decltype(modec)::value;
        constexpr int PAR = decltype(parc)::value;   // parity of the item in this workgroup's sequence
        const int j = item / per, loc = item - j * per;
        uint8_t *const codes = pick3(jobs.codes, j);
        const bool rot_item = M == 1 || (M == 2 && item < nrot * per);
        // y, rotated items: tile nt, lane = token tl, element 4 a + e = output
        // channel 32 nt + 8 a + 4 h + e. Plain items with M = 2: element 4 a + e
        // of tile nt = channel 64 h + 16 nt + 4 a + e (as loaded). With M = 0,
        // y is not formed and x is used as loaded. Signed zeros are kept.
        [[maybe_unused]] f32x16 y[NT];
        float amax = 0.f;
        if constexpr (M != 0) {
            if (rot_item) {
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
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t wd = xb[2 * nt + (a >> 1)][2 * (a & 1) + (e >> 1)];
                            y[nt][4 * a + e] = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
                            amax = fmaxf(amax, fabsf(y[nt][4 * a + e]));
                        }
            }
        } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(xb[kc][i])), fabsf(bf16_hi(xb[kc][i]))));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        // The one barrier per item (LDS only: the next item's loads stay in
        // flight). A wave writes wmax[PAR] again only two items later, after
        // the next item's barrier, which every wave reaches after reading it.
        if (lane == 0) wmax[PAR][w] = amax;
        lds_barrier();
        const float bmax = fmaxf(fmaxf(wmax[PAR][0], wmax[PAR][1]), fmaxf(wmax[PAR][2], wmax[PAR][3]));
        const float s = bmax > 0.f ? bmax / 448.f : 1.f;
        // y / s rounded correctly to fp32. For 2^-80 <= s <= 2^100 (every
        // block of ordinary data) it is refined from q0 = y * RN(1/s) with two
        // exact-residual steps, e = y - q s by fma and q + e RN(1/s) rounded
        // (Markstein's quotient refinement: a faithful q and a correctly rounded
        // reciprocal give the correctly rounded quotient; the first step makes
        // q faithful). In that range a residual can only fall below the normal
        // fp32 range when |y / s| < 2^-22, whose code is a signed zero either
        // way. Outside it, the division instruction sequence. The residual is
        // formed negated, e' = RN(q s - y) = -e exactly, and the step is
        // RN(q - e' r): the same value for y != 0, and for y = -0 every step
        // stays -0 (q s - y and -e' r are then -0 + +0 = +0 and -0 + -0 = -0),
        // so that the sign of a zero needs no separate copy.
        const float r = 1.f / s;
        const bool refine = s >= 0x1p-80f && s <= 0x1p100f;
        auto quot = [s, r](float v, auto fc) {
            if constexpr (decltype(fc)::value) {
                const float q0 = v * r;
                const float q1 = __builtin_fmaf(-__builtin_fmaf(q0, s, -v), r, q0);
                return __builtin_fmaf(-__builtin_fmaf(q1, s, -v), r, q1);
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
            // the low half first; the high half of the old operand (any dead
            // value) is replaced by the second conversion
            const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, __float_as_uint(q0), false);
            return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, lo, true);
        };
        if constexpr (M != 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    // 4 consecutive channels: 16-byte chunk and byte within it
                    const int c16 = (rot_item ? 2 * nt + (a >> 1) : 4 * h + nt) ^ sw;
                    const int off = rot_item ? 8 * (a & 1) + 4 * h : 4 * a;
                    *reinterpret_cast<uint32_t *>(srow + 16 * c16 + off) =
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
        // Each wave stores the rows of its own 32 tokens (4 KiB, contiguous in
        // memory), which it staged itself: its LDS writes and reads complete in
        // issue order, so no barrier is needed between them, and the staging
        // rows are rewritten only by the same wave's next item. The codes are
        // written once and not read back here: non-temporal stores (measured:
        // 28.5 -> 23.6 us per tensor with R, 24.7 -> 20.1 us without; the same
        // hint on the loads, whose 16-byte pieces of a line come from 8
        // different instructions, made them 40 % slower).
        const __amdgpu_buffer_rsrc_t cs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(codes + block_off(loc)), 0, rows_of(loc) * D, kRsrcFlags);
#pragma unroll
        for (int i = 0; i < 32 * D / 16 / 64; ++i) {   // 16-byte pieces of the wave's rows
            const int idx = lane + 64 * i, r = 32 * w + idx / (D / 16), c = idx % (D / 16);
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4 *>(sc + r * D + 16 * (c ^ ((r >> 1) & 7))),
                                                   cs, 16 * (32 * w * (D / 16) + idx), 0, kNonTemporal);
        }
        // one scale per item, from thread 0 (the descriptor holds 4 bytes)
        const __amdgpu_buffer_rsrc_t ss =
            __builtin_amdgcn_make_buffer_rsrc((void *)(pick3(jobs.scales, j) + loc), 0, 4, kRsrcFlags);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), ss, 4 * tid, 0, 0);
    };
    auto process = [&](int item, const u32x4 (&xb)[KC], auto parc) __attribute__((always_inline)) {
        process_as(item, xb, std::integral_constant<int, !ROT ? 0 : MIXED ? 2 : 1>{}, parc);
    };
    u32x4 xa[KC], xc[KC];
    load_item(blockIdx.x, xa);
    for (int item = blockIdx.x; item < total; item += 2 * (int)gridDim.x) {
        load_item(item + gridDim.x, xc);
        process(item, xa, std::integral_constant<int, 0>{});
        if (item + (int)gridDim.x >= total) break;
        load_item(item + 2 * gridDim.x, xa);
        process(item + gridDim.x, xc, std::integral_constant<int, 1>{});
    }
}

}  // namespace

static hipError_t launch_jobs(const QzJobs &jobs, int njobs, const uint16_t *rp, int nrot, int B, int H, int N,
                              hipStream_t stream)
{
    const int nb = (N + kQzBlock - 1) / kQzBlock;
    const int per = B * H * nb, total = per * njobs;
    const int grid = total < kQzGrid ? total : kQzGrid;
    if (nrot == njobs)
        hipLaunchKernelGGL((fp8_quant_kernel<true, false>), dim3((unsigned)grid), dim3(kQzThreads), 0, stream, jobs,
                           rp, nrot, N, nb, per, total);
    else if (nrot > 0)
        hipLaunchKernelGGL((fp8_quant_kernel<true, true>), dim3((unsigned)grid), dim3(kQzThreads), 0, stream, jobs,
                           rp, nrot, N, nb, per, total);
    else
        hipLaunchKernelGGL((fp8_quant_kernel<false, false>), dim3((unsigned)grid), dim3(kQzThreads), 0, stream, jobs,
                           rp, nrot, N, nb, per, total);
    return hipGetLastError();
}

hipError_t launch_fp8_quantize(const void *x, const void *rot, uint8_t *codes, float *scales, int B, int H,
                               int N, hipStream_t stream)
{
    const QzJobs jobs{{static_cast<const uint16_t *>(x), nullptr, nullptr}, {codes, nullptr, nullptr},
                      {scales, nullptr, nullptr}};
    return launch_jobs(jobs, 1, static_cast<const uint16_t *>(rot), rot ? 1 : 0, B, H, N, stream);
}

hipError_t launch_fp8_quantize_qkv(const void *q, const void *k, const void *v, const void *rot, uint8_t *q_codes,
                                   uint8_t *k_codes, uint8_t *v_codes, float *q_scales, float *k_scales,
                                   float *v_scales, int B, int H, int N, hipStream_t stream)
{
    const QzJobs jobs{{static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v)},
                      {q_codes, k_codes, v_codes},
                      {q_scales, k_scales, v_scales}};
    return launch_jobs(jobs, 3, static_cast<const uint16_t *>(rot), rot ? 2 : 0, B, H, N, stream);
}

}  // namespace fa
