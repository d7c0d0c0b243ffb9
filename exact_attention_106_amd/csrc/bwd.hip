// Attention backward on gfx950 MFMA, bf16 in / bf16 out (d = 64, 128).
//
// Recomputation (FlashAttention v1 backward and the v2 "keep only L" change of
// the 91haoming.cn FlashAttention v1-v3 article; backward part of "Flash
// Attention 再学习"): the forward pass keeps O and the row logsumexp L only, and
// the backward pass rebuilds every tile of P = exp(scale Q K^T - L) on chip
// from Q, K and L, so no N x N matrix reaches memory. Per (query i, key j):
//   dV_j += P_ij dO_i                  dP_ij = dO_i . V_j
//   dS_ij = P_ij (dP_ij - D_i),        D_i = dO_i . O_i  (= sum_j P_ij dP_ij)
//   dQ_i += scale dS_ij K_j            dK_j += scale dS_ij Q_i
//
// Parallelisation over column (key) blocks, as in the FlashAttention-2
// backward of the same article: a column block owns its dK and dV, which
// therefore need no communication. dQ, the sum over column blocks, comes from
// a second kernel parallel over row blocks that recomputes P and dP for its
// rows: two more tile products per tile instead of atomic adds into an fp32
// buffer, and the result is deterministic. Three kernels:
//   bwd_dot:   per row -L_i / scale and -D_i, D_i = dO_i . O_i (fp32, into
//              the workspace)
//   bwd_dkdv:  workgroup per (b*h, 128 keys), 4 waves x 32 keys; tiles of 64
//              queries (Q, dO, L, D) stream through LDS
//   bwd_dq:    workgroup per (b*h, 128 queries), 4 waves x 32 queries; tiles
//              of 64 keys (K, V) stream through LDS
// Causal grids are issued heaviest block first.
//
// MFMA orientation (v_mfma_f32_32x32x16_bf16; in its accumulator a lane holds
// one column and 16 rows). bwd_dkdv computes S = Q K^T and dP = dO V^T with
// the wave's 32 keys as columns (K and V are B operands kept in registers), so
// P and dS come out with one key per lane and 16 queries: the B-operand layout
// of dV^T += dO^T P and dK^T += Q^T dS, whose A operands dO^T and Q^T are read
// from the row-major LDS tiles with ds_read_b64_tr_b16, so that each lane gets
// the queries its P registers hold (queries are the summation index there,
// only the pairing matters). bwd_dq is the mirror image with queries as
// columns: S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T.
#include "fa_device.h"
#include "fa_dma.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdBlock = 128;   // keys of a dK/dV workgroup, queries of a dQ workgroup
constexpr int kBwdTile = 64;     // rows of a streamed tile

// ---------------------------------------------------------------------------
// Per row: nl_i = -L_i / scale and nd_i = -D_i = -(dO_i . O_i), fp32, into the
// workspace [2][rows]. They start the S and dP accumulators of bwd_dkdv, so
// that S - L / scale and dP - D come straight out of the MFMAs. D / 8 lanes
// per row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dot_kernel(const uint16_t *__restrict__ O,
                                                              const uint16_t *__restrict__ dO,
                                                              const float *__restrict__ LSE,
                                                              float *__restrict__ ws, long rows,
                                                              float inv_scale)
{
    constexpr int LPR = D / 8;
    const long gid = (long)blockIdx.x * kBwdThreads + threadIdx.x;
    const long row = gid / LPR;
    const int part = (int)(gid % LPR);
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(O + row * D + part * 8);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(dO + row * D + part * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += bf16_lo(a[e]) * bf16_lo(b[e]) + bf16_hi(a[e]) * bf16_hi(b[e]);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (row < rows && part == 0) {
        ws[row] = -LSE[row] * inv_scale;
        ws[rows + row] = -acc;
    }
}

// Block of this workgroup: the rank-th block (heaviest first under causal
// masking) of head bh. Workgroup ids go round-robin over the GPU's 8 XCDs,
// each with its own L2. When B*H is a multiple of 8, XCD x takes heads x,
// x + 8, x + 16, ... one after the other and the consecutive ids it receives
// are consecutive blocks of one head: the 32 or so workgroups that run
// together on an XCD stream the same head's tiles through its L2, which reads
// each tile from HBM about once per such group. Otherwise consecutive ids are
// the heads of one block.
__device__ __forceinline__ void block_of(int &rank, int &bh, int BH, int n_blocks) {
    if (BH % 8 == 0) {
        const int x = blockIdx.x % 8, j = blockIdx.x / 8;
        rank = j % n_blocks;
        bh = x + 8 * (j / n_blocks);
    } else {
        rank = blockIdx.x / BH;
        bh = blockIdx.x % BH;
    }
}

// S (VGPR, in/out) += A (VGPR) x B (VGPR)
__device__ __forceinline__ void mfma_acc_v(f32x16 &acc, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// O (AGPR, in/out) += A (VGPR) x B (VGPR)
__device__ __forceinline__ void mfma_acc_a(f32x16 &acc, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ dO, const float *__restrict__ NL, const float *__restrict__ ND,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int N, int BH, float scale)
{
    constexpr int ROW = 2 * D, CPR = D / 8, KC = D / 16, DT = D / 32;
    constexpr int TILE = kBwdTile * ROW;
    constexpr int NDMA = TILE / 1024 / 4;              // 1 KiB copies per wave, tile and tensor
    constexpr int ROWS = 4 * TILE;                      // nl and nd of the two stages after the tiles
    // [stage][Q, dO] tiles, then [stage][nl, nd][query] fp32
    __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE + 2 * 2 * kBwdTile * 4];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
    int kb, bh;
    block_of(kb, bh, BH, (N + kBwdBlock - 1) / kBwdBlock);
    const int k0 = kb * kBwdBlock;
    const int kw = k0 + 32 * w;
    const int my_key = kw + l32;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * ROW;
    const auto rk = make_rsrc(K + head, head_bytes);
    const auto rv = make_rsrc(V + head, head_bytes);
    const u32x4 rq = sgpr_rsrc(Q + head, head_bytes);
    const u32x4 rdo = sgpr_rsrc(dO + head, head_bytes);
    const u32x4 rnl = sgpr_rsrc(NL + (size_t)bh * N, (uint32_t)N * 4);
    const u32x4 rnd = sgpr_rsrc(ND + (size_t)bh * N, (uint32_t)N * 4);

    // K and V of this lane's key: B operands (keys past N read zeros); dK^T
    // and dV^T accumulate in AGPRs
    u32x4 kr[KC], vr[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const uint32_t off = (uint32_t)my_key * ROW + (16 * kc + 8 * h) * 2;
        kr[kc] = buf_load16(rk, off);
        vr[kc] = buf_load16(rv, off);
    }
    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) dk[t] = dv[t] = f32x16{};
#pragma unroll
    for (int t = 0; t < DT; ++t) asm volatile("" : "+a"(dk[t]), "+a"(dv[t]));

    uint32_t tro[2][DT];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int t = 0; t < DT; ++t) tro[rd][t] = tr_offset<CPR>(lane, rd, t);
    // row-read offsets of this lane (row l32 of a 32-row half; the swizzle
    // only depends on the row mod 16, so the other half is + 32 ROW)
    uint32_t rowo[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) rowo[kc] = row_offset<CPR>(l32, kc, h);

    const int n_qt = (N + kBwdTile - 1) / kBwdTile;
    const int t0 = CAUSAL ? k0 / kBwdTile : 0;
    const float c = scale * kLog2e;

    // Tile copies go from HBM straight into the other LDS stage while the
    // current tile is computed (each wave copies 1 KiB pieces; the source
    // chunks are permuted so that the LDS rows come out swizzled). Rows past N
    // read zeros (nl = nd = 0 too): their P is finite and dO = 0 makes their
    // contributions vanish.
    const uint32_t lds0 = (uint32_t)(size_t)smem;
    uint32_t dma_off[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int pos = (w * NDMA + i) * 64 + lane;
        const int r = pos / CPR, pc = pos % CPR;
        dma_off[i] = (uint32_t)(r * ROW + ((pc ^ swz<CPR>(r)) << 4));
    }
    auto issue = [&](int t, int st) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)(t * kBwdTile) * ROW;
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds0 + st * 2 * TILE + w * NDMA * 1024);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            dma16(rq, base + i * 1024, dma_off[i], soff);
            dma16(rdo, base + TILE + i * 1024, dma_off[i], soff);
        }
        const uint32_t rbase = __builtin_amdgcn_readfirstlane(lds0 + ROWS + (st * 2 + w) * kBwdTile * 4);
        if (w == 0) dma4(rnl, rbase, (uint32_t)lane * 4, (uint32_t)(t * kBwdTile) * 4);
        if (w == 1) dma4(rnd, rbase, (uint32_t)lane * 4, (uint32_t)(t * kBwdTile) * 4);
    };

    // One tile as a fixed sequence of steps, each with its LDS reads issued
    // LA steps ahead of its two MFMAs and a share of the elementwise work:
    //   steps [0, NSD):   S(qt) = Q_qt K^T - L/scale, dP(qt) = dO_qt V^T - D
    //                     (qt = f / KC; the accumulators start from -L/scale
    //                     and -D of their queries)
    //   steps [NSD, NST): dV^T += dO^T P, dK^T += Q^T dS over 16 queries each
    //   P and dS of qt = 0 are formed during steps [KC, 2 KC), of qt = 1
    //   during the first 2 DT dV/dK steps (which only use qt = 0).
    // The MFMAs are inline asm (the compiler cannot see their latency): the
    // S/dP results are read by VALU only after 20 wait states (s_nop at the
    // end of steps KC - 1 and NSD - 1), and P/dS written by VALU are read by
    // an MFMA at least a step later.
    constexpr int NSD = 2 * KC, NST = NSD + 4 * DT, LA = 4;
    auto tile = [&](int t, auto sc, auto mc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        constexpr bool MASKED = decltype(mc)::value;
        constexpr uint32_t QB = S * 2 * TILE, DB = QB + TILE;   // stage bases in LDS
        const uint8_t *lds = smem;
        const float *rows = reinterpret_cast<const float *>(smem + ROWS + S * 2 * kBwdTile * 4);
        const int q0 = t * kBwdTile;
        u32x4 ra[NST], rb[NST];
        f32x16 sacc[2], pacc[2];
        bf16x8 pb[4], dsb[4];
        auto read = [&](auto fc) __attribute__((always_inline)) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f < NSD) {
                constexpr int qt = f / KC, kc = f % KC;
                ra[f] = lds16(lds + QB + qt * 32 * ROW + rowo[kc]);
                rb[f] = lds16(lds + DB + qt * 32 * ROW + rowo[kc]);
                if constexpr (kc == 0) {
                    // element 4a + b of half qt is query qt*32 + 8a + 4h + b
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const f32x4 x = *reinterpret_cast<const f32x4 *>(rows + qt * 32 + 8 * a + 4 * h);
                        const f32x4 y = *reinterpret_cast<const f32x4 *>(rows + kBwdTile + qt * 32 + 8 * a + 4 * h);
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            sacc[qt][4 * a + b] = x[b];
                            pacc[qt][4 * a + b] = y[b];
                        }
                    }
                }
            } else if constexpr (f < NST) {
                constexpr int kq = (f - NSD) / DT, dt = (f - NSD) % DT;
                const u32x2 a0 = lds_tr(lds + DB + 16 * kq * ROW + tro[0][dt]);
                const u32x2 a1 = lds_tr(lds + DB + 16 * kq * ROW + tro[1][dt]);
                const u32x2 b0 = lds_tr(lds + QB + 16 * kq * ROW + tro[0][dt]);
                const u32x2 b1 = lds_tr(lds + QB + 16 * kq * ROW + tro[1][dt]);
                ra[f] = u32x4{a0[0], a0[1], a1[0], a1[1]};
                rb[f] = u32x4{b0[0], b0[1], b1[0], b1[1]};
            }
        };
        auto elem = [&](int qt, int i) __attribute__((always_inline)) {
            float p = exp2_hw(sacc[qt][i] * c);
            if (MASKED && my_key > q0 + qt * 32 + 8 * (i >> 2) + 4 * h + (i & 3)) p = 0.f;
            pb[2 * qt + (i >> 3)][i & 7] = (__bf16)p;
            dsb[2 * qt + (i >> 3)][i & 7] = (__bf16)(p * pacc[qt][i]);
        };
        static_for<LA>([&](auto fc) { read(fc); });
        static_for<NST>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            read(std::integral_constant<int, f + LA>{});
            if constexpr (f < NSD) {
                constexpr int qt = f / KC, kc = f % KC;
                mfma_acc_v(sacc[qt], ra[f], kr[kc]);
                mfma_acc_v(pacc[qt], rb[f], vr[kc]);
                if constexpr (kc == KC - 1) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3");
            } else {
                constexpr int kq = (f - NSD) / DT, dt = (f - NSD) % DT;
                mfma_acc_a(dv[dt], ra[f], __builtin_bit_cast(u32x4, pb[kq]));
                mfma_acc_a(dk[dt], rb[f], __builtin_bit_cast(u32x4, dsb[kq]));
            }
            // elementwise work of half 0 in steps [KC, 2 KC), of half 1 in [NSD, NSD + KC)
            constexpr int EPS = 16 / KC;
            if constexpr (f >= KC && f < 2 * KC) {
#pragma unroll
                for (int i = (f - KC) * EPS; i < (f - KC + 1) * EPS; ++i) elem(0, i);
            }
            if constexpr (f >= NSD && f < NSD + KC) {
#pragma unroll
                for (int i = (f - NSD) * EPS; i < (f - NSD + 1) * EPS; ++i) elem(1, i);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        // fix P and dS here so that no elementwise work sinks past the tile
#pragma unroll
        for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(pb[k]), "+v"(dsb[k]));
    };

    // Tile t uses LDS stage (t - t0) & 1. The causal mask is only needed on
    // the two tiles that meet this block's keys (computed first; a wave whose
    // keys all follow a tile's queries gets zeros from it). The rest run two
    // per loop iteration, so that the stages are constants and the
    // accumulators follow one path through the loop.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using Plain = std::false_type;
    using Masked = std::true_type;
    auto step = [&](int t, auto sc, auto mc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        if (t + 1 < n_qt) issue(t + 1, S ^ 1);
        tile(t, sc, mc);
        wait_vm_n<0>();
        __syncthreads();
    };
    issue(t0, 0);
    wait_vm_n<0>();
    __syncthreads();
    int t = t0;
    if constexpr (CAUSAL) {
        step(t0, S0{}, Masked{});
        if (t0 + 1 < n_qt) step(t0 + 1, S1{}, Masked{});
        t = t0 + 2;
    }
    for (; t + 1 < n_qt; t += 2) {
        step(t, S0{}, Plain{});
        step(t + 1, S1{}, Plain{});
    }
    if (t < n_qt) step(t, S0{}, Plain{});

    // the last MFMAs wrote dK^T / dV^T: cover the MFMA-write -> read distance
    // (the pins after the nops keep the reads of the accumulators below them)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3");
#pragma unroll
    for (int t = 0; t < DT; ++t) asm volatile("" : "+a"(dk[t]), "+a"(dv[t]));
    // element 4a + b of tile dt is channel 32 dt + 8a + 4h + b of this lane's key
    if (my_key < N) {
        uint16_t *dkp = dK + head + (size_t)my_key * D;
        uint16_t *dvp = dV + head + (size_t)my_key * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int ch = 32 * dt + 8 * a + 4 * h;
                *reinterpret_cast<u32x2 *>(dkp + ch) =
                    u32x2{pack_bf16x2(scale * dk[dt][4 * a], scale * dk[dt][4 * a + 1]),
                          pack_bf16x2(scale * dk[dt][4 * a + 2], scale * dk[dt][4 * a + 3])};
                *reinterpret_cast<u32x2 *>(dvp + ch) =
                    u32x2{pack_bf16x2(dv[dt][4 * a], dv[dt][4 * a + 1]),
                          pack_bf16x2(dv[dt][4 * a + 2], dv[dt][4 * a + 3])};
            }
    }
}

// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dq_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ dO, const float *__restrict__ NL, const float *__restrict__ ND,
    uint16_t *__restrict__ dQ, int N, int BH, int n_qb, float scale)
{
    constexpr int ROW = 2 * D, CPR = D / 8, KC = D / 16, DT = D / 32;
    constexpr int TILE = kBwdTile * ROW;
    constexpr int NDMA = TILE / 1024 / 4;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE];   // [stage][K, V]

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
    int rank, bh;
    block_of(rank, bh, BH, n_qb);
    const int qb = CAUSAL ? n_qb - 1 - rank : rank;
    const int qw = qb * kBwdBlock + 32 * w;
    const int my_q = qw + l32;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * ROW;
    const auto rq = make_rsrc(Q + head, head_bytes);
    const auto rdo = make_rsrc(dO + head, head_bytes);
    const u32x4 rk = sgpr_rsrc(K + head, head_bytes);
    const u32x4 rv = sgpr_rsrc(V + head, head_bytes);

    // Q^T and dO^T of this lane's query as B operands; its L and D
    u32x4 qr[KC], dor[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const uint32_t off = (uint32_t)my_q * ROW + (16 * kc + 8 * h) * 2;
        qr[kc] = buf_load16(rq, off);
        dor[kc] = buf_load16(rdo, off);
    }
    const float c = scale * kLog2e;
    // P = 2^(c (S - L / scale)) and dS = P (dP - D) from nl = -L/scale, nd = -D
    const float nlc = my_q < N ? NL[(size_t)bh * N + my_q] * c : 0.f;
    const float nd = my_q < N ? ND[(size_t)bh * N + my_q] : 0.f;
    uint32_t tro[2][DT];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int t = 0; t < DT; ++t) tro[rd][t] = tr_offset<CPR>(lane, rd, t);

    f32x16 dq[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) dq[t] = f32x16{};

    const int kend = CAUSAL ? min(N, qb * kBwdBlock + kBwdBlock) : N;
    const int n_kt = (kend + kBwdTile - 1) / kBwdTile;

    // K and V tiles go from HBM straight into the other LDS stage (as in
    // bwd_dkdv); keys past N read zeros and are masked
    const uint32_t lds0 = (uint32_t)(size_t)smem;
    uint32_t dma_off[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int pos = (w * NDMA + i) * 64 + lane;
        const int r = pos / CPR, pc = pos % CPR;
        dma_off[i] = (uint32_t)(r * ROW + ((pc ^ swz<CPR>(r)) << 4));
    }
    auto issue = [&](int t, int st) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)(t * kBwdTile) * ROW;
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds0 + st * 2 * TILE + w * NDMA * 1024);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            dma16(rk, base + i * 1024, dma_off[i], soff);
            dma16(rv, base + TILE + i * 1024, dma_off[i], soff);
        }
    };

    uint32_t rowo[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) rowo[kc] = row_offset<CPR>(l32, kc, h);

    // One tile as a fixed sequence of steps (reads LA steps ahead):
    //   steps [0, NSD):   S^T(kt) += K_kt Q^T, dP^T(kt) += V_kt dO^T  (kt = f / KC)
    //   steps [NSD, NST): dQ^T += K^T dS^T over 16 keys each
    //   dS of kt = 0 is formed during steps [KC, 2 KC), of kt = 1 during the
    //   first 2 DT dQ steps (which only use kt = 0).
    constexpr int NSD = 2 * KC, NST = NSD + 4 * DT, LA = 4;
    auto tile = [&](int t, auto sc, auto mc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        constexpr bool MASKED = decltype(mc)::value;
        constexpr uint32_t KB = S * 2 * TILE, VB = KB + TILE;
        const uint8_t *lds = smem;
        const int k0 = t * kBwdTile;
        u32x4 ra[NST], rb[NSD];
        f32x16 sacc[2], pacc[2];
        bf16x8 dsb[4];
        auto read = [&](auto fc) __attribute__((always_inline)) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f < NSD) {
                constexpr int kt = f / KC, kc = f % KC;
                ra[f] = lds16(lds + KB + kt * 32 * ROW + rowo[kc]);
                rb[f] = lds16(lds + VB + kt * 32 * ROW + rowo[kc]);
            } else if constexpr (f < NST) {
                constexpr int ch = (f - NSD) / DT, dt = (f - NSD) % DT;
                const u32x2 a0 = lds_tr(lds + KB + 16 * ch * ROW + tro[0][dt]);
                const u32x2 a1 = lds_tr(lds + KB + 16 * ch * ROW + tro[1][dt]);
                ra[f] = u32x4{a0[0], a0[1], a1[0], a1[1]};
            }
        };
        // element 4a + b of half kt is key k0 + kt*32 + 8a + 4h + b
        auto elem = [&](int kt, int i) __attribute__((always_inline)) {
            const int key = k0 + kt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            float p = exp2_hw(sacc[kt][i] * c + nlc);
            if (MASKED && (key >= N || (CAUSAL && key > my_q))) p = 0.f;
            dsb[2 * kt + (i >> 3)][i & 7] = (__bf16)(p * (pacc[kt][i] + nd));
        };
        static_for<LA>([&](auto fc) { read(fc); });
        static_for<NST>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            read(std::integral_constant<int, f + LA>{});
            if constexpr (f < NSD) {
                constexpr int kt = f / KC, kc = f % KC;
                if constexpr (kc == 0) {
                    sacc[kt] = mfma(ra[f], qr[kc], f32x16{});
                    pacc[kt] = mfma(rb[f], dor[kc], f32x16{});
                } else {
                    sacc[kt] = mfma(ra[f], qr[kc], sacc[kt]);
                    pacc[kt] = mfma(rb[f], dor[kc], pacc[kt]);
                }
            } else {
                constexpr int ch = (f - NSD) / DT, dt = (f - NSD) % DT;
                dq[dt] = mfma(ra[f], __builtin_bit_cast(u32x4, dsb[ch]), dq[dt]);
            }
            constexpr int EPS = 16 / KC;
            if constexpr (f >= KC && f < 2 * KC) {
#pragma unroll
                for (int i = (f - KC) * EPS; i < (f - KC + 1) * EPS; ++i) elem(0, i);
            }
            if constexpr (f >= NSD && f < NSD + KC) {
#pragma unroll
                for (int i = (f - NSD) * EPS; i < (f - NSD + 1) * EPS; ++i) elem(1, i);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // Tile t uses LDS stage t & 1. Only the last tiles need the mask: the
    // two that meet this block's queries (causal) and the one holding key N.
    // The others run two per loop iteration (constant stages, one path for
    // the accumulators); the masked ones follow.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using Plain = std::false_type;
    using Masked = std::true_type;
    auto step = [&](int t, auto sc, auto mc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        if (t + 1 < n_kt) issue(t + 1, S ^ 1);
        tile(t, sc, mc);
        wait_vm_n<0>();
        __syncthreads();
    };
    const int n_plain = CAUSAL ? min(n_kt, 2 * qb) : (N % kBwdTile ? n_kt - 1 : n_kt);
    issue(0, 0);
    wait_vm_n<0>();
    __syncthreads();
    int t = 0;
    for (; t + 1 < n_plain; t += 2) {
        step(t, S0{}, Plain{});
        step(t + 1, S1{}, Plain{});
    }
    if (t < n_plain) step(t++, S0{}, Plain{});
    for (; t < n_kt; ++t) {
        if (t & 1) step(t, S1{}, Masked{});
        else step(t, S0{}, Masked{});
    }

    if (my_q < N) {
        uint16_t *dqp = dQ + head + (size_t)my_q * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int ch = 32 * dt + 8 * a + 4 * h;
                *reinterpret_cast<u32x2 *>(dqp + ch) =
                    u32x2{pack_bf16x2(scale * dq[dt][4 * a], scale * dq[dt][4 * a + 1]),
                          pack_bf16x2(scale * dq[dt][4 * a + 2], scale * dq[dt][4 * a + 3])};
            }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dout, void *dq, void *dk, void *dv, int BH, int N, float scale,
                        float *ws, hipStream_t stream)
{
    const auto *Q = static_cast<const uint16_t *>(q), *K = static_cast<const uint16_t *>(k);
    const auto *V = static_cast<const uint16_t *>(v), *O = static_cast<const uint16_t *>(o);
    const auto *G = static_cast<const uint16_t *>(dout);
    const long rows = (long)BH * N;
    const long dot_threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_dot_kernel<D>), dim3((unsigned)((dot_threads + kBwdThreads - 1) / kBwdThreads)),
                       dim3(kBwdThreads), 0, stream, O, G, lse, ws, rows, 1.f / scale);
    const int nb = (N + kBwdBlock - 1) / kBwdBlock;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(nb * BH)), dim3(kBwdThreads), 0, stream,
                       Q, K, V, G, ws, ws + rows, static_cast<uint16_t *>(dk), static_cast<uint16_t *>(dv), N,
                       BH, scale);
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(nb * BH)), dim3(kBwdThreads), 0, stream,
                       Q, K, V, G, ws, ws + rows, static_cast<uint16_t *>(dq), N, BH, nb, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                           const float *lse, const void *dout, void *dq, void *dk, void *dv, int B,
                           int H, int N, int d, float scale, int causal, float *workspace,
                           hipStream_t stream)
{
    const int BH = B * H;
    if (d == 128)
        return causal ? launch_bwd_t<128, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, N, scale, workspace, stream)
                      : launch_bwd_t<128, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, N, scale, workspace, stream);
    return causal ? launch_bwd_t<64, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, N, scale, workspace, stream)
                  : launch_bwd_t<64, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, N, scale, workspace, stream);
}

}  // namespace fa
