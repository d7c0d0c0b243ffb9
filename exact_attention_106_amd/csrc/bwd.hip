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
//   bwd_dot:   D_i = dO_i . O_i in fp32 (into the workspace)
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
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdBlock = 128;   // keys of a dK/dV workgroup, queries of a dQ workgroup
constexpr int kBwdTile = 64;     // rows of a streamed tile

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 lds16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ u32x2 lds_tr(const uint8_t *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(const_cast<uint8_t *>(p)));
    return __builtin_bit_cast(u32x2, r);
}

// A operand X^T (32 channels of channel tile t x 16 rows) of a row-major LDS
// tile X of 16-byte-chunk rows (CPR chunks, swizzled), rows 16 c .. 16 c + 15
// at + 16 c ROW: two ds_read_b64_tr_b16 at these offsets (rd = 0, 1). Each lane
// receives, for its channel, the 8 rows that the B operand made of 8
// consecutive accumulator elements (rows 4h + 0..3 and 8 + 4h + 0..3 of a
// 16-row half of a 32-row accumulator) holds in the same order.
template <int CPR>
__device__ __forceinline__ uint32_t tr_offset(int lane, int rd, int t) {
    const int g = lane >> 4, e = (lane & 15) >> 2, jj = lane & 3;
    const int r = 8 * rd + 4 * (g >> 1) + e;
    const int c = 4 * t + 2 * (g & 1) + (jj >> 1);
    return (uint32_t)(r * CPR * 16 + ((c ^ swz<CPR>(r)) << 4) + 8 * (jj & 1));
}

// A operand row read: row R of a tile, channels 16 kc + 8 h .. + 7
template <int CPR>
__device__ __forceinline__ uint32_t row_offset(int R, int kc, int h) {
    return (uint32_t)(R * CPR * 16 + (((2 * kc + h) ^ swz<CPR>(R)) << 4));
}

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i, fp32. D / 8 lanes per row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dot_kernel(const uint16_t *__restrict__ O,
                                                              const uint16_t *__restrict__ dO,
                                                              float *__restrict__ Dlt, long rows)
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
    if (row < rows && part == 0) Dlt[row] = acc;
}

// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint16_t *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Dlt,
    uint16_t *__restrict__ dK, uint16_t *__restrict__ dV, int N, int BH, float scale)
{
    constexpr int ROW = 2 * D, CPR = D / 8, KC = D / 16, DT = D / 32;
    constexpr int TILE = kBwdTile * ROW;
    constexpr int LD = kBwdTile * CPR / kBwdThreads;   // 16-byte loads per thread, tile and tensor
    __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE];   // [stage][Q, dO]
    __shared__ __attribute__((aligned(16))) float rowv[2][2][kBwdTile]; // [stage][L log2 e, D][query]

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
    const int kb = blockIdx.x / BH, bh = blockIdx.x % BH;
    const int k0 = kb * kBwdBlock;
    const int kw = k0 + 32 * w;
    const int my_key = kw + l32;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * ROW;
    const auto rq = make_rsrc(Q + head, head_bytes);
    const auto rdo = make_rsrc(dO + head, head_bytes);
    const auto rk = make_rsrc(K + head, head_bytes);
    const auto rv = make_rsrc(V + head, head_bytes);

    // K and V of this lane's key as B operands (keys past N read zeros)
    u32x4 kr[KC], vr[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const uint32_t off = (uint32_t)my_key * ROW + (16 * kc + 8 * h) * 2;
        kr[kc] = buf_load16(rk, off);
        vr[kc] = buf_load16(rv, off);
    }
    uint32_t tro[2][DT];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int t = 0; t < DT; ++t) tro[rd][t] = tr_offset<CPR>(lane, rd, t);

    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) dk[t] = dv[t] = f32x16{};

    const int n_qt = (N + kBwdTile - 1) / kBwdTile;
    const int t0 = CAUSAL ? k0 / kBwdTile : 0;
    const float c = scale * kLog2e;

    // tile copies: HBM -> registers (issued before the compute of the
    // previous tile) -> LDS stage (after it). Rows past N read zeros, and
    // their L and D are 0: their P is then finite and dO = 0 makes their
    // contributions vanish.
    u32x4 ldq[LD], lddo[LD];
    float ldr = 0.f;
    auto gload = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int idx = tid + i * kBwdThreads;
            const uint32_t off = (uint32_t)(t * kBwdTile + idx / CPR) * ROW + (idx % CPR) * 16;
            ldq[i] = buf_load16(rq, off);
            lddo[i] = buf_load16(rdo, off);
        }
        const int q = t * kBwdTile + (tid & 63);
        ldr = 0.f;
        if (tid < 128 && q < N) ldr = tid < 64 ? LSE[(size_t)bh * N + q] * kLog2e : Dlt[(size_t)bh * N + q];
    };
    auto sstore = [&](int s) __attribute__((always_inline)) {
        uint8_t *sq = smem + s * 2 * TILE;
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int idx = tid + i * kBwdThreads;
            const int r = idx / CPR, cc = idx % CPR;
            const uint32_t off = (uint32_t)(r * ROW + ((cc ^ swz<CPR>(r)) << 4));
            *reinterpret_cast<u32x4 *>(sq + off) = ldq[i];
            *reinterpret_cast<u32x4 *>(sq + TILE + off) = lddo[i];
        }
        if (tid < 128) rowv[s][tid >> 6][tid & 63] = ldr;
    };

    gload(t0);
    sstore(0);
    __syncthreads();
    for (int t = t0; t < n_qt; ++t) {
        const int s = (t - t0) & 1;
        if (t + 1 < n_qt) gload(t + 1);
        const int q0 = t * kBwdTile;
        // causal: a tile whose queries all precede the wave's keys adds nothing
        if (!CAUSAL || q0 + kBwdTile - 1 >= kw) {
            const uint8_t *sq = smem + s * 2 * TILE, *sdo = sq + TILE;
            bf16x8 pb[4], dsb[4];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                f32x16 sacc = {}, pacc = {};
                const int R = qt * 32 + l32;
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const uint32_t off = row_offset<CPR>(R, kc, h);
                    sacc = mfma(lds16(sq + off), kr[kc], sacc);
                    pacc = mfma(lds16(sdo + off), vr[kc], pacc);
                }
                // element 4a + b of the accumulators is query qt*32 + 8a + 4h + b
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const f32x4 lv = *reinterpret_cast<const f32x4 *>(&rowv[s][0][qt * 32 + 8 * a + 4 * h]);
                    const f32x4 dl = *reinterpret_cast<const f32x4 *>(&rowv[s][1][qt * 32 + 8 * a + 4 * h]);
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int i = 4 * a + b;
                        float p = exp2_hw(sacc[i] * c - lv[b]);
                        if (CAUSAL && my_key > q0 + qt * 32 + 8 * a + 4 * h + b) p = 0.f;
                        const float ds = p * (pacc[i] - dl[b]);
                        pb[2 * qt + (a >> 1)][4 * (a & 1) + b] = (__bf16)p;
                        dsb[2 * qt + (a >> 1)][4 * (a & 1) + b] = (__bf16)ds;
                    }
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS, 16 queries per step
#pragma unroll
            for (int kq = 0; kq < 4; ++kq)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const uint32_t o0 = tro[0][dt] + 16 * kq * ROW, o1 = tro[1][dt] + 16 * kq * ROW;
                    const u32x2 a0 = lds_tr(sdo + o0), a1 = lds_tr(sdo + o1);
                    dv[dt] = mfma(u32x4{a0[0], a0[1], a1[0], a1[1]}, __builtin_bit_cast(u32x4, pb[kq]), dv[dt]);
                    const u32x2 b0 = lds_tr(sq + o0), b1 = lds_tr(sq + o1);
                    dk[dt] = mfma(u32x4{b0[0], b0[1], b1[0], b1[1]}, __builtin_bit_cast(u32x4, dsb[kq]), dk[dt]);
                }
        }
        if (t + 1 < n_qt) sstore(s ^ 1);
        __syncthreads();
    }

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
    const uint16_t *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Dlt,
    uint16_t *__restrict__ dQ, int N, int BH, int n_qb, float scale)
{
    constexpr int ROW = 2 * D, CPR = D / 8, KC = D / 16, DT = D / 32;
    constexpr int TILE = kBwdTile * ROW;
    constexpr int LD = kBwdTile * CPR / kBwdThreads;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE];   // [stage][K, V]

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, h = lane >> 5;
    const int rank = blockIdx.x / BH, bh = blockIdx.x % BH;
    const int qb = CAUSAL ? n_qb - 1 - rank : rank;
    const int qw = qb * kBwdBlock + 32 * w;
    const int my_q = qw + l32;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * ROW;
    const auto rq = make_rsrc(Q + head, head_bytes);
    const auto rdo = make_rsrc(dO + head, head_bytes);
    const auto rk = make_rsrc(K + head, head_bytes);
    const auto rv = make_rsrc(V + head, head_bytes);

    // Q^T and dO^T of this lane's query as B operands; its L and D
    u32x4 qr[KC], dor[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const uint32_t off = (uint32_t)my_q * ROW + (16 * kc + 8 * h) * 2;
        qr[kc] = buf_load16(rq, off);
        dor[kc] = buf_load16(rdo, off);
    }
    const float l2 = my_q < N ? LSE[(size_t)bh * N + my_q] * kLog2e : 0.f;
    const float dd = my_q < N ? Dlt[(size_t)bh * N + my_q] : 0.f;
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
    const float c = scale * kLog2e;

    u32x4 ldk[LD], ldv[LD];
    auto gload = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int idx = tid + i * kBwdThreads;
            const uint32_t off = (uint32_t)(t * kBwdTile + idx / CPR) * ROW + (idx % CPR) * 16;
            ldk[i] = buf_load16(rk, off);
            ldv[i] = buf_load16(rv, off);
        }
    };
    auto sstore = [&](int s) __attribute__((always_inline)) {
        uint8_t *sk = smem + s * 2 * TILE;
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int idx = tid + i * kBwdThreads;
            const int r = idx / CPR, cc = idx % CPR;
            const uint32_t off = (uint32_t)(r * ROW + ((cc ^ swz<CPR>(r)) << 4));
            *reinterpret_cast<u32x4 *>(sk + off) = ldk[i];
            *reinterpret_cast<u32x4 *>(sk + TILE + off) = ldv[i];
        }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int t = 0; t < n_kt; ++t) {
        const int s = t & 1;
        if (t + 1 < n_kt) gload(t + 1);
        const int k0 = t * kBwdTile;
        // causal: a tile whose keys all follow the wave's queries adds nothing
        if (!CAUSAL || k0 <= qw + 31) {
            const uint8_t *sk = smem + s * 2 * TILE, *sv = sk + TILE;
            bf16x8 dsb[4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x16 sacc = {}, pacc = {};
                const int R = kt * 32 + l32;
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const uint32_t off = row_offset<CPR>(R, kc, h);
                    sacc = mfma(lds16(sk + off), qr[kc], sacc);
                    pacc = mfma(lds16(sv + off), dor[kc], pacc);
                }
                // element 4a + b is key k0 + kt*32 + 8a + 4h + b
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + kt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                    float p = exp2_hw(sacc[i] * c - l2);
                    if (key >= N || (CAUSAL && key > my_q)) p = 0.f;
                    dsb[2 * kt + (i >> 3)][i & 7] = (__bf16)(p * (pacc[i] - dd));
                }
            }
            // dQ^T += K^T dS^T, 16 keys per step
#pragma unroll
            for (int ch = 0; ch < 4; ++ch)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const u32x2 a0 = lds_tr(sk + tro[0][dt] + 16 * ch * ROW);
                    const u32x2 a1 = lds_tr(sk + tro[1][dt] + 16 * ch * ROW);
                    dq[dt] = mfma(u32x4{a0[0], a0[1], a1[0], a1[1]}, __builtin_bit_cast(u32x4, dsb[ch]), dq[dt]);
                }
        }
        if (t + 1 < n_kt) sstore(s ^ 1);
        __syncthreads();
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
                        float *dlt, hipStream_t stream)
{
    const auto *Q = static_cast<const uint16_t *>(q), *K = static_cast<const uint16_t *>(k);
    const auto *V = static_cast<const uint16_t *>(v), *O = static_cast<const uint16_t *>(o);
    const auto *G = static_cast<const uint16_t *>(dout);
    const long rows = (long)BH * N;
    const long dot_threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_dot_kernel<D>), dim3((unsigned)((dot_threads + kBwdThreads - 1) / kBwdThreads)),
                       dim3(kBwdThreads), 0, stream, O, G, dlt, rows);
    const int nb = (N + kBwdBlock - 1) / kBwdBlock;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(nb * BH)), dim3(kBwdThreads), 0, stream,
                       Q, K, V, G, lse, dlt, static_cast<uint16_t *>(dk), static_cast<uint16_t *>(dv), N, BH,
                       scale);
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(nb * BH)), dim3(kBwdThreads), 0, stream,
                       Q, K, V, G, lse, dlt, static_cast<uint16_t *>(dq), N, BH, nb, scale);
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
