// Block-sparse attention forward with optional dropout on gfx950 MFMA, bf16,
// d = 128.
//
// Block-sparse FlashAttention (91haoming.cn FlashAttention v1-v3 article,
// v1 results): the same fused tile loop, run only over the (query block, key
// block) pairs a block mask keeps, so masked blocks cost neither reads nor
// flops. Blocks are 128 x 128; one mask [ceil(N/128)]^2 serves every batch
// and head; with causal, key blocks past the query block are dropped as well
// and the diagonal is masked inside. Dropout (the "masking and dropout" the
// same article lists among the fused steps): after the softmax, each weight
// P_ij is kept with probability 1 - p and scaled by 1 / (1 - p); l and L are
// those of the weights before dropout. The keep decision comes from
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): key (seed_lo, seed_hi), counter
// (j / 4, i, b * H + h, 0); word j % 4 of the output is u, and P_ij is dropped
// iff u < threshold = floor(p * 2^32).
//
// Structure: workgroup = 4 waves x 32 queries of one (b, h), XCD-aware
// order, two workgroups per CU; the kept key blocks of the query block are
// listed in LDS first, and their 64-key tiles stream through two LDS stages
// by direct copies one tile ahead; S^T = K Q^T with one query per lane,
// online softmax with a lazy reference max, O^T += V^T P^T.
#include "fa_device.h"
#include "fa_dma.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kSpThreads = 256;
constexpr int kSpBlock = 128;     // queries per workgroup = mask block
constexpr int kSpTile = 64;       // keys per tile (two per mask block)
constexpr int kSpMaxTiles = 2048; // N <= 131072

struct Philox {
    uint32_t x[4];
};

// a ^ b ^ c in one instruction: the three-input bitwise op of gfx950 with
// the truth table of XOR (0x96; the compiler emits two XORs here)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32-10: ten rounds of two 32x32->64 multiplies with key bumps
__device__ __forceinline__ Philox philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0), n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return Philox{{c0, c1, c2, c3}};
}

// Two workgroups share a CU (2 waves per SIMD, at most 256 registers, a
// two-stage ring in 68 KiB of LDS): one workgroup's softmax runs while the
// other's MFMAs do, which a single wave's order (S, softmax, P V) does not
// allow.
template <bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(kSpThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_fwd_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const uint8_t *__restrict__ MASK, uint16_t *__restrict__ O, float *__restrict__ LSE, int N, int BH,
    int n_qb, float scale, uint32_t drop_threshold, float inv_keep, uint32_t seed_lo, uint32_t seed_hi)
{
    constexpr int D = 128, ROW = 2 * D, CPR = D / 8, KC = D / 16, DT = D / 32;
    constexpr int TILE = kSpTile * ROW;
    constexpr int NDMA = TILE / 1024 / 4;          // 1 KiB copies per wave and tensor
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 2 * TILE];
    __shared__ int16_t tiles[kSpMaxTiles];
    __shared__ int n_tiles_sh;

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bh, rank;
    if (BH % 8 == 0) {
        const int x = blockIdx.x % 8, j = blockIdx.x / 8;
        rank = j % n_qb;
        bh = 8 * (j / n_qb) + x;
    } else {
        rank = blockIdx.x / BH;
        bh = blockIdx.x % BH;
    }
    const int qb = n_qb - 1 - rank;
    const int qw = qb * kSpBlock + 32 * w;
    const int my_q = qw + l32;
    const int ntt = (N + kSpTile - 1) / kSpTile;   // 64-key tiles of the sequence
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * ROW;

    // the kept tiles of this query block, in key order: wave 0 scans the mask
    // row 64 blocks at a time (ballot + prefix count)
    if (w == 0) {
        int cnt = 0;
        for (int base = 0; base < n_qb; base += 64) {
            const int kb = base + lane;
            const bool act = kb < n_qb && MASK[(size_t)qb * n_qb + kb] != 0 && (!CAUSAL || kb <= qb);
            const bool act2 = act && 2 * kb + 1 < ntt;
            const uint64_t b1 = __builtin_amdgcn_ballot_w64(act), b2 = __builtin_amdgcn_ballot_w64(act2);
            const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            const int pos = cnt + __builtin_popcountll(b1 & below) + __builtin_popcountll(b2 & below);
            if (act) tiles[pos] = (int16_t)(2 * kb);
            if (act2) tiles[pos + 1] = (int16_t)(2 * kb + 1);
            cnt += __builtin_popcountll(b1) + __builtin_popcountll(b2);
        }
        if (lane == 0) n_tiles_sh = cnt;
    }
    __syncthreads();
    const int n_kt = __builtin_amdgcn_readfirstlane(n_tiles_sh);

    const auto rq = make_rsrc(Q + head, head_bytes);
    const u32x4 rk = sgpr_rsrc(K + head, head_bytes), rv = sgpr_rsrc(V + head, head_bytes);
    u32x4 qr[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qr[kc] = buf_load16(rq, (uint32_t)my_q * ROW + (16 * kc + 8 * h) * 2);
    uint32_t tro[2][DT];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int t = 0; t < DT; ++t) tro[rd][t] = tr_offset<CPR>(lane, rd, t);
    uint32_t rowo[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) rowo[kc] = row_offset<CPR>(l32, kc, h);

    // copies of tile kt: rows 16 w .. 16 w + 15 by wave w (source chunks
    // permuted so that the LDS rows come out swizzled); rows past N read zeros
    uint32_t dma_off[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int pos = (w * NDMA + i) * 64 + lane;
        const int r = pos / CPR, pc = pos % CPR;
        dma_off[i] = (uint32_t)(r * ROW + ((pc ^ swz<CPR>(r)) << 4));
    }
    const uint32_t lds0 = (uint32_t)(size_t)smem;
    auto issue = [&](int u, int st) __attribute__((always_inline)) {
        const int kt = __builtin_amdgcn_readfirstlane((int)tiles[u]);
        const uint32_t soff = (uint32_t)(kt * kSpTile) * ROW;
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds0 + st * 2 * TILE + w * NDMA * 1024);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            dma16(rk, base + i * 1024, dma_off[i], soff);
            dma16(rv, base + TILE + i * 1024, dma_off[i], soff);
        }
    };

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
    float m = neg_inf(), lsum = 0.f;
    const float c = scale * kLog2e;

    constexpr int NSD = 2 * KC, NST = NSD + 4 * DT, LA = 4;
    // One tile body for masked and unmasked tiles (the mask is a uniform
    // branch around the masking): two inlined copies made the compiler give O
    // different registers in each and copy all 64 accumulators at the join.
    auto tile = [&](int kt, auto sc, bool masked) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        constexpr uint32_t KB = S * 2 * TILE, VB = KB + TILE;
        const uint8_t *lds = smem;
        const int k0 = kt * kSpTile;
        u32x4 ra[NST];
        f32x16 sacc[2];
        bf16x8 pf[4];
        auto read = [&](auto fc) __attribute__((always_inline)) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f < NSD) {
                constexpr int half = f / KC, kc = f % KC;
                ra[f] = lds16(lds + KB + half * 32 * ROW + rowo[kc]);
            } else if constexpr (f < NST) {
                constexpr int ch = (f - NSD) / DT, dt = (f - NSD) % DT;
                const u32x2 a0 = lds_tr(lds + VB + 16 * ch * ROW + tro[0][dt]);
                const u32x2 a1 = lds_tr(lds + VB + 16 * ch * ROW + tro[1][dt]);
                ra[f] = u32x4{a0[0], a0[1], a1[0], a1[1]};
            }
        };
        auto softmax = [&]() __attribute__((always_inline)) {
            if (masked) {
                // element 4a + b of half s2 is key k0 + 32 s2 + 8a + 4h + b;
                // keys past N, and past the query when causal, are masked
                const int lim = (CAUSAL ? min(my_q, N - 1) : N - 1) - (k0 + 4 * h);
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (32 * s2 + 8 * (i >> 2) + (i & 3) > lim) sacc[s2][i] = neg_inf();
            }
            float mx = neg_inf();
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[s2][i]);
            mx = other_half_max(mx) * c;
            const bool move = mx > m + kRescaleSlack;
            const float m_new = move ? mx : m;
            const float alpha = move ? exp2_hw(m - m_new) : 1.f;
            if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
                for (int t2 = 0; t2 < DT; ++t2) oacc[t2] *= alpha;
            }
            lsum *= alpha;
            m = m_new;
            const float mu = m == neg_inf() ? 0.f : m;
            float rs = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    Philox u{};
                    if constexpr (DROPOUT)
                        u = philox4x32_10((uint32_t)((k0 + 32 * s2 + 8 * a + 4 * h) >> 2), (uint32_t)my_q,
                                          (uint32_t)bh, 0u, seed_lo, seed_hi);
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int i = 4 * a + b;
                        const float p = exp2_hw(fmaf(sacc[s2][i], c, -mu));
                        rs += p;
                        float pv = p;
                        if constexpr (DROPOUT) pv = u.x[b] < drop_threshold ? 0.f : p * inv_keep;
                        pf[2 * s2 + (i >> 3)][i & 7] = (__bf16)pv;
                    }
                }
            lsum += rs;
        };
        static_for<LA>([&](auto fc) { read(fc); });
        static_for<NST>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            read(std::integral_constant<int, f + LA>{});
            if constexpr (f < NSD) {
                constexpr int half = f / KC, kc = f % KC;
                sacc[half] = mfma(ra[f], qr[kc], kc == 0 ? f32x16{} : sacc[half]);
                if constexpr (f == NSD - 1) softmax();
            } else {
                constexpr int ch = (f - NSD) / DT, dt = (f - NSD) % DT;
                oacc[dt] = mfma(ra[f], __builtin_bit_cast(u32x4, pf[ch]), oacc[dt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // Entry u of the list uses LDS stage u mod 2; its step issues the copies
    // of entry u + 1 into the other stage (free since the last barrier) and
    // ends once they have landed. A tile needs the mask when it reaches past
    // N or (causal) past the wave's first query.
    auto step = [&](int u, auto sc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        if (u + 1 < n_kt) issue(u + 1, S ^ 1);
        const int kt = __builtin_amdgcn_readfirstlane((int)tiles[u]);
        const int last_key = kt * kSpTile + kSpTile - 1;
        tile(kt, sc, last_key >= N || (CAUSAL && last_key > qw));
        wait_vm_n<0>();
        __syncthreads();
    };
    if (n_kt > 0) {
        issue(0, 0);
        wait_vm_n<0>();
        __syncthreads();
        int u = 0;
        for (; u + 1 < n_kt; u += 2) {
            step(u, std::integral_constant<int, 0>{});
            step(u + 1, std::integral_constant<int, 1>{});
        }
        if (u < n_kt) step(u, std::integral_constant<int, 0>{});
    }

    // epilogue: O = O~ / l, L = (m + log2 l) ln 2; a row with nothing kept
    // gets O = 0 and L = -inf
    const float lt = other_half_sum(lsum);
    if (my_q < N) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        uint16_t *orow = O + head + (size_t)my_q * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int ch = 32 * dt + 8 * a + 4 * h;
                *reinterpret_cast<u32x2 *>(orow + ch) =
                    u32x2{pack_bf16x2(oacc[dt][4 * a] * inv, oacc[dt][4 * a + 1] * inv),
                          pack_bf16x2(oacc[dt][4 * a + 2] * inv, oacc[dt][4 * a + 3] * inv)};
            }
        if (LSE && h == 0) LSE[(size_t)bh * N + my_q] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : neg_inf();
    }
}

template <bool CAUSAL, bool DROPOUT>
hipError_t launch_sparse_t(const void *q, const void *k, const void *v, const uint8_t *mask, void *o,
                           float *lse, int BH, int N, float scale, uint32_t thr, float inv_keep,
                           uint64_t seed, hipStream_t stream)
{
    const int n_qb = (N + kSpBlock - 1) / kSpBlock;
    hipLaunchKernelGGL((sparse_fwd_kernel<CAUSAL, DROPOUT>), dim3((unsigned)(n_qb * BH)), dim3(kSpThreads), 0,
                       stream, static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), mask, static_cast<uint16_t *>(o), lse, N, BH, n_qb,
                       scale, thr, inv_keep, (uint32_t)seed, (uint32_t)(seed >> 32));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_block_sparse(const void *q, const void *k, const void *v, const uint8_t *block_mask,
                                   void *o, float *lse, int B, int H, int N, float scale, int causal,
                                   float dropout_p, uint64_t seed, hipStream_t stream)
{
    const int BH = B * H;
    const uint32_t thr = (uint32_t)((double)dropout_p * 4294967296.0);
    const float inv_keep = 1.f / (1.f - dropout_p);
    if (thr == 0) {
        return causal ? launch_sparse_t<true, false>(q, k, v, block_mask, o, lse, BH, N, scale, 0, 1.f, seed, stream)
                      : launch_sparse_t<false, false>(q, k, v, block_mask, o, lse, BH, N, scale, 0, 1.f, seed, stream);
    }
    return causal ? launch_sparse_t<true, true>(q, k, v, block_mask, o, lse, BH, N, scale, thr, inv_keep, seed, stream)
                  : launch_sparse_t<false, true>(q, k, v, block_mask, o, lse, BH, N, scale, thr, inv_keep, seed, stream);
}

}  // namespace fa
