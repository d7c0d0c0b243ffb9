// Fused attention forward on gfx950 MFMA: bf16 (d = 64, 128) and FP8 E4M3
// with per-block scales (d = 128), one kernel template for both.
//
// Work decomposition (FlashAttention-2 parallelisation, 91haoming.cn article,
// "FlashAttention v2 / parallelisation improvements"; "Flash Attention 再学习",
// thread-block and warp sections):
//   * one workgroup per (batch*head, row block of 256 queries), no
//     communication between workgroups; causal grids are issued heaviest row
//     block first;
//   * 8 waves per workgroup (two per SIMD), each owning 32 query rows
//     (split-Q);
//   * K/V tiles of 64 keys stream through a 4-stage LDS ring, three tiles
//     ahead of the compute, by buffer loads that write LDS directly (no
//     register staging). LDS rows are dense; 16-byte chunks are XOR-swizzled by
//     row so that both the MFMA operand reads of K and the transpose reads of
//     V are free of bank conflicts.
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

constexpr int kBR = 256;       // query rows per workgroup
constexpr int kBC = 64;        // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;     // LDS ring depth; tiles are fetched kStages - 1 ahead
constexpr int kScaleBlock = 128;

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D, bool FP8>
struct Layout {
    static constexpr int KROW = FP8 ? D : 2 * D;   // bytes of a K (and HBM V) row
    static constexpr int VROW = 2 * D;             // bytes of a V row in LDS (bf16)
    static constexpr int K_TILE = kBC * KROW;
    static constexpr int V_TILE = kBC * VROW;
    static constexpr int STAGE = K_TILE + V_TILE;
    static constexpr int K_DMA = K_TILE / 1024 / kWaves;   // 1 KiB direct loads per wave per tile
    static constexpr int V_DMA = FP8 ? 0 : V_TILE / 1024 / kWaves;
    static constexpr int DMA = K_DMA + V_DMA;
    static constexpr int V8_LOADS = FP8 ? kBC * D / 16 / kThreads : 0;   // 16-byte E4M3 chunks per thread
};

// XOR swizzle of the 16-byte chunks of LDS row r (cpr chunks per row). With it,
// 16 rows read at one logical chunk land on 16 different chunk positions, and
// 8 consecutive rows read at four consecutive chunks cover every bank twice.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// two E4M3 bytes (selected 16-bit half of w) -> two bf16 in one dword, exact
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
    const f32x2 f = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
}

__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(const_cast<uint8_t *>(p)));
}

// Plain buffer descriptor (base, no stride, num_records = bytes, raw access):
// reads past `bytes` return zeros. Built in SGPRs for use in inline asm.
__device__ __forceinline__ u32x4 sgpr_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// The tile copies below are issued as inline asm and tracked by hand with
// explicit vmcnt waits: the compiler treats its own LDS-DMA intrinsic as a
// store that may alias every later LDS read and would wait for all of them,
// which would serialise the prefetch ring.

// 16-byte global -> LDS copy per lane: lane l writes lds_addr + 16 l
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
// 16- and 8-byte global -> register loads whose completion is also tracked by hand
__device__ __forceinline__ u32x4 vload16(u32x4 rsrc, uint32_t voff, uint32_t soff) {
    u32x4 v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen" : "=v"(v) : "v"(voff), "s"(rsrc), "s"(soff) : "memory");
    return v;
}
__device__ __forceinline__ u32x2 vload8(u32x4 rsrc, uint32_t voff, uint32_t soff) {
    u32x2 v;
    asm volatile("buffer_load_dwordx2 %0, %1, %2, %3 offen" : "=v"(v) : "v"(voff), "s"(rsrc), "s"(soff) : "memory");
    return v;
}

// wait until at most n vector-memory operations of this wave are outstanding
template <int n>
__device__ __forceinline__ void wait_vm_n() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(n) : "memory");
}
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
    case 0: wait_vm_n<0>(); break;
    case 1: wait_vm_n<1>(); break;
    case 2: wait_vm_n<2>(); break;
    case 3: wait_vm_n<3>(); break;
    case 4: wait_vm_n<4>(); break;
    case 5: wait_vm_n<5>(); break;
    case 6: wait_vm_n<6>(); break;
    case 7: wait_vm_n<7>(); break;
    default: wait_vm_n<8>(); break;
    }
}
// workgroup barrier that orders LDS only (no wait on outstanding global loads)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D, bool CAUSAL, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(
    const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K, const uint8_t *__restrict__ V,
    const float *__restrict__ QS, const float *__restrict__ KSc, const float *__restrict__ VSc,
    uint16_t *__restrict__ O, float *__restrict__ LSE, int N, int BH, int n_rb, float c0)
{
    using L = Layout<D, FP8>;
    constexpr int KCPR = L::KROW / 16;
    constexpr int VCPR = L::VROW / 16;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * L::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    const int rank = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    const int rb = CAUSAL ? (n_rb - 1 - rank) : rank;
    const size_t head_off = (size_t)bh * N * L::KROW;
    const uint32_t head_bytes = (uint32_t)N * L::KROW;
    // loads past row N - 1 of this head return zeros
    const u32x4 rq = sgpr_rsrc(Q + head_off, head_bytes);
    const u32x4 rk = sgpr_rsrc(K + head_off, head_bytes);
    const u32x4 rv = sgpr_rsrc(V + head_off, head_bytes);

    const int q0 = rb * kBR;
    const int qw = q0 + w * 32;
    const int my_q = qw + l32;

    float c = c0;
    const float *ks_h = nullptr, *vs_h = nullptr;
    if constexpr (FP8) {
        const int nsb = (N + kScaleBlock - 1) / kScaleBlock;
        // a wave's 32 queries lie in one 128-token scale block (clamped for padding rows)
        c = c0 * QS[(size_t)bh * nsb + min(qw / kScaleBlock, nsb - 1)];
        ks_h = KSc + (size_t)bh * nsb;
        vs_h = VSc + (size_t)bh * nsb;
    }

    // Q fragments: B operand, lane (query l32, channel group hf) of each 16-channel
    // chunk; loaded first, waited for after the prologue copies are issued
    typedef typename std::conditional<FP8, u32x2, u32x4>::type QRaw;
    QRaw qraw[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
        if constexpr (FP8)
            qraw[kc] = vload8(rq, (uint32_t)(my_q * D + 16 * kc + 8 * hf), 0);
        else
            qraw[kc] = vload16(rq, (uint32_t)(my_q * D + 16 * kc + 8 * hf) * 2, 0);
    }

    const int kend = CAUSAL ? min(N, q0 + kBR) : N;
    const int n_tiles = (kend + kBC - 1) / kBC;
    // tiles this wave computes: a prefix 0 .. last (causal waves stop at their diagonal)
    const int last = CAUSAL ? min(n_tiles - 1, (qw + 31) / kBC) : n_tiles - 1;

    // direct-load source offsets (within a tile) of this lane, for its wave's 1 KiB blocks
    uint32_t kdma_off[L::K_DMA];
#pragma unroll
    for (int i = 0; i < L::K_DMA; ++i) {
        const int pos = (w * L::K_DMA + i) * 64 + lane;   // 16-byte chunk position in the tile
        const int r = pos / KCPR, pc = pos % KCPR;
        kdma_off[i] = (uint32_t)(r * L::KROW + ((pc ^ swz<KCPR>(r)) << 4));
    }
    uint32_t vdma_off[L::V_DMA > 0 ? L::V_DMA : 1];
#pragma unroll
    for (int i = 0; i < L::V_DMA; ++i) {
        const int pos = (w * L::V_DMA + i) * 64 + lane;
        const int r = pos / VCPR, pc = pos % VCPR;
        vdma_off[i] = (uint32_t)(r * L::VROW + ((pc ^ swz<VCPR>(r)) << 4));
    }
    const uint32_t lds_base = (uint32_t)(size_t)smem;
    auto issue_tile = [&](int j) {
        const uint32_t sk = lds_base + (j % kStages) * L::STAGE;
        const uint32_t soff = (uint32_t)(j * kBC) * L::KROW;
#pragma unroll
        for (int i = 0; i < L::K_DMA; ++i) dma16(rk, sk + (w * L::K_DMA + i) * 1024, kdma_off[i], soff);
#pragma unroll
        for (int i = 0; i < L::V_DMA; ++i) dma16(rv, sk + L::K_TILE + (w * L::V_DMA + i) * 1024, vdma_off[i], soff);
    };
    // FP8 V: E4M3 chunks through registers, widened to bf16 into the swizzled V tile
    u32x4 v8reg[L::V8_LOADS > 0 ? L::V8_LOADS : 1];
    auto load_v8 = [&](int j) {
        const uint32_t base = (uint32_t)(j * kBC) * L::KROW;
#pragma unroll
        for (int i = 0; i < L::V8_LOADS; ++i) v8reg[i] = vload16(rv, (uint32_t)(tid + i * kThreads) * 16, base);
    };
    // wait for the E4M3 registers (at most n later copies still in flight); the
    // registers pass through the asm so no use can be scheduled before the wait
    auto wait_v8 = [&](int n) {
        wait_vm(n);
#pragma unroll
        for (int i = 0; i < L::V8_LOADS; ++i) asm volatile("" : "+v"(v8reg[i]));
    };
    auto store_v8 = [&](int j) {
        uint8_t *sv = smem + (j % kStages) * L::STAGE + L::K_TILE;
#pragma unroll
        for (int i = 0; i < L::V8_LOADS; ++i) {
            const int idx = tid + i * kThreads;
            const int r = idx / (D / 16), c8 = idx % (D / 16);   // 16 E4M3 channels = bf16 chunks 2c8, 2c8+1
            u32x4 lo, hi;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                lo[2 * e] = e4m3x2_to_bf16x2(v8reg[i][e], false);
                lo[2 * e + 1] = e4m3x2_to_bf16x2(v8reg[i][e], true);
                hi[2 * e] = e4m3x2_to_bf16x2(v8reg[i][2 + e], false);
                hi[2 * e + 1] = e4m3x2_to_bf16x2(v8reg[i][2 + e], true);
            }
            *reinterpret_cast<u32x4 *>(sv + r * L::VROW + (((2 * c8) ^ swz<VCPR>(r)) << 4)) = lo;
            *reinterpret_cast<u32x4 *>(sv + r * L::VROW + (((2 * c8 + 1) ^ swz<VCPR>(r)) << 4)) = hi;
        }
    };

    // operand-read offsets of this lane (row bits below 16 are the lane's, so the
    // swizzle is a per-lane constant for each logical chunk)
    uint32_t koff[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
        if constexpr (FP8)
            koff[kc] = (uint32_t)(l32 * L::KROW + ((kc ^ swz<KCPR>(l32)) << 4) + 8 * hf);
        else
            koff[kc] = (uint32_t)(l32 * L::KROW + (((2 * kc + hf) ^ swz<KCPR>(l32)) << 4));
    }
    // transpose reads: 16-lane group G supplies 4 keys x 16 channels; lane s = 4e + j
    // of the group points at key 4 (G/2) + e (+ 8 rd), channels 16 (G%2) + 4 j .. +3 (+ 32 t)
    const int tr_G = lane >> 4, tr_e = (lane & 15) >> 2, tr_j = lane & 3;
    uint32_t voff[2][D / 32];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
            const int r = 8 * rd + 4 * (tr_G >> 1) + tr_e;
            const int cidx = 4 * t + 2 * (tr_G & 1) + (tr_j >> 1);
            voff[rd][t] = (uint32_t)(r * L::VROW + ((cidx ^ swz<VCPR>(r)) << 4) + 8 * (tr_j & 1));
        }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) oacc[t] = f32x16{};
    float m = neg_inf();  // reference max (base 2), moved only by more than kRescaleSlack
    float lsum = 0.f;     // this lane's share of l (fp32 weights)
    float lsumb = 0.f;    // same, over the bf16-rounded weights the P.V product uses

    // zero the ring once: rows past N of a partial tile then hold zeros or
    // earlier finite values, never uninitialised bits (their weights are 0)
    for (int i = tid; i < kStages * L::STAGE / 16; i += kThreads)
        reinterpret_cast<u32x4 *>(smem)[i] = u32x4{};
    lds_barrier();

    // prologue: tiles 0 .. kStages-2 in flight
    const int pro = min(n_tiles, kStages - 1);
    if constexpr (FP8) load_v8(0);
    for (int jj = 0; jj < pro; ++jj) issue_tile(jj);
    // Q (issued before everything else) has landed once at most the copies and
    // E4M3 loads issued after it are outstanding
    wait_vm(pro * L::DMA + (FP8 ? L::V8_LOADS : 0));
    typedef typename std::conditional<FP8, long, bf16x8>::type QFrag;
    QFrag qf[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
        asm volatile("" : "+v"(qraw[kc]));
        qf[kc] = __builtin_bit_cast(QFrag, qraw[kc]);
    }
    if constexpr (FP8) {
        wait_v8((pro - 1) * L::DMA);   // the E4M3 registers and tile 0 (issued before tiles 1..)
        store_v8(0);
    } else {
        wait_vm((pro - 1) * L::DMA);
    }
    lds_barrier();

    for (int j = 0; j < n_tiles; ++j) {
        const int st = j % kStages;
        const bool next_v8 = FP8 && j + 1 < n_tiles;
        if constexpr (FP8)
            if (next_v8) load_v8(j + 1);
        const bool ahead = j + kStages - 1 < n_tiles;
        if (ahead) issue_tile(j + kStages - 1);
        if (j <= last) {
            const int k0 = j * kBC;
            const uint8_t *sk = smem + st * L::STAGE;
            const uint8_t *sv = sk + L::K_TILE;
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
                        const long a = *reinterpret_cast<const long *>(sk + kt * 32 * L::KROW + koff[kc]);
                        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, qf[kc], sacc[kt], 0, 0, 0);
                    } else {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sk + kt * 32 * L::KROW + koff[kc]);
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
                    const uint8_t *p0 = sv + 16 * ch * L::VROW;
                    const s16x4 lo = lds_read_tr16(p0 + voff[0][t]);
                    const s16x4 hi = lds_read_tr16(p0 + voff[1][t]);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ch], oacc[t], 0, 0, 0);
                }
        }

        // tile j+1 must have landed: the copies of tiles j+2 .. j+kStages-1 may
        // still be in flight (the E4M3 loads of tile j+1 were issued before tile
        // j+kStages-1's copies, so the same count covers them)
        const int in_flight = (min(n_tiles - 1, j + kStages - 1) - min(n_tiles - 1, j + 1)) * L::DMA;
        if constexpr (FP8) {
            if (next_v8) {
                wait_v8(ahead ? L::DMA : 0);
                store_v8(j + 1);
            }
        }
        wait_vm(in_flight);
        lds_barrier();
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
