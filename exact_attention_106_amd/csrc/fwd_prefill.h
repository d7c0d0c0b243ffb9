// Fused attention forward on gfx950 MFMA: bf16 (d = 64, 128) and FP8 E4M3
// with per-block scales (d = 64, 128), one kernel template for both. The
// instantiations live in fwd_prefill_{bf16,bf16_d64,fp8,fp8_d64,paged}.hip.
//
// Work decomposition (FlashAttention-2 parallelisation, 91haoming.cn article,
// "FlashAttention v2 / parallelisation improvements"; "Flash Attention 再学习",
// thread-block and warp sections):
//   * one workgroup per (batch*head, row block of 256 queries), no
//     communication between workgroups; causal grids are issued heaviest row
//     block first;
//   * 4 waves per workgroup, one per SIMD with the whole register file; a
//     wave owns 64 query rows as two groups of 32 (split-Q), and every K or V
//     fragment it reads from LDS feeds the MFMAs of both groups;
//   * K and V tiles of 64 keys stream through 4-stage LDS rings (at most 3
//     K and 4 V tiles live) by buffer loads that write LDS directly, two tiles ahead of the
//     compute. LDS rows are dense; 16-byte chunks are XOR-swizzled by row so
//     that both the MFMA operand reads of K and the transpose reads of V are
//     free of bank conflicts.
//
// MFMA orientation. S^T = K_j Q_i^T (A = 32 keys x 16 channels from LDS,
// B = 32 queries in AGPRs). In the 32x32 accumulator layout a lane holds one
// query and 16 keys, so the row max and sum of the online softmax are in-lane
// reductions plus one exchange between the wave halves (v_permlane32_swap).
// The same values, rounded to bf16, are directly the B operand of
// O^T += V_j^T P^T. V stays row-major in LDS and the A operand V^T is read with
// ds_read_b64_tr_b16, whose lane transpose delivers 4 keys of one channel per
// lane; the keys a lane reads are the ones its P registers hold (keys are a
// summation index, so only the pairing matters).
//
// Online softmax (pseudocode of the FlashAttentionV1 section and the V2
// equations of "FlashAttention系列优化"): running reference max m, unscaled
// sums, unscaled O accumulator, one final division, L = (m + log2 l) ln 2, in
// base 2 (t = s * scale * log2 e). The reference max only moves when a row max
// exceeds it by more than kRescaleSlack, so O is rarely rescaled. The
// softmax of a tile overlaps the MFMAs of its neighbours (P.V of the previous
// tile, Q.K of the next), the ping-pong of the FlashAttentionV3 section of the
// same page done inside one wave.
//
// FP8 (FlashAttention-3 block quantisation, "FlashAttention系列优化",
// FlashAttentionV3 / FP低精度): S^T = K8 Q8^T on v_mfma_f32_32x32x64_f8f6f4
// (E4M3 x E4M3, 64 channels per MFMA, products exact), twice the bf16 MFMA
// rate. A 64-key tile lies in one 128-row scale block, so dequantisation is
// one scalar per tile: the Q and K scales join the softmax multiplier and
// log2 of the V scale joins the exponent's bias (P of the tile comes out
// multiplied by the V scale; l takes its sum back in plain units). V is
// widened E4M3 -> bf16 (exact) on its way into LDS and P.V runs on bf16 MFMA.
// P is not quantised to E4M3: with V outliers of tens, a 3-bit mantissa on P
// would exceed this path's accuracy bound.
//
// Paged mode (chunked prefill, PagedAttention section of the same page: K/V
// live in a cache of 16-token pages named by a block table): the same kernel
// with positions. Query i of sequence s sits at position ctx[s] - N + i and
// sees keys 0 .. its position; a wave's share of a 64-key tile (rows
// 16 w .. 16 w + 15) is exactly page 4 t + w, copied with a descriptor that
// covers the page's valid rows only, so the last page's tail and pages past
// the context arrive as zeros. Page ids are read one step ahead with scalar
// loads. With an arbitrary offset between query and key positions a wave may
// need the mask on two tiles; a query that sees no key gets O = 0, L = -inf.
#pragma once

#include "fa_device.h"
#include "fa_dma.h"
#include "fa_frag.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kBR = 256;       // query rows per workgroup
// bound on a lane's sum of weights 2^(t - m) over its keys of a tile, past
// which the tile is redone against its exact row max (2^kRescaleSlack)
constexpr float kWeightBound = 1048576.f;
static_assert(kRescaleSlack == 20.f, "kWeightBound is 2^kRescaleSlack");
constexpr int kBC = 64;        // keys per tile
constexpr int kScaleBlock = 128;

// ---------------------------------------------------------------------------
// Hand-scheduled kernel: 4 waves x 64 queries (two 32-query groups g0, g1 per
// wave), one wave per SIMD. Every K or V fragment read from LDS feeds the MFMA
// of both groups. A block is a fixed sequence of slots; a slot holds at most
// one MFMA, the LDS reads that run a few MFMAs ahead, an exact lgkmcnt wait,
// and a fixed share of the softmax VALU work:
//
//   block j:  slots [0, NS_PV):  O(g) += V_{j-1}^T P_{j-1}^T(g)   | max of S_j, reference
//                                                                 | move, weights of keys 0..31
//             slots [NS_PV, NS): S_{j+1}(g) = K_{j+1} Q_g^T        | weights of keys 32..63
//
// MFMAs and LDS reads are inline asm so that their order, the registers they
// use (S and P in VGPRs, O and Q in AGPRs) and the waits are fixed here; the
// compiler only places the VALU work inside each slot. Register hazards the
// compiler cannot see are avoided by distance: S written by a block is read
// in the next one, P written in a block is read in the next one, P of the
// previous tile is overwritten only slots after its last MFMA read, and the
// only AGPR writes (rescale) sit between blocks.
//
// K and V have 4 LDS stages each; at most 3 K tiles (K(j+1) read by the
// block, K(j+2), K(j+3) in flight) and 4 V tiles are live. Block j (or the idle step j of a wave
// that is done) issues the copies of V(j+2) and K(j+3); the step before block
// j waits for V(j) and K(j+1). V(j) is read at the end of block j to prefetch
// the first fragments of the next block. fp8 V is staged through registers
// (loaded at the start of block j-1, converted to bf16 and stored before
// block j).
constexpr int kThreads3 = 256;
constexpr int kPageWin = 128;   // paged: tiles per window of page ids held in LDS
constexpr int kRing = 4;    // LDS stages of K and of V


// LDS reads taken by fragment f of a block (0 if it does not exist)
template <int NFV, int NFK, int KR, bool HAS_PV, bool HAS_QK, bool PREF>
constexpr int frag_reads(int f) {
    return f < NFV ? (HAS_PV ? 2 : 0) : f < NFV + NFK ? (HAS_QK ? KR : 0) : (PREF ? 2 : 0);
}
template <int NFV, int NFK, int KR, bool HAS_PV, bool HAS_QK, bool PREF>
constexpr int reads_between(int a, int b) {
    int c = 0;
    for (int f = a; f <= b; ++f) c += frag_reads<NFV, NFK, KR, HAS_PV, HAS_QK, PREF>(f);
    return c;
}
// fragment f is read in slot 2 (f - PRE); fragments below PRE come from the step before
template <int PRE>
constexpr int frag_issue_slot(int f) { return 2 * (f - PRE) < 0 ? 0 : 2 * (f - PRE); }

// softmax element e (0..31) of a block: its fma slot, for keys 0..31 (part 1)
// and keys 32..63 (part 2); e_first(s) is the first element whose slot is >= s
template <int S0, int W>
constexpr int elem_slot(int e) { return S0 + (e * W) / 32; }
template <int S0, int W>
constexpr int elem_first(int s) {
    int e = 0;
    while (e < 32 && elem_slot<S0, W>(e) < s) ++e;
    return e;
}
// softmax element E (0..63; keys 32 (E / 32) + E % 32 of group (E % 32) / 16)
// of a block with NS_PV PV slots and NS_QK QK slots, row max in slots
// [0, MX]: its fma slot (keys 0..31 before the QK MFMAs rewrite their S
// registers at slot NS_PV, keys 32..63 in the first half of the QK slots),
// and its exp slot: an even spread over slots MX + 2 .. NS - 2, never before
// the slot after its fma. Its sum and pack follow one slot after the exp.
template <int MX, int NS_PV, int NS_QK>
constexpr int fma_slot(int E) {
    if (NS_QK < NS_PV)   // fp8: short QK chains, every fma in the PV slots
        return MX + 1 + (E * (NS_PV - MX - 1)) / 64;
    return E < 32 ? elem_slot<MX + 1, NS_PV - MX - 1>(E) : elem_slot<NS_PV, NS_QK / 2>(E - 32);
}
template <int MX, int NS_PV, int NS_QK>
constexpr int exp_slot_raw(int E) {
    // fp8: a QK slot lasts two PV slots; spread in time
    const int WQ = NS_QK < NS_PV ? 2 : 1;
    const int u0 = MX + 2, u1 = NS_PV + (NS_QK - 2) * WQ;
    const int u = u0 + (E * (u1 - u0 + 1)) / 64;
    const int even = u < NS_PV ? u : NS_PV + (u - NS_PV) / WQ;
    const int after = fma_slot<MX, NS_PV, NS_QK>(E) + 1;
    // the pack one slot later must follow the last PV MFMA reading the P
    // registers it overwrites (pf[g][c] feeds slots up to 2 (c DT + DT - 1) + 1)
    const int DT = NS_PV / 8, c = 2 * (E / 32) + ((E % 16) >> 3);
    const int need = 2 * (c * DT + DT - 1) + 1;
    const int m1 = even > after ? even : after;
    return m1 > need ? m1 : need;
}
// the exp slots, made non-decreasing in E (the pack constraint can push an
// element past its successors' even-spread slots), tabulated once per
// schedule so that the per-slot lookups stay cheap to compile
template <int MX, int NS_PV, int NS_QK>
struct ExpSlots {
    struct Table {
        signed char v[64];
    };
    static constexpr Table make() {
        Table t{};
        int r = 0;
        for (int e = 0; e < 64; ++e) {
            const int v = exp_slot_raw<MX, NS_PV, NS_QK>(e);
            r = v > r ? v : r;
            t.v[e] = (signed char)r;
        }
        return t;
    }
    static constexpr Table table = make();
};
template <int MX, int NS_PV, int NS_QK>
constexpr int exp_slot(int E) { return ExpSlots<MX, NS_PV, NS_QK>::table.v[E]; }
template <int MX, int NS_PV, int NS_QK>
constexpr int exp_first(int s) {
    int E = 0;
    while (E < 64 && exp_slot<MX, NS_PV, NS_QK>(E) < s) ++E;
    return E;
}
template <int MX, int NS_PV, int NS_QK>
constexpr int fma_first(int s) {
    int E = 0;
    while (E < 64 && fma_slot<MX, NS_PV, NS_QK>(E) < s) ++E;
    return E;
}
// the schedule's order constraints: slots ascend with E; every fma of keys
// 0..31 precedes slot NS_PV and of keys 32..63 the QK MFMAs of those keys
// (slot NS_PV + NS_QK / 2); every pack lands inside the block and after the
// last PV MFMA that reads the P registers it overwrites (pf[g][c] feeds the
// PV fragments c * DT .. c * DT + DT - 1, slots 2 f and 2 f + 1)
template <int MX, int NS_PV, int NS_QK, int DT>
constexpr bool spread_ok() {
    for (int E = 0; E < 64; ++E) {
        const int f = fma_slot<MX, NS_PV, NS_QK>(E), x = exp_slot<MX, NS_PV, NS_QK>(E);
        if (E > 0 && x < exp_slot<MX, NS_PV, NS_QK>(E - 1)) return false;
        if (f <= MX || x <= f || x + 1 > NS_PV + NS_QK - 1) return false;
        if (E < 32 ? f >= NS_PV : f >= NS_PV + NS_QK / 2) return false;
        const int c = 2 * (E / 32) + ((E % 16) >> 3);
        if (x + 1 <= 2 * (c * DT + DT - 1) + 1) return false;
    }
    return true;
}

template <int D, bool FP8>
struct Layout3 {
    static constexpr int KROW = FP8 ? D : 2 * D;
    static constexpr int VROW = 2 * D;
    static constexpr int K_TILE = kBC * KROW;
    static constexpr int V_TILE = kBC * VROW;
    static constexpr int K_DMA = K_TILE / 1024 / 4;                 // 1 KiB copies per wave
    static constexpr int V_DMA = FP8 ? 0 : V_TILE / 1024 / 4;
    static constexpr int V8_LOADS = FP8 ? kBC * D / 16 / kThreads3 : 0;
    static constexpr int LDS = kRing * (K_TILE + V_TILE);
    static constexpr int KC = FP8 ? D / 64 : D / 16;   // QK k-steps
    static constexpr int KR = FP8 ? 2 : 1;   // LDS reads per K fragment
    static constexpr int DT = D / 32;        // PV output tiles
    static constexpr int NFV = 4 * DT;       // PV fragments (f = ch * DT + t)
    static constexpr int NFK = 2 * KC;       // QK fragments (f = kt * KC + kc)
    static constexpr int NS_PV = 2 * NFV;    // PV slots
    static constexpr int NS_QK = 2 * NFK;    // QK slots
    static constexpr int NS = NS_PV + NS_QK;
    static constexpr int PRE = 4;            // fragments read ahead
    static constexpr int MX = NS_PV / 4;     // slots of the row max
};

// Paged K/V (chunked prefill through a block table, PagedAttention section of
// "FlashAttention系列优化"): K and V are caches [pages, H, 16, D]; the N new
// queries of sequence s sit at positions ctx[s] - N .. ctx[s] - 1 and see
// cached keys 0 .. their position.
struct PagedArgs {
    const int32_t *bt;      // [S, max_blocks] page of each logical block
    const int32_t *ctx;     // [S] context length (cached tokens, new ones included)
    uint64_t page_stride;   // bytes from one page to the next (H * 16 * D * 2)
    int max_blocks;
    int H;
};

template <int D, bool CAUSAL, bool FP8, bool PAGED>
__global__ __launch_bounds__(kThreads3, 1) void fwd_kernel3(
    const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K, const uint8_t *__restrict__ V,
    const float *__restrict__ QS, const float *__restrict__ KSc, const float *__restrict__ VSc,
    uint16_t *__restrict__ O, float *__restrict__ LSE, int N, int BH, int n_rb, float c0, PagedArgs pg)
{
    static_assert(!PAGED || (CAUSAL && !FP8 && D == 128), "paged: causal bf16, d = 128");
    static_assert(!FP8 || D == 128 || D == 64, "fp8: d = 64 or 128");
    using L = Layout3<D, FP8>;
    constexpr int KCPR = L::KROW / 16;
    constexpr int VCPR = L::VROW / 16;
    constexpr int KC = L::KC, DT = L::DT, NFV = L::NFV, NFK = L::NFK;
    constexpr int NS_PV = L::NS_PV, NS_QK = L::NS_QK, NS = L::NS, PRE = L::PRE, MX = L::MX;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[L::LDS];
    [[maybe_unused]] __shared__ int page_win[2][PAGED ? 4 * kPageWin : 1];   // paged: page ids, see fill_pages

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hf = lane >> 5;

    // Workgroup ids go round-robin over the 8 XCDs. Dense: consecutive ids are
    // the heads of one row block, so all blocks of a head share an XCD. Paged
    // (many sequence-heads): when B*H is a multiple of 8, all row blocks of one
    // (sequence, head) get ids of one residue mod 8 and consecutive ids on it,
    // so they run together on one XCD and read the same pages through its L2
    int rank = blockIdx.x / BH, bh = blockIdx.x % BH;
    if constexpr (PAGED) {
        if (BH % 8 == 0) {
            const int jx = blockIdx.x / 8;
            rank = jx % n_rb;
            bh = 8 * (jx / n_rb) + blockIdx.x % 8;
        }
    }
    const int rb = CAUSAL ? (n_rb - 1 - rank) : rank;
    const size_t head_off = (size_t)bh * N * L::KROW;
    const uint32_t head_bytes = (uint32_t)N * L::KROW;
    const u32x4 rq = sgpr_rsrc(Q + head_off, head_bytes);
    const u32x4 rk = sgpr_rsrc(K + head_off, head_bytes);
    const u32x4 rv = sgpr_rsrc(V + head_off, head_bytes);

    const int q0 = rb * kBR;
    const int qw = q0 + w * 64;
    const int my_q[2] = {qw + l32, qw + 32 + l32};
    // keys are positions 0 .. kmax - 1; query i sits at position base_pos + i
    int kmax = N, base_pos = 0, s_seq = 0, hd = 0;
    if constexpr (PAGED) {
        s_seq = bh / pg.H;
        hd = bh % pg.H;
        kmax = pg.ctx[s_seq];
        base_pos = kmax - N;
        if (base_pos + q0 + kBR <= 0 || kmax <= 0) {
            // no query of the block sees a key: O = 0, L = -inf
#pragma unroll
            for (int g = 0; g < 2; ++g)
                if (my_q[g] < N) {
                    uint16_t *orow = O + ((size_t)bh * N + my_q[g]) * D;
#pragma unroll
                    for (int t = 0; t < L::DT; ++t)
#pragma unroll
                        for (int gg = 0; gg < 4; ++gg)
                            *reinterpret_cast<u32x2 *>(orow + t * 32 + 8 * gg + 4 * hf) = u32x2{0u, 0u};
                    if (LSE && hf == 0) LSE[(size_t)bh * N + my_q[g]] = neg_inf();
                }
            return;
        }
    }

    float cg[2] = {c0, c0};
    const float *ks_h = nullptr, *vs_h = nullptr;
    if constexpr (FP8) {
        const int nsb = (N + kScaleBlock - 1) / kScaleBlock;
        const float *qs_h = QS + (size_t)bh * nsb;
        // Q and K scales below 2^-100 (zero included) act as 2^-100, so that
        // the multiplier stays positive and masked -inf scores stay -inf
        cg[0] = c0 * fmaxf(qs_h[min(qw / kScaleBlock, nsb - 1)], 0x1p-100f);
        cg[1] = c0 * fmaxf(qs_h[min((qw + 32) / kScaleBlock, nsb - 1)], 0x1p-100f);
        ks_h = KSc + (size_t)bh * nsb;
        vs_h = VSc + (size_t)bh * nsb;
    }

    // Q fragments of both groups (B operand of S = K Q^T)
    typedef typename std::conditional<FP8, u32x8, u32x4>::type QF;
    QF qa[2][KC];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            if constexpr (FP8) {
                const uint32_t a = (uint32_t)(my_q[g] * D + 64 * kc + 32 * hf);
                qa[g][kc] = __builtin_shufflevector(vload16(rq, a, 0), vload16(rq, a + 16, 0), 0, 1, 2, 3, 4, 5,
                                                    6, 7);
            } else
                qa[g][kc] = vload16(rq, (uint32_t)(my_q[g] * D + 16 * kc + 8 * hf) * 2, 0);
        }

    const int kend = CAUSAL ? min(kmax, base_pos + q0 + kBR) : kmax;
    const int n_tiles = (kend + kBC - 1) / kBC;
    const int pw = base_pos + qw;   // position of the wave's first query
    // last tile of this wave; for causal the diagonal one (qw is a multiple of
    // 64, so both groups end on it)
    const int last = CAUSAL ? min(n_tiles - 1, pw + kBC - 1 < 0 ? 0 : (pw + kBC - 1) / kBC) : n_tiles - 1;
    // tiles below j_mask are fully visible to the wave's 64 queries; the
    // tiles from j_mask to `last` need the mask (one, or two when the queries'
    // positions are not a multiple of 64 apart from the keys')
    const int j_mask = CAUSAL ? max(0, (min(pw, kmax - 1) + 1) / kBC) : min(n_tiles, kmax / kBC);

    // ---- copies (tiles past the end read zeros into a free stage) ----
    uint32_t kdma_off[L::K_DMA];
#pragma unroll
    for (int i = 0; i < L::K_DMA; ++i) {
        const int pos = (w * L::K_DMA + i) * 64 + lane;
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
    // paged: the wave's quarter of tile t (rows 16 w .. 16 w + 15) is page 4 t + w;
    // its descriptor covers the page's valid rows only, so rows past the
    // context (the last page's tail, pages past the table) read as zeros
    [[maybe_unused]] uint32_t kpoff[L::K_DMA], vpoff[L::V_DMA > 0 ? L::V_DMA : 1];
    [[maybe_unused]] const int32_t *bt_s = nullptr;
    [[maybe_unused]] const uint8_t *kpage0 = nullptr, *vpage0 = nullptr;
    if constexpr (PAGED) {
#pragma unroll
        for (int i = 0; i < L::K_DMA; ++i) kpoff[i] = kdma_off[i] - (uint32_t)w * L::K_DMA * 1024;
#pragma unroll
        for (int i = 0; i < L::V_DMA; ++i) vpoff[i] = vdma_off[i] - (uint32_t)w * L::V_DMA * 1024;
        bt_s = pg.bt + (size_t)s_seq * pg.max_blocks;
        kpage0 = K + (size_t)hd * (16 * L::KROW);
        vpage0 = V + (size_t)hd * (16 * L::VROW);
    }
    auto valid_rows = [&](int t) { return min(max(kmax - 16 * (4 * t + w), 0), 16); };
    auto page_rsrc = [&](const uint8_t *page0, int t, int pid) {
        return sgpr_rsrc(page0 + (size_t)pid * pg.page_stride, (uint32_t)valid_rows(t) * L::KROW);
    };
    [[maybe_unused]] u32x4 pk_cur{}, pv_cur{};   // copies of the current step: K(j+3), V(j+2)
    [[maybe_unused]] int p2 = 0, p3 = 0;         // pages of tiles j+2, j+3 for the next step
    // Page ids come from LDS: a double-buffered window of the sequence's table
    // row, kPageWin tiles (4 kPageWin entries, wave w's page of tile t at
    // 4 (t mod kPageWin) + w), window c in buffer c mod 2. The prologue fills
    // windows 0 and 1; the step of tile c kPageWin (c >= 1) fills window c + 1
    // into the buffer of window c - 1, which every wave has left. Entries past
    // the row read 0. (A global load of the entry inside the loop would be
    // followed by a wait for every outstanding vector-memory operation, the
    // ring's copies included.)
    auto fill_pages = [&](int c) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            for (int idx = tid; idx < 4 * kPageWin; idx += kThreads3) {
                const long e = (long)c * 4 * kPageWin + idx;
                page_win[c & 1][idx] = e < pg.max_blocks ? bt_s[e] : 0;
            }
        }
    };
    auto page_of = [&](int t) -> int {
        return valid_rows(t) > 0 ? page_win[(t / kPageWin) & 1][4 * (t % kPageWin) + w] : 0;
    };
    const uint32_t lds_k = (uint32_t)(size_t)smem;
    const uint32_t lds_v = lds_k + kRing * L::K_TILE;
    // this wave's share of a K / V tile in LDS (stage 0)
    const uint32_t wk_base = __builtin_amdgcn_readfirstlane(lds_k + w * L::K_DMA * 1024);
    const uint32_t wv_base = __builtin_amdgcn_readfirstlane(lds_v + w * L::V_DMA * 1024);
    auto issue_k_part = [&](int j, int i) {
        if constexpr (PAGED)
            dma16(page_rsrc(kpage0, j, page_of(j)), wk_base + (uint32_t)(j & (kRing - 1)) * L::K_TILE + i * 1024,
                  kpoff[i], 0u);
        else
            dma16(rk, wk_base + (uint32_t)(j & (kRing - 1)) * L::K_TILE + i * 1024, kdma_off[i],
                  (uint32_t)(j * kBC) * L::KROW);
    };
    // fp8 V: 16-byte chunk idx = tid + 256 i of a tile is row v8_row(idx),
    // chunk v8_chunk(idx) (16 E4M3 values; CH8 = D / 16 chunks per row). The 16 lanes of one LDS write pass
    // then hold 16 consecutive rows at one chunk, which the row swizzle spreads
    // over all banks (a row-major assignment puts 8 lanes of a pass on the even
    // chunks of one row and 8 on those of the next: two-way conflicts)
    constexpr int CH8 = D / 16;
    auto v8_row = [](int idx) { return (idx & 15) + 16 * (idx / (16 * CH8)); };
    auto v8_chunk = [](int idx) { return (idx >> 4) % CH8; };
    auto v8_goff = [&](int i) {
        const int idx = tid + i * kThreads3;
        return (uint32_t)(v8_row(idx) * D + 16 * v8_chunk(idx));
    };
    u32x4 v8reg[L::V8_LOADS > 0 ? L::V8_LOADS : 1];
    auto issue_v_part = [&](int j, int i) {
        const uint32_t soff = (uint32_t)(j * kBC) * L::KROW;
        if constexpr (FP8) {
            v8reg[i] = vload16(rv, v8_goff(i), soff);
        } else if constexpr (PAGED) {
            dma16(page_rsrc(vpage0, j, page_of(j)), wv_base + (uint32_t)(j & (kRing - 1)) * L::V_TILE + i * 1024,
                  vpoff[i], 0u);
        } else {
            dma16(rv, wv_base + (uint32_t)(j & (kRing - 1)) * L::V_TILE + i * 1024, vdma_off[i], soff);
        }
    };
    constexpr int NV_ISSUE = FP8 ? L::V8_LOADS : L::V_DMA;
    constexpr int N_ISSUE = NV_ISSUE + L::K_DMA;
    // the copies of step j: V first (fp8: V(j+1) into registers; bf16: V(j+2)), then K(j+3).
    // PH >= 0: j & 3 == PH is known here, so the LDS stages are constants.
    auto issue_part = [&](int j, auto ic, auto phc) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        constexpr int PH = decltype(phc)::value;
        if constexpr (PAGED) {
            // descriptors of this step's pages, built in the step before the block
            if constexpr (i < NV_ISSUE) {
                if constexpr (PH < 0)
                    dma16(pv_cur, wv_base + (uint32_t)((j + 2) & (kRing - 1)) * L::V_TILE + i * 1024, vpoff[i], 0u);
                else
                    dma16c<((PH + 2) & (kRing - 1)) * L::V_TILE + i * 1024>(pv_cur, wv_base, vpoff[i], 0u);
            } else {
                constexpr int ik = i - NV_ISSUE;
                if constexpr (PH < 0)
                    dma16(pk_cur, wk_base + (uint32_t)((j + 3) & (kRing - 1)) * L::K_TILE + ik * 1024, kpoff[ik], 0u);
                else
                    dma16c<((PH + 3) & (kRing - 1)) * L::K_TILE + ik * 1024>(pk_cur, wk_base, kpoff[ik], 0u);
            }
        } else if constexpr (PH < 0) {
            if constexpr (i < NV_ISSUE) issue_v_part(FP8 ? j + 1 : j + 2, i);
            else issue_k_part(j + 3, i - NV_ISSUE);
        } else if constexpr (i < NV_ISSUE) {
            const uint32_t soff = (uint32_t)((FP8 ? j + 1 : j + 2) * kBC) * L::KROW;
            if constexpr (FP8)
                v8reg[i] = vload16(rv, v8_goff(i), soff);
            else
                dma16c<((PH + 2) & (kRing - 1)) * L::V_TILE + i * 1024>(rv, wv_base, vdma_off[i], soff);
        } else {
            constexpr int ik = i - NV_ISSUE;
            dma16c<((PH + 3) & (kRing - 1)) * L::K_TILE + ik * 1024>(rk, wk_base, kdma_off[ik],
                                                                     (uint32_t)((j + 3) * kBC) * L::KROW);
        }
    };
    // widen the i-th register load of V(j) to bf16 and store it in V(j)'s stage
    auto store_v8_part = [&](int j, int i) __attribute__((always_inline)) {
        uint8_t *sv = smem + kRing * L::K_TILE + (j & (kRing - 1)) * L::V_TILE;
        asm volatile("" : "+v"(v8reg[i]));
        const int idx = tid + i * kThreads3;
        const int r = v8_row(idx), c8 = v8_chunk(idx);
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
    };
    auto store_v8 = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < L::V8_LOADS; ++i) store_v8_part(j, i);
    };

    // ---- operand-read offsets of this lane ----
    // K fragment of a lane: its key row, channels [64 kc + 32 hf, +32) for
    // fp8 (two 16-byte chunks), [16 kc + 8 hf, +8) for bf16; Q is loaded with
    // the same channel assignment, so the pairing in the MFMA is right
    uint32_t koff[KC][L::KR];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int h2 = 0; h2 < L::KR; ++h2) {
            const int c = FP8 ? 4 * kc + 2 * hf + h2 : 2 * kc + hf;
            koff[kc][h2] = (uint32_t)(l32 * L::KROW + ((c ^ swz<KCPR>(l32)) << 4));
        }
    const int tr_G = lane >> 4, tr_e = (lane & 15) >> 2, tr_j = lane & 3;
    uint32_t voff[2][DT];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const int r = 8 * rd + 4 * (tr_G >> 1) + tr_e;
            const int cidx = 4 * t + 2 * (tr_G & 1) + (tr_j >> 1);
            voff[rd][t] = (uint32_t)(r * L::VROW + ((cidx ^ swz<VCPR>(r)) << 4) + 8 * (tr_j & 1));
        }

#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int h2 = 0; h2 < L::KR; ++h2) koff[kc][h2] += lds_k;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
        for (int t = 0; t < DT; ++t) voff[rd][t] += lds_v;

    typedef typename std::conditional<FP8, u32x8, u32x4>::type KF;
    f32x16 oacc[2][DT];
    f32x16 sacc[2][2];          // S^T of the newest tile (VGPR)
    bf16x8 pf[2][4];            // P^T of the tile the next PV consumes
    u32x2 pre_lo[PRE], pre_hi[PRE];   // V fragments read ahead for the next block
    float m[2] = {neg_inf(), neg_inf()};
    float lsum[2] = {0.f, 0.f};
    float alpha[2] = {1.f, 1.f};
    bool moved[2] = {false, false};
    float ctj[2] = {cg[0], cg[1]};   // scale (and log2 e) of the current tile
    float lps = 0.f, ipsj = 1.f;     // log2 and inverse of the V dequant scale of the current tile
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int t = 0; t < DT; ++t) oacc[g][t] = f32x16{};

    // One block. HAS_PV: O += V_{j-1}^T P^T; HAS_QK: S = K_{j+1} Q^T;
    // HAS_SM: softmax of tile j; PREF: read the first V_j fragments for the
    // next PV; ISSUE: the copies of step j. PH = j & 3 when known (the LDS
    // stages then go into the instructions' offset fields), else -1.
    auto block = [&](int j, bool masked, auto has_pv_c, auto has_qk_c, auto has_sm_c, auto pref_c,
                     auto issue_c, auto phc, auto exact_c) __attribute__((always_inline)) {
        constexpr bool HAS_PV = decltype(has_pv_c)::value;
        constexpr bool HAS_QK = decltype(has_qk_c)::value;
        constexpr bool HAS_SM = decltype(has_sm_c)::value;
        constexpr bool PREF = decltype(pref_c)::value;
        constexpr bool ISSUE = decltype(issue_c)::value;
        constexpr int PH = decltype(phc)::value;
        // EXACT: the tile's row max sets the reference (the first tile, which
        // holds key 0 and so a visible key of every query that has one).
        // Otherwise the weights are formed against the current reference and
        // checked afterwards (see the end of the block). FP8 keeps the exact
        // max on every tile: with outliers in Q and K (the FP8 workload) some
        // row of a 64-row wave passed the bound often enough that redoing the
        // wave's tile cost more than the max it saves (measured 29 % slower).
        constexpr bool EXACT = decltype(exact_c)::value || FP8;
        constexpr int MXS = EXACT ? MX : 0;   // slots of the row max
        constexpr int NF = NFV + NFK + PRE;
        constexpr int KIMM = PH < 0 ? 0 : ((PH + 1) & (kRing - 1)) * L::K_TILE;
        constexpr int VIMM = PH < 0 ? 0 : ((PH + kRing - 1) & (kRing - 1)) * L::V_TILE;
        constexpr int NIMM = PH < 0 ? 0 : (PH & (kRing - 1)) * L::V_TILE;
        uint32_t ka[KC][L::KR], va[2][DT], vn[2][DT];
        if constexpr (HAS_QK) {
            const uint32_t kb = PH < 0 ? (uint32_t)((j + 1) & (kRing - 1)) * L::K_TILE : 0u;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                for (int h2 = 0; h2 < L::KR; ++h2) ka[kc][h2] = PH < 0 ? kb + koff[kc][h2] : koff[kc][h2];
        }
        if constexpr (HAS_PV) {
            const uint32_t vb = PH < 0 ? (uint32_t)((j - 1) & (kRing - 1)) * L::V_TILE : 0u;
#pragma unroll
            for (int rd = 0; rd < 2; ++rd)
#pragma unroll
                for (int t = 0; t < DT; ++t) va[rd][t] = PH < 0 ? vb + voff[rd][t] : voff[rd][t];
        }
        if constexpr (PREF) {
            const uint32_t vb = PH < 0 ? (uint32_t)(j & (kRing - 1)) * L::V_TILE : 0u;
#pragma unroll
            for (int rd = 0; rd < 2; ++rd)
#pragma unroll
                for (int t = 0; t < DT; ++t) vn[rd][t] = PH < 0 ? vb + voff[rd][t] : voff[rd][t];
        }
        u32x2 vlo[NFV], vhi[NFV];
        KF kfr[NFK];
        u32x2 nlo[PRE], nhi[PRE];
        auto read = [&](auto fc) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f < NFV) {
                if constexpr (HAS_PV && f >= PRE) {
                    constexpr int ch = f / DT, t = f % DT;
                    vlo[f] = ds_tr16<VIMM + 16 * ch * L::VROW>(va[0][t]);
                    vhi[f] = ds_tr16<VIMM + 16 * ch * L::VROW>(va[1][t]);
                }
            } else if constexpr (f < NFV + NFK) {
                if constexpr (HAS_QK) {
                    constexpr int q = f - NFV, kt = q / KC, kc = q % KC;
                    if constexpr (FP8)
                        kfr[q] = __builtin_shufflevector(ds_b128<KIMM + kt * 32 * L::KROW>(ka[kc][0]),
                                                         ds_b128<KIMM + kt * 32 * L::KROW>(ka[kc][1]), 0, 1, 2,
                                                         3, 4, 5, 6, 7);
                    else kfr[q] = ds_b128<KIMM + kt * 32 * L::KROW>(ka[kc][0]);
                }
            } else {
                if constexpr (PREF) {
                    constexpr int p = f - NFV - NFK, ch = p / DT, t = p % DT;
                    nlo[p] = ds_tr16<NIMM + 16 * ch * L::VROW>(vn[0][t]);
                    nhi[p] = ds_tr16<NIMM + 16 * ch * L::VROW>(vn[1][t]);
                }
            }
        };

        // softmax state of this block
        float mx[2] = {neg_inf(), neg_inf()};
        float mt[2][11];
        float mu[2] = {0.f, 0.f};
        float x[2][2][16];
        float rsum[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
        [[maybe_unused]] const float lsum_prev[2] = {lsum[0], lsum[1]};
        [[maybe_unused]] float rs_tile[2] = {0.f, 0.f};   // a lane's sum of this tile's weights
        [[maybe_unused]] bool over = false;   // a lane's weights of this tile passed the bound
        if constexpr (HAS_SM && !EXACT) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                mu[g] = m[g] == neg_inf() ? 0.f : m[g];
                if constexpr (FP8) mu[g] -= lps;
            }
        }
        // S was written by the MFMAs at the end of the previous block: cover
        // the MFMA-write -> VALU-access distance before the softmax touches it
        // (the fp8 QK MFMA has 16 passes, the bf16 one 8)
        if constexpr (HAS_SM) {
            if constexpr (FP8) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3");
            else asm volatile("s_nop 7\n\ts_nop 7");
        }
        if (HAS_SM && masked) {
            const int k0 = j * kBC;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int lim = (CAUSAL ? min(base_pos + qw + 32 * g + l32, kmax - 1) : kmax - 1) - (k0 + 4 * hf);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (kt * 32 + 8 * (i >> 2) + (i & 3) > lim) sacc[g][kt][i] = neg_inf();
            }
        }

        static_for<NS>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            // 1. LDS reads issued in this slot
            if constexpr (s % 2 == 0 && s / 2 + PRE < NF) read(std::integral_constant<int, s / 2 + PRE>{});
            // 2./3. wait for this slot's fragment, then its MFMA
            constexpr int n = s / 2, g = s % 2;
            constexpr bool mf = s < NS_PV ? HAS_PV : HAS_QK;
            if constexpr (mf) {
                // one wait per two fragments: at the first MFMA of an even
                // fragment n, wait until fragments n and n + 1 are in
                if constexpr (s % 4 == 0 && !(HAS_PV && n + 1 < PRE)) {
                    constexpr int lastf = (n + PRE) < NF - 1 ? (n + PRE) : NF - 1;
                    wait_lgkm<reads_between<NFV, NFK, L::KR, HAS_PV, HAS_QK, PREF>(n + 2, lastf)>();
                }
                if constexpr (s < NS_PV) {
                    constexpr int ch = n / DT, t = n % DT;
                    u32x4 a;
                    if constexpr (n < PRE) a = u32x4{pre_lo[n][0], pre_lo[n][1], pre_hi[n][0], pre_hi[n][1]};
                    else a = u32x4{vlo[n][0], vlo[n][1], vhi[n][0], vhi[n][1]};
                    mfma_o(oacc[g][t], a, __builtin_bit_cast(u32x4, pf[g][ch]));
                } else {
                    constexpr int q = n - NFV, kt = q / KC, kc = q % KC;
                    if constexpr (kc == 0) mfma_s_first(sacc[g][kt], kfr[q], qa[g][kc]);
                    else mfma_s(sacc[g][kt], kfr[q], qa[g][kc]);
                }
            }
            // 4. softmax work of this slot
            if constexpr (HAS_SM) {
                // row max of the 32 scores of a lane as a tree of v_max3:
                // 11 ops in slots [0, MX-2), 4 in slot MX-2, 2 in slot MX-1
                if constexpr (EXACT && s < MX - 2) {
                    constexpr int a0 = s * 11 / (MX - 2), a1 = (s + 1) * 11 / (MX - 2);
#pragma unroll
                    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
                        for (int a = a0; a < a1; ++a) {
                            const int v = 3 * a;
                            if (a < 10)
                                mt[gg][a] = max3f(sacc[gg][v >> 4][v & 15], sacc[gg][(v + 1) >> 4][(v + 1) & 15],
                                                  sacc[gg][(v + 2) >> 4][(v + 2) & 15]);
                            else
                                mt[gg][a] = fmaxf(sacc[gg][1][14], sacc[gg][1][15]);
                        }
                }
                if constexpr (EXACT && s == MX - 2) {
#pragma unroll
                    for (int gg = 0; gg < 2; ++gg) {
                        mt[gg][0] = max3f(mt[gg][0], mt[gg][1], mt[gg][2]);
                        mt[gg][3] = max3f(mt[gg][3], mt[gg][4], mt[gg][5]);
                        mt[gg][6] = max3f(mt[gg][6], mt[gg][7], mt[gg][8]);
                        mt[gg][9] = fmaxf(mt[gg][9], mt[gg][10]);
                    }
                }
                if constexpr (EXACT && s == MX - 1) {
#pragma unroll
                    for (int gg = 0; gg < 2; ++gg)
                        mx[gg] = fmaxf(max3f(mt[gg][0], mt[gg][3], mt[gg][6]), mt[gg][9]);
                }
                if constexpr (EXACT && s == MX) {
#pragma unroll
                    for (int gg = 0; gg < 2; ++gg) {
                        const float mxc = other_half_max(mx[gg]) * ctj[gg];
                        const bool move = mxc > m[gg] + kRescaleSlack;
                        const float m_new = move ? mxc : m[gg];
                        // a row that has seen no key yet keeps m = -inf, and
                        // 2^(-inf - -inf) would be NaN: alpha is 1 unless m moves
                        alpha[gg] = move ? exp2_hw(m[gg] - m_new) : 1.f;
                        moved[gg] = __builtin_amdgcn_ballot_w64(move) != 0;
                        m[gg] = m_new;
                        mu[gg] = m_new == neg_inf() ? 0.f : m_new;
                        if constexpr (FP8) mu[gg] -= lps;
                        lsum[gg] *= alpha[gg];
                    }
                }
                // fma of keys 0..31 before slot NS_PV (their S registers are
                // rewritten from there on), of keys 32..63 in the first half of
                // the QK slots; the exps, sums and packs of all 64 follow one
                // even spread over the rest of the block
                constexpr int S1 = MXS + 1, W1 = NS_PV - MXS - 1;
                constexpr int S2 = NS_PV, W2 = NS_QK / 2;
                static_assert(spread_ok<MXS, NS_PV, NS_QK, DT>(), "softmax slot schedule");
                if constexpr (NS_QK < NS_PV) {
                    constexpr int F0 = fma_first<MXS, NS_PV, NS_QK>(s), F1 = fma_first<MXS, NS_PV, NS_QK>(s + 1);
#pragma unroll
                    for (int E = F0; E < F1; ++E)
                        x[(E & 31) / 16][E / 32][E % 16] =
                            fmaf(sacc[(E & 31) / 16][E / 32][E % 16], ctj[(E & 31) / 16], -mu[(E & 31) / 16]);
                } else {
#pragma unroll
                    for (int e = elem_first<S1, W1>(s); e < elem_first<S1, W1>(s + 1); ++e)
                        x[e / 16][0][e % 16] = fmaf(sacc[e / 16][0][e % 16], ctj[e / 16], -mu[e / 16]);
#pragma unroll
                    for (int e = elem_first<S2, W2>(s); e < elem_first<S2, W2>(s + 1); ++e)
                        x[e / 16][1][e % 16] = fmaf(sacc[e / 16][1][e % 16], ctj[e / 16], -mu[e / 16]);
                }
                constexpr int X0 = exp_first<MXS, NS_PV, NS_QK>(s - 1), X1 = exp_first<MXS, NS_PV, NS_QK>(s),
                              X2 = exp_first<MXS, NS_PV, NS_QK>(s + 1);
#pragma unroll
                for (int E = X1; E < X2; ++E)
                    x[(E & 31) / 16][E / 32][E % 16] = exp2_hw(x[(E & 31) / 16][E / 32][E % 16]);
#pragma unroll
                for (int E = X0; E < X1; ++E) {
                    const int gg = (E & 31) / 16, kt = E / 32, i = E % 16;
                    rsum[gg][kt] += x[gg][kt][i];
                    if (i & 1) {
                        pf[gg][2 * kt + (i >> 3)][(i & 7) - 1] = (__bf16)x[gg][kt][i - 1];
                        pf[gg][2 * kt + (i >> 3)][i & 7] = (__bf16)x[gg][kt][i];
                    }
                }
                if constexpr (s == NS - 1) {
#pragma unroll
                    for (int gg = 0; gg < 2; ++gg) {
                        const float rs = FP8 ? (rsum[gg][0] + rsum[gg][1]) * ipsj : rsum[gg][0] + rsum[gg][1];
                        lsum[gg] += rs;
                        // every weight of the lane is at most its sum, so a sum
                        // within the bound keeps each 2^(t - m) <= 2^kRescaleSlack
                        // (an overflow to inf fails the test as well)
                        if constexpr (!EXACT) {
                            rs_tile[gg] = rs;
                            over = over || !(rs <= kWeightBound);
                        }
                    }
                }
            }
            // fp8: V(j+1), loaded at the start of this block, is widened and
            // stored into its stage in the first QK slots (that stage held
            // V(j-3), whose last reads every wave finished before the barrier
            // of this step). Only this block's V loads and older copies are
            // outstanding there (its K copies come later), so the wait is
            // for all of them; the next step's barrier publishes the stores.
            if constexpr (FP8 && ISSUE) {
                if constexpr (s == NS_PV) {
                    wait_vm_n<0>();
                    store_v8_part(j + 1, 0);
                }
                if constexpr (L::V8_LOADS > 1 && s == NS_PV + 2) store_v8_part(j + 1, 1);
            }
            // 5. copies of this step: tile copies in the last slots, which
            // carry the least VALU work; fp8 V register loads in the first
            // slots, so that they have the whole block to arrive before the
            // step that stores them (issued late they left only a few slots,
            // and the wait before the next block stalled on memory latency)
            if constexpr (ISSUE) {
                static_for<N_ISSUE>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    constexpr int slot = (FP8 && i < NV_ISSUE) ? 2 * i : NS - 2 * N_ISSUE + 2 * i;
                    if constexpr (slot == s) issue_part(j, ic, phc);
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        // A lane whose weights passed the bound (its row max grew by more than
        // kRescaleSlack over the reference, or the sum overflowed): the wave
        // redoes those rows exactly. S_j is recomputed from K(j), still in its
        // LDS stage (K(j+4) is copied there only after the next barrier), and
        // Q; a redone row's max moves its reference, O~ is rescaled at the next
        // step (moved, alpha) and l restarts from its value before the tile.
        // Rows whose two half-lanes stayed within the bound keep what the fast
        // path computed, so a row's result never depends on other rows' keys.
        if constexpr (HAS_SM && !EXACT) {
            if (__builtin_amdgcn_ballot_w64(over) != 0) {
                wait_lgkm<0>();   // every LDS read of the block, the next block's prefetch included
                if constexpr (PREF) {
#pragma unroll
                    for (int p = 0; p < PRE; ++p) asm volatile("" : "+v"(nlo[p]), "+v"(nhi[p]));
                }
                const uint32_t kb = (uint32_t)(j & (kRing - 1)) * L::K_TILE;
                f32x16 st[2][2];
                static_for<2 * KC>([&](auto qc) {
                    constexpr int q = decltype(qc)::value, kt = q / KC, kc = q % KC;
                    KF kf;
                    if constexpr (FP8) {
                        u32x4 lo8 = ds_b128<kt * 32 * L::KROW>(kb + koff[kc][0]);
                        u32x4 hi8 = ds_b128<kt * 32 * L::KROW>(kb + koff[kc][1]);
                        wait_lgkm<0>();
                        asm volatile("" : "+v"(lo8), "+v"(hi8));
                        kf = __builtin_shufflevector(lo8, hi8, 0, 1, 2, 3, 4, 5, 6, 7);
                    } else {
                        kf = ds_b128<kt * 32 * L::KROW>(kb + koff[kc][0]);
                        wait_lgkm<0>();
                        asm volatile("" : "+v"(kf));
                    }
                    asm volatile("s_nop 1");
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        if constexpr (kc == 0) mfma_s_first(st[g][kt], kf, qa[g][kc]);
                        else mfma_s(st[g][kt], kf, qa[g][kc]);
                    }
                    // the next fragment's LDS read may land in kf's registers
                    // (the compiler takes the asm MFMAs as done with them at
                    // issue): let both MFMAs (the second starts when the first
                    // ends; 16 passes each for fp8, 8 for bf16) read them first
                    if constexpr (FP8)
                        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
                                     "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
                                     "s_nop 7\n\ts_nop 7");
                    else
                        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
                                     "s_nop 7\n\ts_nop 7");
                });
                if constexpr (FP8) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3");
                else asm volatile("s_nop 7\n\ts_nop 7");
                // the compiler takes asm results as ready at once and would hoist
                // their reads above the nops: pin them after the wait
#pragma unroll
                for (int g = 0; g < 2; ++g) asm volatile("" : "+v"(st[g][0]), "+v"(st[g][1]));
                if (masked) {
                    const int k0 = j * kBC;
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        const int lim =
                            (CAUSAL ? min(base_pos + qw + 32 * g + l32, kmax - 1) : kmax - 1) - (k0 + 4 * hf);
#pragma unroll
                        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                            for (int i = 0; i < 16; ++i)
                                if (kt * 32 + 8 * (i >> 2) + (i & 3) > lim) st[g][kt][i] = neg_inf();
                    }
                }
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    // the row is redone iff either half-lane's sum passed the bound
                    // (sums of non-negative weights: inf at worst, never NaN)
                    const bool redo = !(other_half_max(rs_tile[g]) <= kWeightBound);
                    float mxl = neg_inf();
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 16; ++i) mxl = fmaxf(mxl, st[g][kt][i]);
                    const float mxc = other_half_max(mxl) * ctj[g];
                    const bool move = redo && mxc > m[g];
                    const float m_new = move ? mxc : m[g];
                    alpha[g] = move ? exp2_hw(m[g] - m_new) : 1.f;
                    moved[g] = __builtin_amdgcn_ballot_w64(move) != 0;
                    m[g] = m_new;
                    // the redone values replace the fast path's by selection (no
                    // branch: the hand-scheduled code around stays one region)
                    float mug = m_new == neg_inf() ? 0.f : m_new;
                    if constexpr (FP8) mug -= lps;
                    float rs = 0.f;
                    bf16x8 pn[4];
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int i = 0; i < 16; i += 2) {
                            const float p0 = exp2_hw(fmaf(st[g][kt][i], ctj[g], -mug));
                            const float p1 = exp2_hw(fmaf(st[g][kt][i + 1], ctj[g], -mug));
                            rs += p0 + p1;
                            pn[2 * kt + (i >> 3)][i & 7] = (__bf16)p0;
                            pn[2 * kt + (i >> 3)][(i & 7) + 1] = (__bf16)p1;
                        }
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const u32x4 a = __builtin_bit_cast(u32x4, pf[g][c]), b = __builtin_bit_cast(u32x4, pn[c]);
                        u32x4 r;
#pragma unroll
                        for (int e = 0; e < 4; ++e) r[e] = redo ? b[e] : a[e];
                        pf[g][c] = __builtin_bit_cast(bf16x8, r);
                    }
                    lsum[g] = redo ? lsum_prev[g] * alpha[g] + (FP8 ? rs * ipsj : rs) : lsum[g];
                }
            }
        }
        // reads scheduled past the last slot (next-block prefetch of short blocks)
        static_for<NF>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f >= PRE && 2 * (f - PRE) >= NS) read(fc);
        });
        // No LDS read of the block is in flight past its end. The compiler takes
        // an asm result as ready at once; where blocks join (loop edges, the
        // peeled first and last blocks) it may copy such a value or reuse the
        // registers of one it thinks dead, and a read landing late would then
        // be lost or overwrite them. The next step's barrier waits for these
        // reads a few instructions later anyway.
        wait_lgkm<0>();
        if constexpr (PREF) {
#pragma unroll
            for (int p = 0; p < PRE; ++p) {
                asm volatile("" : "+v"(nlo[p]), "+v"(nhi[p]));
                pre_lo[p] = nlo[p];
                pre_hi[p] = nhi[p];
            }
        }
        // fix the block's softmax results here, so that none of its work is
        // sunk into the next block
        if constexpr (HAS_SM) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                asm volatile("" : "+v"(pf[g][0]), "+v"(pf[g][1]), "+v"(pf[g][2]), "+v"(pf[g][3]));
                asm volatile("" : "+v"(lsum[g]), "+v"(m[g]), "+v"(alpha[g]));
            }
        }
    };
    using T = std::true_type;
    using F = std::false_type;

    // O of a group whose reference moved: scale the AGPRs in place (their last
    // MFMA write is a block away; the trailing nops cover the next MFMA read)
    auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
            if (moved[g]) {
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float tmp;
                        asm volatile("v_accvgpr_read_b32 %1, %0\n\t"
                                     "v_mul_f32 %1, %1, %2\n\t"
                                     "v_accvgpr_write_b32 %0, %1"
                                     : "+a"(oacc[g][t][i]), "=&v"(tmp)
                                     : "v"(alpha[g]));
                    }
                moved[g] = false;
                asm volatile("s_nop 4");
            }
    };
    // the step before block j: V(j) and K(j+1) in (fp8: V(0) stored here,
    // later tiles by the block before), barrier
    [[maybe_unused]] float ks_nx = 0.f, vs_nx = 0.f;   // fp8: K and V scales of the next tile
    auto mid = [&](int j) __attribute__((always_inline)) {
        if constexpr (FP8) {
            wait_vm(j == 0 ? 0 : L::K_DMA);
            if (j == 0) store_v8(0);
            const float ksj = fmaxf(ks_nx, 0x1p-100f);
            ctj[0] = cg[0] * ksj;
            ctj[1] = cg[1] * ksj;
            // P of the tile is computed as vs * exp2(t): log2 vs joins the
            // exponent's bias and l gets the sum back in units of exp2(t).
            // Scales below 2^-100 (zero included) act as 2^-100: such a
            // block's V is 0 to far below bf16 resolution.
            lps = __builtin_amdgcn_logf(fmaxf(vs_nx, 0x1p-100f));
            ipsj = exp2_hw(-lps);
            asm volatile("" : "+v"(ctj[0]), "+v"(ctj[1]), "+v"(lps), "+v"(ipsj));
        } else {
            wait_vm(L::V_DMA + L::K_DMA);
        }
        lds_barrier();
        if constexpr (FP8) {
            // the next tile's scales, loaded a step ahead (the barrier above
            // waits on every scalar load, so one issued before it would stall it)
            ks_nx = ks_h[min(j + 1, n_tiles - 1) * kBC / kScaleBlock];
            vs_nx = vs_h[min(j + 1, n_tiles - 1) * kBC / kScaleBlock];
        }
        if constexpr (PAGED) {
            p3 = page_of(j + 3);
            pv_cur = page_rsrc(vpage0, j + 2, p2);
            pk_cur = page_rsrc(kpage0, j + 3, p3);
            p2 = p3;
            if (j >= kPageWin && j % kPageWin == 0) fill_pages(j / kPageWin + 1);
        }
    };

    // ---- prologue ----
    if constexpr (FP8) {
        ks_nx = ks_h[0];
        vs_nx = vs_h[0];
    }
    for (int i = tid; i < L::LDS / 16; i += kThreads3) reinterpret_cast<u32x4 *>(smem)[i] = u32x4{};
    fill_pages(0);
    fill_pages(1);
    lds_barrier();
    if constexpr (FP8) {
#pragma unroll
        for (int jj = 0; jj < 3; ++jj)
#pragma unroll
            for (int i = 0; i < L::K_DMA; ++i) issue_k_part(jj, i);
#pragma unroll
        for (int i = 0; i < L::V8_LOADS; ++i) issue_v_part(0, i);
        wait_vm(2 * L::K_DMA + L::V8_LOADS);     // Q and K(0)
    } else {
        if constexpr (PAGED) p2 = page_of(2);
#pragma unroll
        for (int i = 0; i < L::K_DMA; ++i) issue_k_part(0, i);
#pragma unroll
        for (int i = 0; i < L::V_DMA; ++i) issue_v_part(0, i);
#pragma unroll
        for (int i = 0; i < L::K_DMA; ++i) issue_k_part(1, i);
#pragma unroll
        for (int i = 0; i < L::V_DMA; ++i) issue_v_part(1, i);
#pragma unroll
        for (int i = 0; i < L::K_DMA; ++i) issue_k_part(2, i);
        wait_vm(2 * L::K_DMA + 2 * L::V_DMA);     // Q and K(0)
    }
    // the loads are asm: pin their results after the wait (a copy placed
    // before it would read registers still being filled), then move to AGPRs
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) asm volatile("" : "+v"(qa[g][kc]));
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) asm volatile("" : "+a"(qa[g][kc]));
    asm volatile("s_nop 7");
    lds_barrier();
    using G = std::integral_constant<int, -1>;   // LDS stages from j at run time
    block(-1, false, F{}, T{}, F{}, F{}, F{}, G{}, F{});        // S(0) = K(0) Q^T

    // ---- block 0 ----
    mid(0);
    if (last >= 1) block(0, 0 >= j_mask, F{}, T{}, T{}, T{}, T{}, G{}, T{});
    else block(0, true, F{}, F{}, T{}, T{}, T{}, G{}, T{});
    // ---- blocks 1 .. last-1 ----
    auto step = [&](int j, auto phc, bool masked) __attribute__((always_inline)) {
        rescale();
        mid(j);
        block(j, masked, T{}, T{}, T{}, T{}, T{}, phc, F{});
    };
    int j = 1;
    // blocks below j_open need no mask (dense: only `last` can need one)
    const int j_open = PAGED ? min(last, j_mask) : last;
    for (; j + 3 < j_open; j += 4) {   // unrolled over the 4 LDS stages (j & 3 == 1, 2, 3, 0)
        step(j, std::integral_constant<int, 1>{}, false);
        step(j + 1, std::integral_constant<int, 2>{}, false);
        step(j + 2, std::integral_constant<int, 3>{}, false);
        step(j + 3, std::integral_constant<int, 0>{}, false);
    }
    for (; j < last; ++j) step(j, G{}, PAGED && j >= j_mask);
    // ---- block last ----
    if (last >= 1) {
        rescale();
        mid(last);
        block(last, last >= j_mask, T{}, F{}, T{}, T{}, T{}, G{}, F{});
    }
    // ---- PV(last) with the fragments read ahead by the block before (no
    // step in between, so wait for those reads here) ----
    rescale();
    wait_lgkm<0>();
    block(last + 1, false, T{}, F{}, F{}, F{}, F{}, G{}, F{});
    // causal: the remaining copies are issued for the other waves
    for (int jj = last + 1; jj < n_tiles; ++jj) {
        mid(jj);
        static_for<N_ISSUE>([&](auto ic) { issue_part(jj, ic, G{}); });
        if constexpr (FP8) {   // what the block of this step would store: V(jj+1)
            wait_vm(L::K_DMA);
            store_v8(jj + 1);
        }
    }
    wait_vm(0);
    // fp8: keeping the last register loads of V live up to the wait stops
    // their registers from being reused while in flight
#pragma unroll
    for (int i = 0; i < L::V8_LOADS; ++i) asm volatile("" : "+v"(v8reg[i]));

    asm volatile("s_nop 15\n\ts_nop 15");

    // ---- epilogue: O = O~ / l ; L = (m + log2 l) ln 2 ----
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const float lt = other_half_sum(lsum[g]);
        if (my_q[g] < N) {
            const float inv = lt > 0.f ? 1.f / lt : 0.f;   // a query with no visible key: O = 0
            uint16_t *orow = O + ((size_t)bh * N + my_q[g]) * D;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg) {
                    u32x2 packed;
                    packed[0] = pack_bf16x2(oacc[g][t][4 * gg + 0] * inv, oacc[g][t][4 * gg + 1] * inv);
                    packed[1] = pack_bf16x2(oacc[g][t][4 * gg + 2] * inv, oacc[g][t][4 * gg + 3] * inv);
                    *reinterpret_cast<u32x2 *>(orow + t * 32 + 8 * gg + 4 * hf) = packed;
                }
            if (LSE && hf == 0) LSE[(size_t)bh * N + my_q[g]] = lt > 0.f ? (m[g] + __log2f(lt)) * kLn2 : neg_inf();
        }
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
    hipLaunchKernelGGL((fwd_kernel3<D, CAUSAL, FP8, false>), grid, dim3(kThreads3), 0, stream,
                       static_cast<const uint8_t *>(q), static_cast<const uint8_t *>(k),
                       static_cast<const uint8_t *>(v), qs, ks, vs, static_cast<uint16_t *>(o), lse, N,
                       BH, n_rb, scale * kLog2e, PagedArgs{});
    return hipGetLastError();
}

}  // namespace

// bf16 and FP8 forward with d = 64 (their own translation units, compiled in parallel)
hipError_t launch_fwd_bf16_d64(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                               int N, float scale, int causal, hipStream_t stream);
hipError_t launch_fwd_fp8_d64(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8, const float *qs,
                              const float *ks, const float *vs, void *o, float *lse, int B, int H, int N,
                              float scale, int causal, hipStream_t stream);

}  // namespace fa
