// Paged (chunked) prefill on gfx950 MFMA, bf16, d = 128, page_size = 16.
//
// The new tokens of a sequence attend to everything in its paged KV cache up
// to their own position (causal), reading K/V through the block table
// (PagedAttention, "FlashAttention系列优化": logical blocks map to physical
// pages anywhere in the pool). The tile loop is the FlashAttention-2 forward of
// the same page (Q row block outer, K/V tiles inner, online softmax with an
// unscaled accumulator and one final 1/l; L = m + ln l).
//
// Query i of sequence s sits at position p = ctx_s - n_new + i and sees cached
// tokens 0..p. Workgroup = 4 waves x 32 queries of one (sequence, head); grid
// ceil(n_new / 128) * S * H, XCD-aware (below), last query blocks first. A tile is
// 64 keys = 4 pages: wave w copies page 4t + w of K and of V straight from the
// cache into LDS (1 KiB pieces, rows swizzled) two tiles ahead of the compute,
// through three LDS stages. Orientation as in the prefill kernel: S^T = K Q^T with the wave's
// queries as columns (one query per lane, so the softmax is in-lane plus one
// exchange between the wave halves), O^T += V^T P^T with V^T read transposed
// from LDS. Slots past ctx_s in the last page may hold anything: their scores
// are masked and their V rows are zeroed in LDS before use.
#include "fa_device.h"
#include "fa_dma.h"
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kPpThreads = 256;
constexpr int kPpBlock = 128;   // queries per workgroup
constexpr int kPpTile = 64;     // keys per tile
constexpr int kPpPage = 16;     // tokens per page

__global__ __launch_bounds__(kPpThreads, 1) void paged_prefill_kernel(
    const uint16_t *__restrict__ Q, const uint8_t *__restrict__ Kc, const uint8_t *__restrict__ Vc,
    const int32_t *__restrict__ BT, const int32_t *__restrict__ CTX, uint16_t *__restrict__ O,
    float *__restrict__ LSE, int SH, int H, int n_new, int n_qb, int max_blocks, float scale)
{
    constexpr int D = 128, ROW = 2 * D, CPR = D / 8, KC = D / 16, DT = D / 32;
    constexpr int TILE = kPpTile * ROW;              // 16 KiB of K or V
    constexpr int PAGE = kPpPage * ROW;              // one (page, head): 4 KiB
    constexpr int STAGES = 3;                         // tile copies run two tiles ahead
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * 2 * TILE];   // [stage][K, V]

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: table reads are scalar
    // Workgroup ids go round-robin over the 8 XCDs. When S*H is a multiple of
    // 8, all query blocks of one (sequence, head) get ids of one residue mod 8
    // and consecutive ids on it, so they run together on one XCD and read
    // the same K/V pages through its L2; each head's blocks run heaviest first.
    int sh, rank;
    if (SH % 8 == 0) {
        const int x = blockIdx.x % 8, j = blockIdx.x / 8;
        rank = j % n_qb;
        sh = 8 * (j / n_qb) + x;
    } else {
        rank = blockIdx.x / SH;
        sh = blockIdx.x % SH;
    }
    const int s = sh / H, hd = sh % H;
    const int qb = n_qb - 1 - rank;
    const int ctx = CTX[s];
    const int base_pos = ctx - n_new;                 // position of query 0
    const int qw = qb * kPpBlock + 32 * w;            // first query of the wave
    const int my_q = qw + l32;
    const int my_p = base_pos + my_q;                 // this lane's position
    const int last_q = min(n_new, qb * kPpBlock + kPpBlock) - 1;
    const int kend = min(ctx, base_pos + last_q + 1); // keys the block needs
    const int n_kt = kend > 0 ? (kend + kPpTile - 1) / kPpTile : 0;
    const int n_pages = (ctx + kPpPage - 1) / kPpPage;
    const int32_t *bt = BT + (size_t)s * max_blocks;
    const size_t head_page = (size_t)hd * PAGE;       // offset of this head inside a page
    const size_t page_stride = (size_t)H * PAGE;

    // Q^T of this lane's query as the B operand (queries past n_new read zeros)
    const auto rq = make_rsrc(Q + (size_t)sh * n_new * D, (uint32_t)n_new * ROW);
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

    // page 4t + w of K and V: four 1 KiB pieces each; lane l of piece i
    // carries tile row 16 w + 4 i + l / 16 (its row within the page is
    // 4 i + l / 16), LDS chunk l % 16 of it, which holds the source chunk
    // (l % 16) ^ swz(row)
    uint32_t src_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * i + (lane >> 4), pc = lane & 15;
        src_off[i] = (uint32_t)((4 * i + (lane >> 4)) * ROW + ((pc ^ swz<CPR>(r)) << 4));
    }
    const uint32_t lds0 = (uint32_t)(size_t)smem;
    // the page of tile t + 2 is looked up in the block table one step before
    // its copy is issued, so the lookup's latency hides behind a tile
    auto page_of = [&](int t) __attribute__((always_inline)) {
        const int blk = t * 4 + w;
        return blk < n_pages ? __builtin_amdgcn_readfirstlane(bt[blk]) : -1;
    };
    // returns the number of copies issued (8, or 0 past the table)
    auto issue = [&](int pid, int st) __attribute__((always_inline)) {
        if (pid >= 0) {
            const size_t off = (size_t)pid * page_stride + head_page;
            const u32x4 rk = sgpr_rsrc(Kc + off, PAGE), rv = sgpr_rsrc(Vc + off, PAGE);
            const uint32_t base = __builtin_amdgcn_readfirstlane(lds0 + st * 2 * TILE + w * PAGE);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dma16(rk, base + i * 1024, src_off[i], 0);
                dma16(rv, base + TILE + i * 1024, src_off[i], 0);
            }
        }
        return pid >= 0;
    };

    f32x16 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
    float m = neg_inf(), lsum = 0.f;
    const float c = scale * kLog2e;

    // One tile: S^T = K Q^T (two 32-key halves), online softmax, O^T += V^T P^T.
    // Reads run LA steps ahead of their MFMAs.
    constexpr int NSD = 2 * KC, NST = NSD + 4 * DT, LA = 4;
    auto tile = [&](int t, auto sc, auto mc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        constexpr bool MASKED = decltype(mc)::value;
        constexpr uint32_t KB = S * 2 * TILE, VB = KB + TILE;
        const uint8_t *lds = smem;
        const int k0 = t * kPpTile;
        u32x4 ra[NST];
        f32x16 sacc[2];
        bf16x8 pf[4];
        auto read = [&](auto fc) __attribute__((always_inline)) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f < NSD) {
                constexpr int kt = f / KC, kc = f % KC;
                ra[f] = lds16(lds + KB + kt * 32 * ROW + rowo[kc]);
            } else if constexpr (f < NST) {
                constexpr int ch = (f - NSD) / DT, dt = (f - NSD) % DT;
                const u32x2 a0 = lds_tr(lds + VB + 16 * ch * ROW + tro[0][dt]);
                const u32x2 a1 = lds_tr(lds + VB + 16 * ch * ROW + tro[1][dt]);
                ra[f] = u32x4{a0[0], a0[1], a1[0], a1[1]};
            }
        };
        // softmax of the tile once S^T is complete (before the P.V steps)
        auto softmax = [&]() __attribute__((always_inline)) {
            if constexpr (MASKED) {
                // element 4a + b of half kt is key k0 + kt*32 + 8a + 4h + b
                const int lim = my_p - (k0 + 4 * h);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (kt * 32 + 8 * (i >> 2) + (i & 3) > lim) sacc[kt][i] = neg_inf();
            }
            float mx = neg_inf();
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
            mx = other_half_max(mx) * c;
            // the reference max moves only when the tile's max exceeds it by
            // more than kRescaleSlack; then O~ and l are rescaled
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
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = exp2_hw(fmaf(sacc[kt][i], c, -mu));
                    rs += p;
                    pf[2 * kt + (i >> 3)][i & 7] = (__bf16)p;
                }
            lsum += rs;
        };
        static_for<LA>([&](auto fc) { read(fc); });
        static_for<NST>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            read(std::integral_constant<int, f + LA>{});
            if constexpr (f < NSD) {
                constexpr int kt = f / KC, kc = f % KC;
                sacc[kt] = mfma(ra[f], qr[kc], kc == 0 ? f32x16{} : sacc[kt]);
                if constexpr (f == NSD - 1) softmax();
            } else {
                constexpr int ch = (f - NSD) / DT, dt = (f - NSD) % DT;
                oacc[dt] = mfma(ra[f], __builtin_bit_cast(u32x4, pf[ch]), oacc[dt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // keys at or past ctx in the tile that holds ctx - 1 (the last page's
    // tail, and pages past the table) get V = 0, so that 0-weight slots
    // cannot bring NaN into O
    auto zero_tail = [&](int t, int st) __attribute__((always_inline)) {
        const int valid = ctx - t * kPpTile;
        if (valid < kPpTile) {
            uint8_t *sv = smem + st * 2 * TILE + TILE;
#pragma unroll
            for (int i = 0; i < kPpTile * CPR / kPpThreads; ++i) {
                const int idx = tid + i * kPpThreads, r = idx / CPR;
                if (r >= valid) *reinterpret_cast<u32x4 *>(sv + r * ROW + (idx % CPR) * 16) = u32x4{};
            }
            __syncthreads();
        }
    };
    // tiles entirely at or below the wave's first position need no mask
    const int wave_p0 = base_pos + qw;
    // Tile t uses LDS stage t mod 3. The step of tile t issues the copies of
    // tile t + 2 (its page looked up during the step before), looks up the
    // page of tile t + 3, and ends once tile t + 1 is in LDS.
    int pid_next = -1;
    auto step = [&](int t, auto sc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        const bool ahead = t + 2 < n_kt && issue(pid_next, (S + 2) % STAGES);
        pid_next = t + 3 < n_kt ? page_of(t + 3) : -1;
        zero_tail(t, S);
        if (t * kPpTile + kPpTile - 1 <= wave_p0) tile(t, sc, std::false_type{});
        else tile(t, sc, std::true_type{});
        if (ahead) wait_vm_n<8>();
        else wait_vm_n<0>();
        __syncthreads();
    };
    if (n_kt > 0) {
        issue(page_of(0), 0);
        bool ahead = 1 < n_kt && issue(page_of(1), 1);
        pid_next = 2 < n_kt ? page_of(2) : -1;
        if (ahead) wait_vm_n<8>();
        else wait_vm_n<0>();
        __syncthreads();
        int t = 0;
        for (; t + 2 < n_kt; t += 3) {
            step(t, std::integral_constant<int, 0>{});
            step(t + 1, std::integral_constant<int, 1>{});
            step(t + 2, std::integral_constant<int, 2>{});
        }
        if (t < n_kt) step(t, std::integral_constant<int, 0>{});
        if (t + 1 < n_kt) step(t + 1, std::integral_constant<int, 1>{});
    }

    // epilogue: O = O~ / l (rows of this lane's query), L = (m + log2 l) ln 2
    const float lt = other_half_sum(lsum);
    if (my_q < n_new) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        uint16_t *orow = O + ((size_t)sh * n_new + my_q) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int ch = 32 * dt + 8 * a + 4 * h;
                *reinterpret_cast<u32x2 *>(orow + ch) =
                    u32x2{pack_bf16x2(oacc[dt][4 * a] * inv, oacc[dt][4 * a + 1] * inv),
                          pack_bf16x2(oacc[dt][4 * a + 2] * inv, oacc[dt][4 * a + 3] * inv)};
            }
        if (LSE && h == 0) LSE[(size_t)sh * n_new + my_q] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : neg_inf();
    }
}

}  // namespace

hipError_t launch_paged_prefill(const void *q, const void *kcache, const void *vcache,
                                const int32_t *block_table, const int32_t *ctx_lens, void *o,
                                float *lse, int num_seqs, int H, int n_new, int max_blocks_per_seq,
                                float scale, hipStream_t stream)
{
    const int n_qb = (n_new + kPpBlock - 1) / kPpBlock;
    hipLaunchKernelGGL(paged_prefill_kernel, dim3((unsigned)(n_qb * num_seqs * H)), dim3(kPpThreads), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint8_t *>(kcache),
                       static_cast<const uint8_t *>(vcache), block_table, ctx_lens,
                       static_cast<uint16_t *>(o), lse, num_seqs * H, H, n_new, n_qb, max_blocks_per_seq, scale);
    return hipGetLastError();
}

}  // namespace fa
