// Paged-KV decode attention, split over KV chunks, then merged (d = 128,
// 16-token pages).
//
// The cache is addressed through a per-sequence block table of fixed-size
// pages (PagedAttention section of "FlashAttention系列优化"): token t of
// sequence s is slot t % 16 of physical page block_table[s][t / 16]; pages
// may be shared between sequences and are only read here.
//
// The split kernel: one workgroup per (KV chunk of 32 pages, head, sequence).
// Each of its 4 waves walks every 4th page of the chunk. A (page, head) block
// of K or V is 16 tokens x 128 channels of bf16 = 4 KiB contiguous; a wave
// reads it with four fully coalesced 1 KiB loads, so lane l holds tokens
// 4i + l/16 (i = 0..3) at channels 8 (l % 16) .. +7. Scores are reduced over
// the 16 lanes of a row group; every lane then runs the online-softmax update
// (running max, unscaled sum, unscaled 8-channel output) over the tokens it
// sees. The four token groups of a wave and then the four waves are combined
// with the rescale identity of the FlashAttention-2 accumulator
// ("FlashAttention系列优化", FlashAttentionV2 equations), and the chunk's
// partial (m, l, O~) goes to the workspace. This kernel is HBM-bound: the only
// traffic that matters is reading each needed page once.
// Within a full chunk each wave keeps the next page's loads in flight while
// it consumes one.
//
// The merge kernel: one workgroup per (head, sequence) combines its chunks'
// partials the same way and writes O (bf16) and L = (m + log2 l) ln 2.
// Slots past the context in the last page may be loaded (they lie in the
// page) but never contribute.
#include "fa_device.h"
#include "fa_launch.h"

#include <mutex>

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kPS = 16;
constexpr int kPPS = kDecodePagesPerSplit;
constexpr int kWaves = 4;
constexpr int kPF = kD + 2;   // floats per partial

struct State {
    float m, l, o[8];
};

// 16 bytes of a K or V page: every (page, head) block is read by exactly one
// workgroup, once, so the loads carry the non-temporal hint (a plain
// streaming-read probe on this GPU reaches 6.1 TB/s with it, 5.65 without)
__device__ __forceinline__ u32x4 stream_load(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ void merge_into(State &a, float m2, float l2, const float *o2) {
    const float mm = fmaxf(a.m, m2);
    const float mu = mm == neg_inf() ? 0.f : mm;
    const float wa = exp2_hw(a.m - mu);
    const float wb = exp2_hw(m2 - mu);
    a.l = a.l * wa + l2 * wb;
#pragma unroll
    for (int e = 0; e < 8; ++e) a.o[e] = a.o[e] * wa + o2[e] * wb;
    a.m = mm;
}

// ---- prefix sharing between sequences (PagedAttention section) ----
// Two sequences whose block tables name the same 32 pages for a full chunk
// read those pages once: one workgroup computes both queries' partials.
// Chunks are grouped into classes of equal page lists with a hash table
// (expected O(1) work per chunk, any number of sequences), and the members of
// a class are paired two by two. Which members end up paired does not change
// any result: a query's partial is computed by the same operations alone or
// in a pair. pair[s][c] = partner sequence, -1 alone, -2 handled by the partner.
//
// every slot of chunk c lies inside sequence s's context
__device__ __forceinline__ bool chunk_full(const int32_t *ctx_lens, int s, int c) {
    return (c + 1) * kPPS * kPS <= ctx_lens[s];
}
// the 32 block-table entries of chunk c of sequence s
__device__ __forceinline__ const int32_t *chunk_entries(const int32_t *block_table, int max_blocks, int s, int c) {
    return block_table + (size_t)s * max_blocks + c * kPPS;
}
// Per chunk: its hash (0: not a full chunk) and pair slot; the hash table and
// the pair count are cleared for this call.
__global__ __launch_bounds__(256) void decode_plan_kernel(const int32_t *__restrict__ block_table,
                                                          const int32_t *__restrict__ ctx_lens,
                                                          uint64_t *__restrict__ hash, int *__restrict__ pair,
                                                          unsigned long long *__restrict__ tab,
                                                          int *__restrict__ waiting, int *__restrict__ n_pairs,
                                                          int S, int max_blocks, int max_splits, int T) {
    const int n_chunks = S * max_splits;
    const int n = n_chunks > T ? n_chunks : T;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
        if (i == 0) *n_pairs = 0;
        if (i < T) {
            tab[i] = 0ull;
            waiting[i] = -1;
        }
        if (i < n_chunks) {
            const int s = i / max_splits, c = i % max_splits;
            uint64_t hv = 0;
            if (chunk_full(ctx_lens, s, c)) {
                const int32_t *e = chunk_entries(block_table, max_blocks, s, c);
                hv = 1469598103934665603ull;   // FNV-1a over the chunk index and its 32 entries
                hv ^= (uint32_t)c;
                hv *= 1099511628211ull;
                for (int k = 0; k < kPPS; ++k) {
                    hv ^= (uint32_t)e[k];
                    hv *= 1099511628211ull;
                }
                hv |= 1;
            }
            hash[i] = hv;
            pair[i] = -1;
        }
    }
}
// Per full chunk i = s * max_splits + c: find its class in the hash table (a
// slot holds the upper 32 bits of the hash and the first member; a member
// whose page list differs from the slot's first member goes on probing), then
// pair with the member parked at the slot, or park there. T is a power of two
// of at least twice the chunk count, so probing ends at a free slot.
__global__ __launch_bounds__(256) void decode_pair_kernel(const int32_t *__restrict__ block_table,
                                                          const uint64_t *__restrict__ hash,
                                                          int *__restrict__ pair,
                                                          unsigned long long *__restrict__ tab,
                                                          int *__restrict__ waiting, int *__restrict__ n_pairs,
                                                          int *__restrict__ pair_list, int S, int max_blocks,
                                                          int max_splits, int T) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= S * max_splits) return;
    const uint64_t hv = hash[i];
    if (hv == 0) return;
    const int s = i / max_splits, c = i % max_splits;
    const int32_t *e = chunk_entries(block_table, max_blocks, s, c);
    const uint32_t key = (uint32_t)(hv >> 32);
    const unsigned long long mine = ((unsigned long long)key << 32) | (unsigned long long)(uint32_t)(i + 1);
    int slot = -1;
    for (int probe = 0, t = (int)(hv & (uint64_t)(T - 1)); probe < T; ++probe, t = (t + 1) & (T - 1)) {
        const unsigned long long old = atomicCAS(&tab[t], 0ull, mine);
        if (old == 0ull) {   // a new class, this chunk its first member
            slot = t;
            break;
        }
        if ((uint32_t)(old >> 32) != key) continue;
        const int first = (int)(uint32_t)old - 1;   // chunk index of the slot's first member
        if (first % max_splits != c) continue;
        const int32_t *f = chunk_entries(block_table, max_blocks, first / max_splits, c);
        bool same = true;
        for (int k = 0; k < kPPS; ++k) same = same && f[k] == e[k];
        if (same) {
            slot = t;
            break;
        }
    }
    if (slot < 0) return;   // not reached (a free slot always exists): the chunk stays alone
    // pair with the parked member or park: every successful exchange ends one
    // member's loop, so the loop ends; the bound only guards against misuse
    int partner = -1;
    for (int it = 0; it < (1 << 20); ++it) {
        const int cur = __hip_atomic_load(&waiting[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (cur < 0) {
            if (atomicCAS(&waiting[slot], -1, i) == -1) break;   // parked; a later member may pair with it
        } else if (atomicCAS(&waiting[slot], cur, -1) == cur) {
            partner = cur;
            break;
        }
    }
    if (partner < 0) return;
    const int lead = min(i, partner), follow = max(i, partner);
    pair[lead] = follow / max_splits;   // the partner's sequence (same chunk index)
    pair[follow] = -2;
    pair_list[atomicAdd(n_pairs, 1)] = lead;
}

// One (chunk, head, sequence) with NQ = 1 query, or a shared chunk with the
// queries of a pair (NQ = 2).
template <int NQ>
__device__ __forceinline__ void split_chunk(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ ctx_lens,
    float *__restrict__ ws, int H, int max_blocks, int max_splits, float c, int split, int h, int s,
    int partner)
{
    const int ctx = ctx_lens[s];
    const int n_pages = (ctx + kPS - 1) / kPS;
    const int p_begin = split * kPPS;
    const int p_end = min(n_pages, p_begin + kPPS);
    const int tid = threadIdx.x;
    const int seq[2] = {s, NQ == 2 ? partner : s};

    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tg = lane >> 4;        // token group: tokens 4i + tg
    const int d0 = 8 * (lane & 15);  // channels d0 .. d0+7

    // query slices, pre-multiplied by scale * log2 e
    float qv[NQ][8];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
        const u32x4 raw = *reinterpret_cast<const u32x4 *>(q + ((size_t)seq[u] * H + h) * kD + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[u][2 * e] = bf16_lo(raw[e]) * c;
            qv[u][2 * e + 1] = bf16_hi(raw[e]) * c;
        }
    }

    State stq[NQ];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
        stq[u].m = neg_inf();
        stq[u].l = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) stq[u].o[e] = 0.f;
    }

    const int32_t *bt = block_table + (size_t)s * max_blocks;
    // K and V of one page for this lane: tokens 4i + tg, channels d0 .. d0+7
    struct Page {
        u32x4 k[4], v[4];
    };
    auto load_page = [&](int pg, Page &pp) {
        const int phys = __builtin_amdgcn_readfirstlane(bt[pg]);
        const size_t base = ((size_t)phys * H + h) * (kPS * kD);
        const int tok0 = pg * kPS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 4 * i + tg;
            const bool valid = tok0 + tok < ctx;
            pp.k[i] = valid ? stream_load(kc + base + tok * kD + d0) : u32x4{};
            pp.v[i] = valid ? stream_load(vc + base + tok * kD + d0) : u32x4{};
        }
    };
    auto load_full = [&](int phys, Page &pp) {
        const size_t base = ((size_t)phys * H + h) * (kPS * kD);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 4 * i + tg;
            pp.k[i] = stream_load(kc + base + tok * kD + d0);
            pp.v[i] = stream_load(vc + base + tok * kD + d0);
        }
    };
    // sum over the 16 lanes of a DPP row (the lanes holding one token)
    auto row_sum = [](float a) {
        a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
        a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
        a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x141, 0xF, 0xF, false)); // row_half_mirror
        a += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), 0x140, 0xF, 0xF, false)); // row_mirror
        return a;
    };
    auto consume = [&](int pg, const Page &pp) {
        const int tok0 = pg * kPS;
        // slots past the context may hold anything (even NaN): their weight
        // is 0 and their V must not reach the sum (a shared chunk is full
        // for both queries)
        u32x4 vv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[i] = tok0 + 4 * i + tg < ctx ? pp.v[i] : u32x4{};
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            State &st = stq[u];
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float a = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a = fmaf(qv[u][2 * e], bf16_lo(pp.k[i][e]), a);
                    a = fmaf(qv[u][2 * e + 1], bf16_hi(pp.k[i][e]), a);
                }
                a = row_sum(a);
                sc[i] = tok0 + 4 * i + tg < ctx ? a : neg_inf();
            }
            const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            const float m_new = fmaxf(st.m, mx);
            const float mu = m_new == neg_inf() ? 0.f : m_new;
            const float alpha = exp2_hw(st.m - mu);
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = exp2_hw(sc[i] - mu);
            st.l = st.l * alpha + (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float lo = st.o[2 * e] * alpha, hi = st.o[2 * e + 1] * alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo = fmaf(p[i], bf16_lo(vv[i][e]), lo);
                    hi = fmaf(p[i], bf16_hi(vv[i][e]), hi);
                }
                st.o[2 * e] = lo;
                st.o[2 * e + 1] = hi;
            }
            st.m = m_new;
        }
    };
    if (p_end - p_begin == kPPS) {
        // full chunk: this wave's 8 pages are known, so all loads are
        // unconditional and the next page is always in flight while the
        // current one is consumed (slots past the context are read but
        // zeroed in consume)
        constexpr int NP = kPPS / kWaves;
        const int pg0 = p_begin + w;
        // the block-table entries first (scalar loads, off the vector-load queue)
        int phys[NP];
#pragma unroll
        for (int k = 0; k < NP; ++k) phys[k] = bt[pg0 + k * kWaves];
        Page buf[2];
        load_full(phys[0], buf[0]);
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            if (k + 1 < NP) load_full(phys[k + 1], buf[(k + 1) & 1]);
            consume(pg0 + k * kWaves, buf[k & 1]);
        }
    } else if constexpr (NQ == 1) {
        for (int pg = p_begin + w; pg < p_end; pg += kWaves) {
            Page pp;
            load_page(pg, pp);
            consume(pg, pp);
        }
    }

    // combine the 4 token groups of the wave (lanes l, l^16, l^32, l^48 share
    // channels), then the 4 waves through LDS; one query at a time
    __shared__ float red[kWaves][kPF];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
        State &st = stq[u];
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float m2 = __shfl_xor(st.m, off);
            const float l2 = __shfl_xor(st.l, off);
            float o2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(st.o[e], off);
            merge_into(st, m2, l2, o2);
        }
        if (u > 0) __syncthreads();
        if (lane < 16) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red[w][2 + d0 + e] = st.o[e];
            if (lane == 0) {
                red[w][0] = st.m;
                red[w][1] = st.l;
            }
        }
        __syncthreads();
        if (tid < kD) {
            float mm = neg_inf();
#pragma unroll
            for (int k = 0; k < kWaves; ++k) mm = fmaxf(mm, red[k][0]);
            const float mu = mm == neg_inf() ? 0.f : mm;
            float l = 0.f, o = 0.f;
#pragma unroll
            for (int k = 0; k < kWaves; ++k) {
                const float wk = exp2_hw(red[k][0] - mu);
                l += wk * red[k][1];
                o += wk * red[k][2 + tid];
            }
            float *dst = ws + (((size_t)seq[u] * H + h) * max_splits + split) * kPF;
            dst[2 + tid] = o;
            if (tid == 0) {
                dst[0] = mm;
                dst[1] = l;
            }
        }
    }
}

// every (chunk, head, sequence) that no pair handles
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ ctx_lens,
    float *__restrict__ ws, const int *__restrict__ pair, int H, int max_blocks, int max_splits, float c,
    int head_fastest)
{
    // head fastest: the workgroups that run together read the 32 heads' slices
    // of the same pages, which lie next to each other in the cache
    const int split = head_fastest ? blockIdx.y : blockIdx.x;
    const int h = head_fastest ? blockIdx.x : blockIdx.y;
    const int s = blockIdx.z;
    const int n_pages = (ctx_lens[s] + kPS - 1) / kPS;
    if (split * kPPS >= n_pages) return;   // whole workgroup: chunk past the context
    if (pair[(size_t)s * max_splits + split] != -1) return;   // read by a pair
    split_chunk<1>(q, kc, vc, block_table, ctx_lens, ws, H, max_blocks, max_splits, c, split, h, s, s);
}

// The shared chunks: a fixed grid walks the pair list (its length is only
// known on the device); every workgroup leaves when the list is done. A
// kernel of its own, because the two-query path needs about twice the
// registers of the single one and would halve the split kernel's occupancy.
constexpr int kPairGrid = 512;
__global__ __launch_bounds__(256) void decode_pair_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ ctx_lens,
    float *__restrict__ ws, const int *__restrict__ pair, const int *__restrict__ n_pairs,
    const int *__restrict__ pair_list, int H, int max_blocks, int max_splits, float c)
{
    const int n = *n_pairs * H;
    for (int item = blockIdx.x; item < n; item += gridDim.x) {
        const int sc = pair_list[item / H];
        const int h = item % H;
        const int s = sc / max_splits, split = sc % max_splits;
        split_chunk<2>(q, kc, vc, block_table, ctx_lens, ws, H, max_blocks, max_splits, c, split, h, s,
                       pair[sc]);
        __syncthreads();   // the LDS of the wave combine is reused by the next item
    }
}

// Merge: one workgroup per (head, sequence). The chunks' partials are copied
// to LDS with coalesced loads (a batch of up to kMergeBatch chunks at a time,
// all loads of a batch issued together), then thread t < 128 folds channel t
// over the batch into its running (m, l, O~) with the rescale identity.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 64;
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(
    const float *__restrict__ ws, const int32_t *__restrict__ ctx_lens, uint16_t *__restrict__ o,
    float *__restrict__ lse, int H, int max_splits)
{
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int tid = threadIdx.x;
    const int ctx = ctx_lens[s];
    const int n_pages = (ctx + kPS - 1) / kPS;
    const int n_splits = (n_pages + kPPS - 1) / kPPS;
    const float *src = ws + ((size_t)s * H + h) * max_splits * kPF;
    __shared__ float part[kMergeBatch * kPF];
    float m = neg_inf(), l = 0.f, acc = 0.f;
    for (int b0 = 0; b0 < n_splits; b0 += kMergeBatch) {
        const int nb = min(kMergeBatch, n_splits - b0);
        __syncthreads();
        for (int i = tid; i < nb * kPF; i += kMergeThreads) part[i] = src[(size_t)b0 * kPF + i];
        __syncthreads();
        if (tid < kD) {
            float mm = m;
            for (int k = 0; k < nb; ++k) mm = fmaxf(mm, part[k * kPF]);
            const float mu = mm == neg_inf() ? 0.f : mm;
            const float a = exp2_hw(m - mu);
            l *= a;
            acc *= a;
            for (int k = 0; k < nb; ++k) {
                const float wk = exp2_hw(part[k * kPF] - mu);
                l += wk * part[k * kPF + 1];
                acc += wk * part[k * kPF + 2 + tid];
            }
            m = mm;
        }
    }
    if (tid >= kD) return;
    const float out = l > 0.f ? acc / l : 0.f;
    o[((size_t)s * H + h) * kD + tid] = __builtin_bit_cast(uint16_t, (__bf16)out);
    if (lse && tid == 0) lse[(size_t)s * H + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : neg_inf();
}

}  // namespace

hipError_t launch_paged_decode(const void *q, const void *kcache, const void *vcache,
                               const int32_t *block_table, const int32_t *ctx_lens, void *o,
                               float *lse, int num_seqs, int H, int d, int page_size,
                               int max_blocks_per_seq, float scale, float *workspace,
                               hipStream_t stream)
{
    (void)d;
    (void)page_size;
    const int max_splits = decode_max_splits(max_blocks_per_seq);
    const int n_chunks = num_seqs * max_splits;
    const int T = decode_table_slots(num_seqs, max_blocks_per_seq);
    uint8_t *tail = reinterpret_cast<uint8_t *>(workspace) +
                    decode_partials_floats(num_seqs, H, max_blocks_per_seq) * sizeof(float);
    uint64_t *hash = reinterpret_cast<uint64_t *>(tail);
    unsigned long long *tab = reinterpret_cast<unsigned long long *>(tail + (size_t)n_chunks * sizeof(uint64_t));
    int *pair = reinterpret_cast<int *>(tab + T);
    int *pair_list = pair + n_chunks;
    int *waiting = pair_list + n_chunks;
    int *n_pairs = waiting + T;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const uint16_t *kk = static_cast<const uint16_t *>(kcache);
    const uint16_t *vv = static_cast<const uint16_t *>(vcache);
    const float c = scale * kLog2e;
    const int n_init = n_chunks > T ? n_chunks : T;
    const dim3 g0((unsigned)min((n_init + 255) / 256, 4096));
    hipLaunchKernelGGL(decode_plan_kernel, g0, dim3(256), 0, stream, block_table, ctx_lens, hash, pair, tab, waiting,
                       n_pairs, num_seqs, max_blocks_per_seq, max_splits, T);
    const dim3 gp((unsigned)((n_chunks + 255) / 256));
    hipLaunchKernelGGL(decode_pair_kernel, gp, dim3(256), 0, stream, block_table, hash, pair, tab, waiting, n_pairs,
                       pair_list, num_seqs, max_blocks_per_seq, max_splits, T);
    // heads on x where the chunk count fits the y dimension (65535; x has no
    // such limit), else chunks on x
    const int head_fastest = max_splits <= 65535 ? 1 : 0;
    const dim3 g1 = head_fastest ? dim3((unsigned)H, (unsigned)max_splits, (unsigned)num_seqs)
                                 : dim3((unsigned)max_splits, (unsigned)H, (unsigned)num_seqs);
    hipLaunchKernelGGL(decode_split_kernel, g1, dim3(256), 0, stream, qq, kk, vv, block_table, ctx_lens,
                       workspace, pair, H, max_blocks_per_seq, max_splits, c, head_fastest);
    hipLaunchKernelGGL(decode_pair_split_kernel, dim3(kPairGrid), dim3(256), 0, stream, qq, kk, vv,
                       block_table, ctx_lens, workspace, pair, n_pairs, pair_list, H, max_blocks_per_seq,
                       max_splits, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)H, (unsigned)num_seqs);
    hipLaunchKernelGGL(decode_merge_kernel, g2, dim3(kMergeThreads), 0, stream, workspace, ctx_lens,
                       static_cast<uint16_t *>(o), lse, H, max_splits);
    return hipGetLastError();
}

// ---- the same decode with a static workspace (no allocation anywhere) ----
// For callers that cannot allocate device memory. Each device holds its own
// copy of this buffer from the time the library's code is loaded on it until
// the process ends. Host code never passes `scratch` itself to a kernel (on
// the host that name is only a stand-in): its device address is looked up
// once per device with hipGetSymbolAddress and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device (looked up on its first use)
hipError_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

hipError_t launch_paged_decode_noalloc(const void *q, const void *kcache, const void *vcache,
                                       const int32_t *block_table, const int32_t *ctx_lens, void *o,
                                       float *lse, int num_seqs, int H, int d, int page_size,
                                       int max_blocks_per_seq, float scale, hipStream_t stream)
{
    if (decode_workspace_bytes(num_seqs, H, max_blocks_per_seq) > kNoallocScratchBytes)
        return hipErrorInvalidValue;   // the C ABI rejects such sizes before this
    void *ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    // every word of the workspace the kernels read is written earlier in the
    // same call (the first kernel writes the hashes and pair slots and clears
    // the hash table and the pair count; the partials are written before the
    // merge reads them), so the buffer needs no clearing between calls
    return launch_paged_decode(q, kcache, vcache, block_table, ctx_lens, o, lse, num_seqs, H, d, page_size,
                               max_blocks_per_seq, scale, static_cast<float *>(ws), stream);
}

}  // namespace fa
