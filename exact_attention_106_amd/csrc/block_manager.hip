// Paged KV block manager (host), the page copy of its copy-on-write, and a
// device check of block tables against the paged kernels' contract.
//
// PagedAttention ("FlashAttention系列优化", PagedAttention section): a
// sequence's KV cache is cut into fixed-size blocks of tokens; a block table
// maps its logical blocks to physical pages anywhere in the pool, and pages
// are taken on demand as tokens arrive. Sequences share pages by mapping
// logical blocks to the same physical page (a prompt shared by several
// samples); each physical page carries a reference count, and a sequence that
// is about to write into a page it shares first gets a private copy
// (copy-on-write).
//
// The manager's state lives in caller-provided host memory (the library
// allocates nothing): a header, then refcount[num_pages], a stack of free
// pages, len[max_seqs] (-1 = no such sequence) and table[max_seqs][max_blocks].
// Every operation checks its arguments and the free-page supply first and
// changes nothing when it fails.
#include <string.h>

#include "../../include/fa.h"
#include "fa_device.h"

namespace {

constexpr int32_t kMagic = 0x424d4146;

struct Header {
    int32_t magic, num_pages, max_seqs, max_blocks, page_size, free_top;
};

struct View {
    Header *h;
    int32_t *ref, *free_stack, *len, *table;
};

size_t state_bytes(int num_pages, int max_seqs, int max_blocks)
{
    return sizeof(Header) +
           sizeof(int32_t) * (2 * (size_t)num_pages + (size_t)max_seqs + (size_t)max_seqs * max_blocks);
}

View view_of(void *state)
{
    View v;
    v.h = static_cast<Header *>(state);
    v.ref = reinterpret_cast<int32_t *>(v.h + 1);
    v.free_stack = v.ref + v.h->num_pages;
    v.len = v.free_stack + v.h->num_pages;
    v.table = v.len + v.h->max_seqs;
    return v;
}

bool valid(const void *state) { return state && static_cast<const Header *>(state)->magic == kMagic; }

int blocks_for(const Header *h, int tokens) { return (tokens + h->page_size - 1) / h->page_size; }

int32_t pop_page(View &v) { return v.free_stack[--v.h->free_top]; }

void release(View &v, int32_t page)
{
    if (--v.ref[page] == 0) v.free_stack[v.h->free_top++] = page;
}

// one page (all heads, page_size tokens, d channels, bf16) of K and of V:
// 16-byte pieces, grid-stride
__global__ __launch_bounds__(256) void copy_pages_kernel(uint8_t *__restrict__ kc, uint8_t *__restrict__ vc,
                                                         const int32_t *__restrict__ src,
                                                         const int32_t *__restrict__ dst, size_t page_bytes)
{
    const size_t s = (size_t)src[blockIdx.y] * page_bytes, t = (size_t)dst[blockIdx.y] * page_bytes;
    for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 16; i < page_bytes; i += (size_t)gridDim.x * 256 * 16) {
        *reinterpret_cast<fa::u32x4 *>(kc + t + i) = *reinterpret_cast<const fa::u32x4 *>(kc + s + i);
        *reinterpret_cast<fa::u32x4 *>(vc + t + i) = *reinterpret_cast<const fa::u32x4 *>(vc + s + i);
    }
}

// result = {0, -1} before the check. A fill kernel rather than a memset, so
// that the two launches of a check may be recorded into a HIP graph.
__global__ void check_tables_init(int32_t *__restrict__ result)
{
    if (threadIdx.x == 0) {
        result[0] = 0;
        result[1] = -1;
    }
}

// One wave per sequence: ctx_lens[s] must lie in [0, max_blocks * page_size]
// and the first ceil(ctx_lens[s] / page_size) entries of its block-table row
// in [0, num_pages). A sequence that breaks either adds 1 to result[0] and
// lowers result[1] to its index (unsigned minimum, so -1 = 0xffffffff stands
// for "none yet"). Entries past a sequence's used blocks are not read.
__global__ __launch_bounds__(256) void check_tables_kernel(const int32_t *__restrict__ bt,
                                                           const int32_t *__restrict__ ctx, int num_seqs,
                                                           int max_blocks, int page_size, int num_pages,
                                                           int32_t *__restrict__ result)
{
    const int lane = threadIdx.x & 63;
    for (long long s = blockIdx.x * 4ll + (threadIdx.x >> 6); s < num_seqs; s += gridDim.x * 4ll) {
        const long long len = ctx[s];
        bool bad = len < 0 || len > (long long)max_blocks * page_size;
        if (!bad) {
            const int used = (int)((len + page_size - 1) / page_size);
            const int32_t *row = bt + (size_t)s * max_blocks;
            bool lane_bad = false;
            for (int e = lane; e < used; e += 64) {
                const int32_t p = row[e];
                lane_bad |= p < 0 || p >= num_pages;
            }
            bad = __any(lane_bad);
        }
        if (bad && lane == 0) {
            atomicAdd(result, 1);
            atomicMin(reinterpret_cast<unsigned *>(result + 1), (unsigned)s);
        }
    }
}

}  // namespace

extern "C" {

size_t fa_bm_state_bytes(int num_pages, int max_seqs, int max_blocks_per_seq)
{
    if (num_pages <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0) return 0;
    return state_bytes(num_pages, max_seqs, max_blocks_per_seq);
}

fa_status fa_bm_init(void *state, size_t bytes, int num_pages, int max_seqs, int max_blocks_per_seq,
                     int page_size)
{
    if (!state) return FA_ERR_NULL_PTR;
    if (num_pages <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0 || page_size <= 0) return FA_ERR_BAD_SHAPE;
    if (bytes < state_bytes(num_pages, max_seqs, max_blocks_per_seq)) return FA_ERR_WORKSPACE;
    Header *h = static_cast<Header *>(state);
    *h = Header{kMagic, num_pages, max_seqs, max_blocks_per_seq, page_size, num_pages};
    View v = view_of(state);
    memset(v.ref, 0, sizeof(int32_t) * num_pages);
    // pages are handed out from the top of the stack: 0, 1, 2, ... first
    for (int p = 0; p < num_pages; ++p) v.free_stack[p] = num_pages - 1 - p;
    for (int s = 0; s < max_seqs; ++s) v.len[s] = -1;
    for (size_t i = 0; i < (size_t)max_seqs * max_blocks_per_seq; ++i) v.table[i] = -1;
    return FA_OK;
}

fa_status fa_bm_add_seq(void *state, int seq, int num_tokens)
{
    if (!valid(state)) return FA_ERR_STATE;
    View v = view_of(state);
    if (seq < 0 || seq >= v.h->max_seqs || num_tokens < 0) return FA_ERR_BAD_SHAPE;
    if (v.len[seq] >= 0) return FA_ERR_STATE;
    const int nb = blocks_for(v.h, num_tokens);
    if (nb > v.h->max_blocks) return FA_ERR_BAD_SHAPE;
    if (nb > v.h->free_top) return FA_ERR_NO_PAGES;
    int32_t *row = v.table + (size_t)seq * v.h->max_blocks;
    for (int b = 0; b < nb; ++b) {
        row[b] = pop_page(v);
        v.ref[row[b]] = 1;
    }
    v.len[seq] = num_tokens;
    return FA_OK;
}

fa_status fa_bm_fork(void *state, int parent, int child)
{
    if (!valid(state)) return FA_ERR_STATE;
    View v = view_of(state);
    if (parent < 0 || parent >= v.h->max_seqs || child < 0 || child >= v.h->max_seqs) return FA_ERR_BAD_SHAPE;
    if (v.len[parent] < 0 || v.len[child] >= 0) return FA_ERR_STATE;
    const int nb = blocks_for(v.h, v.len[parent]);
    const int32_t *prow = v.table + (size_t)parent * v.h->max_blocks;
    int32_t *crow = v.table + (size_t)child * v.h->max_blocks;
    for (int b = 0; b < nb; ++b) {
        crow[b] = prow[b];
        ++v.ref[prow[b]];
    }
    v.len[child] = v.len[parent];
    return FA_OK;
}

fa_status fa_bm_append_token(void *state, int seq, int32_t *cow_src, int32_t *cow_dst)
{
    if (!valid(state)) return FA_ERR_STATE;
    if (!cow_src || !cow_dst) return FA_ERR_NULL_PTR;
    View v = view_of(state);
    if (seq < 0 || seq >= v.h->max_seqs) return FA_ERR_BAD_SHAPE;
    if (v.len[seq] < 0) return FA_ERR_STATE;
    const int pos = v.len[seq], blk = pos / v.h->page_size;
    if (blk >= v.h->max_blocks) return FA_ERR_BAD_SHAPE;
    int32_t *row = v.table + (size_t)seq * v.h->max_blocks;
    *cow_src = *cow_dst = -1;
    if (pos % v.h->page_size == 0) {
        // first token of a new logical block: a fresh page
        if (v.h->free_top == 0) return FA_ERR_NO_PAGES;
        row[blk] = pop_page(v);
        v.ref[row[blk]] = 1;
    } else if (v.ref[row[blk]] > 1) {
        // the token lands in a page other sequences still map: copy on write
        if (v.h->free_top == 0) return FA_ERR_NO_PAGES;
        const int32_t page = pop_page(v);
        v.ref[page] = 1;
        --v.ref[row[blk]];
        *cow_src = row[blk];
        *cow_dst = page;
        row[blk] = page;
    }
    v.len[seq] = pos + 1;
    return FA_OK;
}

fa_status fa_bm_free_seq(void *state, int seq)
{
    if (!valid(state)) return FA_ERR_STATE;
    View v = view_of(state);
    if (seq < 0 || seq >= v.h->max_seqs) return FA_ERR_BAD_SHAPE;
    if (v.len[seq] < 0) return FA_ERR_STATE;
    int32_t *row = v.table + (size_t)seq * v.h->max_blocks;
    const int nb = blocks_for(v.h, v.len[seq]);
    for (int b = 0; b < nb; ++b) {
        release(v, row[b]);
        row[b] = -1;
    }
    v.len[seq] = -1;
    return FA_OK;
}

int fa_bm_num_free_pages(const void *state)
{
    return valid(state) ? static_cast<const Header *>(state)->free_top : -1;
}

int fa_bm_seq_len(const void *state, int seq)
{
    if (!valid(state)) return -1;
    View v = view_of(const_cast<void *>(state));
    return (seq < 0 || seq >= v.h->max_seqs) ? -1 : v.len[seq];
}

int fa_bm_page_refcount(const void *state, int page)
{
    if (!valid(state)) return -1;
    View v = view_of(const_cast<void *>(state));
    return (page < 0 || page >= v.h->num_pages) ? -1 : v.ref[page];
}

fa_status fa_bm_block_table(const void *state, int32_t *block_table, int32_t *ctx_lens)
{
    if (!valid(state)) return FA_ERR_STATE;
    if (!block_table || !ctx_lens) return FA_ERR_NULL_PTR;
    View v = view_of(const_cast<void *>(state));
    memcpy(block_table, v.table, sizeof(int32_t) * (size_t)v.h->max_seqs * v.h->max_blocks);
    for (int s = 0; s < v.h->max_seqs; ++s) ctx_lens[s] = v.len[s] < 0 ? 0 : v.len[s];
    return FA_OK;
}

fa_status fa_copy_pages(void *kcache, void *vcache, const int32_t *src, const int32_t *dst, int n,
                        int num_pages, int H, int d, int page_size, void *stream)
{
    if (!kcache || !vcache || !src || !dst) return FA_ERR_NULL_PTR;
    if (n < 0 || num_pages <= 0 || H <= 0 || d <= 0 || page_size <= 0) return FA_ERR_BAD_SHAPE;
    const size_t page_bytes = (size_t)H * page_size * d * 2;
    if (page_bytes % 16) return FA_ERR_UNSUPPORTED;
    if (n == 0) return FA_OK;
    if (n > 65535) return FA_ERR_BAD_SHAPE;
    const unsigned gx = (unsigned)((page_bytes / 16 + 255) / 256 < 64 ? (page_bytes / 16 + 255) / 256 : 64);
    hipLaunchKernelGGL(copy_pages_kernel, dim3(gx, (unsigned)n), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint8_t *>(kcache), static_cast<uint8_t *>(vcache), src, dst, page_bytes);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_check_paged_tables(const int32_t *block_table, const int32_t *ctx_lens, int num_seqs,
                                int max_blocks_per_seq, int page_size, int num_pages, int32_t *result,
                                void *stream)
{
    if (!block_table || !ctx_lens || !result) return FA_ERR_NULL_PTR;
    if (num_seqs <= 0 || max_blocks_per_seq <= 0 || page_size <= 0 || num_pages <= 0) return FA_ERR_BAD_SHAPE;
    if (((uintptr_t)block_table | (uintptr_t)ctx_lens | (uintptr_t)result) & 3) return FA_ERR_UNSUPPORTED;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(check_tables_init, dim3(1), dim3(64), 0, st, result);
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    const long long wgs = ((long long)num_seqs + 3) / 4;
    hipLaunchKernelGGL(check_tables_kernel, dim3((unsigned)(wgs < 1024 ? wgs : 1024)), dim3(256), 0, st,
                       block_table, ctx_lens, num_seqs, max_blocks_per_seq, page_size, num_pages, result);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
