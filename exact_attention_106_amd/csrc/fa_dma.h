// Global -> LDS and global -> register copies whose completion the kernels
// track themselves (inline asm, explicit vmcnt waits), for gfx950.
#pragma once

#include "fa_device.h"

namespace fa {

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

// Tile copies are issued as inline asm and tracked by hand with explicit
// vmcnt waits: the compiler treats its own LDS-DMA intrinsic as a store that
// may alias every later LDS read and would wait for all of them, which would
// serialise a prefetch ring.

// 16-byte global -> LDS copy per lane: lane l writes lds_addr + 16 l
// (an SALU write of M0 needs one wait state before an LDS-DMA reads it)
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
// 4-byte global -> LDS copy per lane: lane l writes lds_addr + 4 l
__device__ __forceinline__ void dma4(u32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}
// the same with the LDS address given as an SGPR base plus a constant
template <uint32_t IMM>
__device__ __forceinline__ void dma16c(u32x4 rsrc, uint32_t lds_base, uint32_t voff, uint32_t soff) {
    asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff), "n"(IMM) : "memory");
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

}  // namespace fa
