// Operand fragments of the gfx950 attention kernels: LDS reads, waits and
// MFMAs as inline asm (their order, registers and waits are fixed by the
// kernels), and the E4M3 -> bf16 widening.
#pragma once

#include "fa_device.h"

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// two E4M3 bytes (selected 16-bit half of w) -> two bf16 in one dword; with
// a unit scale the conversion is exact (every E4M3 value is a bf16 value)
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
    const bf16x2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    return __builtin_bit_cast(uint32_t, r);
}

template <int OFF> __device__ __forceinline__ u32x4 ds_b128(uint32_t a) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "n"(OFF));
    return r;
}
template <int OFF> __device__ __forceinline__ u32x2 ds_b64(uint32_t a) {
    u32x2 r;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(a), "n"(OFF));
    return r;
}
template <int OFF> __device__ __forceinline__ u32x2 ds_tr16(uint32_t a) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "n"(OFF));
    return r;
}
template <int N> __device__ __forceinline__ void wait_lgkm() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
// S (VGPR) = / += A (VGPR) x B (AGPR)
__device__ __forceinline__ void mfma_s_first(f32x16 &s, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s(f32x16 &s, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "a"(b));
}
// E4M3 x E4M3 over 64 channels (both operand formats default to E4M3)
__device__ __forceinline__ void mfma_s_first(f32x16 &s, u32x8 a, u32x8 b) {
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s(f32x16 &s, u32x8 a, u32x8 b) {
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(s) : "v"(a), "a"(b));
}
// O (AGPR) += A (VGPR) x B (VGPR)
__device__ __forceinline__ void mfma_o(f32x16 &o, u32x4 a, u32x4 b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}

// (files built with -fno-honor-nans turn the two maxes into one v_max3)
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

}  // namespace fa
