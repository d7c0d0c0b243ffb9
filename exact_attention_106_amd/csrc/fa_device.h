// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware 2^x (v_exp_f32). Masked scores are -inf and give exactly 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Value of lane l ^ 32 (the other half of the wave), without LDS: permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second, so with both operands x the two results are x's lower and upper
// halves broadcast to both halves.
__device__ __forceinline__ float other_half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float other_half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over [base, base + bytes): loads past the end return zeros,
// which is how tiles that run past N are padded without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): an
// unrolled loop whose index is a compile-time constant in the body
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// XOR swizzle of the 16-byte chunks of an LDS row of CPR chunks (CPR = 16:
// 256-byte rows, CPR = 8: 128-byte rows, CPR = 4: 64-byte rows): chunk c of
// row r is stored at c ^ swz<CPR>(r). With it, 16-byte reads of one chunk
// column by 32 rows and the 8-byte transpose reads (ds_read_b64_tr_b16) of
// 4 x 4 row-chunk blocks are both free of bank conflicts (64-byte rows carry
// only 16-byte column reads: rows r and r + 4 share banks, the swizzle
// moves them to different chunks).
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    static_assert(CPR == 16 || CPR == 8 || CPR == 4, "swizzle for 4, 8 or 16 chunks per row");
    if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (CPR == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return (r >> 2) & 3;
}

// The running reference max of the online softmax only moves when a row's
// tile max exceeds it by more than this (base-2 units); until then the terms
// 2^(t - m) stay below 2^kRescaleSlack, and O~ and l are rescaled only when it
// moves. The final O~/l and m + log2(l) are exact for any common reference
// (floating point is scale-free), so the slack only has to keep the sums far
// from fp32 overflow: l <= N 2^20 and |O~| <= l max|v|. With outliers in Q
// and K (the FP8 workload), a slack of 8 moved the reference in 20 % of the
// 32-query group tiles and 20 in about 3.5 %.
constexpr float kRescaleSlack = 20.0f;

}  // namespace fa
