// MFMA tile helpers shared by the compiler-scheduled gfx950 kernels (the
// backward and the paged prefill): the 32x32x16 bf16 MFMA, 16-byte row reads
// and transpose reads of swizzled row-major LDS tiles.
#pragma once

#include "fa_device.h"

namespace fa {

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

}  // namespace fa
