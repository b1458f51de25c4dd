// Device helpers of the step-by-step walks (moments.hip, ssd_backward.hip):
// state tiles held as 16 x 16 accumulators of v_mfma_f32_16x16x16_bf16 (or the
// fp32 16x16x4 MFMA), 16 rows in four lane groups of 4 and 16 columns across
// the lanes of a group.
#ifndef SSD_STEP_H
#define SSD_STEP_H

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace ssd_step {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Four consecutive rows r0 .. r0 + 3 of column colbase + (lane % 16) of a
// row-major bf16 LDS tile, for every lane: one transposed 8-byte read per lane
// (lane s of a 16-lane group reads 4 elements of row r0 + s / 4 at column
// colbase + 4 (s % 4)). r0 may differ between the four lane groups.
__device__ __forceinline__ s16x4 tr_rows4(const uint16_t* tile, int ld, int r0, int colbase, int lane) {
    const int s = lane & 15;
    const uint16_t* p = tile + (r0 + (s >> 2)) * ld + colbase + 4 * (s & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// Four consecutive elements of one row (8 bytes of bf16), as an operand.
__device__ __forceinline__ s16x4 row4(const uint16_t* p) { return *reinterpret_cast<const s16x4*>(p); }

__device__ __forceinline__ s16x4 pack4_bf16(f32x4 v) {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
    return __builtin_bit_cast(s16x4, __builtin_convertvector(v, bf16x4));
}

// partner lane l ^ 1 (column n ^ 1 of the same rows): DPP quad_perm [1, 0, 3, 2]
__device__ __forceinline__ float swap_pair(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
}

__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma4f(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr float kInv2Pi = 0.15915494309189535f;

}  // namespace ssd_step

#endif  // SSD_STEP_H
