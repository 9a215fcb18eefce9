// qmm_device.h -- device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> fp32 (exact: bf16 is the top half of a binary32).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int t) {
    return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
}

// D = X . Y^T + D on a 16x16 tile with a 32-deep reduction (v_mfma_f32_16x16x32_bf16).
// Lane l supplies row (l % 16) of X and row (l % 16) of Y, each as the eight
// reduction values of slot (l / 16); it receives D[4*(l/16) + e][l % 16], e = 0..3.
// The reduction order inside one instruction is the hardware's; any assignment of
// k values to (slot, element) is valid as long as X and Y use the same one.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 x, bf16x8 y, f32x4 d) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, d, 0, 0, 0);
}

}  // namespace qmm_dev
