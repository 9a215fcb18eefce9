// qmm_device.h -- device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 bit pattern -> fp32 (exact: bf16 is the top half of a binary32).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Dequantise the eight 4-bit weights of one packed word, w_i = scale * q_i + bias
// (q_i = bits 4i..4i+3), into four bf16 pairs in k order: .x = (w0, w1), ..., .w = (w6, w7).
// The even and odd nibbles are isolated into bytes (one mask; one shift and mask) and
// converted two at a time by the fp8-to-fp32 conversion: a byte b < 16 read as an OCP
// e4m3 number is exactly b * 2^-9 (a subnormal for b < 8, exponent 1 for 8..15). The
// caller passes sc512 = scale * 2^9 (exact), so fma(b * 2^-9, sc512, bias) is the same
// real number as fma(q, scale, bias), rounded once: every weight is bitwise
// RNE_bf16(fma(q, scale, bias)) for |scale| < 2^118. 19 VALU instructions per 8 weights.
__device__ __forceinline__ uint4 dequant8(uint32_t x, float sc512, float bi) {
    const uint32_t lo = x & 0x0F0F0F0Fu;         // q0, q2, q4, q6
    const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;  // q1, q3, q5, q7
    const f32x2 e01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);  // q0, q2 (times 2^-9)
    const f32x2 e23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);   // q4, q6
    const f32x2 o01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);  // q1, q3
    const f32x2 o23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);   // q5, q7
    uint4 r;
    r.x = pack_bf16x2(__builtin_fmaf(e01.x, sc512, bi), __builtin_fmaf(o01.x, sc512, bi));
    r.y = pack_bf16x2(__builtin_fmaf(e01.y, sc512, bi), __builtin_fmaf(o01.y, sc512, bi));
    r.z = pack_bf16x2(__builtin_fmaf(e23.x, sc512, bi), __builtin_fmaf(o23.x, sc512, bi));
    r.w = pack_bf16x2(__builtin_fmaf(e23.y, sc512, bi), __builtin_fmaf(o23.y, sc512, bi));
    return r;
}

// Dequantise eight 8-bit codes, the bytes of x0 then of x1 (lowest byte first), into
// four bf16 pairs in k order: w_i = fma(q_i, scale, bias) in fp32, rounded to bf16.
// Each byte converts with one byte-to-float instruction: 20 VALU instructions per 8 weights.
__device__ __forceinline__ uint4 dequant8_u8(uint32_t x0, uint32_t x1, float sc, float bi) {
    uint4 r;
    r.x = pack_bf16x2(__builtin_fmaf((float)(x0 & 0xFFu), sc, bi), __builtin_fmaf((float)((x0 >> 8) & 0xFFu), sc, bi));
    r.y = pack_bf16x2(__builtin_fmaf((float)((x0 >> 16) & 0xFFu), sc, bi), __builtin_fmaf((float)(x0 >> 24), sc, bi));
    r.z = pack_bf16x2(__builtin_fmaf((float)(x1 & 0xFFu), sc, bi), __builtin_fmaf((float)((x1 >> 8) & 0xFFu), sc, bi));
    r.w = pack_bf16x2(__builtin_fmaf((float)((x1 >> 16) & 0xFFu), sc, bi), __builtin_fmaf((float)(x1 >> 24), sc, bi));
    return r;
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

// D = X . Y^T + D on a 32x32 tile with a 16-deep reduction (v_mfma_f32_32x32x16_bf16,
// the full-rate bf16 MFMA on gfx950). Lane l supplies row (l % 32) of X and of Y, as
// the eight reduction values of slot (l / 32); it receives D[r][l % 32] for
// r = (v % 4) + 4*(l / 32) + 8*(v / 4), v = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 x, bf16x8 y, f32x16 d) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, d, 0, 0, 0);
}

// Butterfly partners 16 and 32 lanes apart on the vector ALU: v_permlane16_swap
// (v_permlane32_swap) of two copies of v leaves lane i holding, between the two copies,
// its own value and that of lane i ^ 16 (i ^ 32), in an order that depends on the lane.
// A sum or maximum of the pair is therefore the butterfly step, the same on both partner
// lanes and bit-identical to v + __shfl_xor(v, 16 or 32), without the round trip through
// LDS that ds_bpermute makes.
__device__ __forceinline__ float xor16_add(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_add(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over the 16 lanes of each row of the wave, left in every lane of the row, by DPP
// moves: partners i ^ 1 and i ^ 2 (quad permutes), then the other quad of the half-row
// (half-row mirror) and the other half of the row (row mirror). Each pairing is its own
// inverse and every lane adds its value and its partner's, so all lanes of a row end
// with the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_mov<0x141>(v);  // row_half_mirror
    v += dpp_mov<0x140>(v);  // row_mirror
    return v;
}

}  // namespace qmm_dev
