// Shared device helpers for the libfattn kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, one
// wave of 64 lanes; lane = 32 * grp + col):
//   A operand (32 x 16, row-major in the contraction): lane holds row `col`,
//     8 consecutive contraction elements 8*grp .. 8*grp+7 (one 16-byte value).
//   B operand (16 x 32): lane holds column `col`, the same 8 contraction
//     elements 8*grp .. 8*grp+7.
//   D (32 x 32 fp32): lane holds column `col`, register r holds row
//     8*(r/4) + 4*grp + (r%4).
// Any consistent numbering of the contraction index works for A and B, so
// only the D layout is relied upon when a result becomes the next operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma_32x32x16_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair (round to nearest even, hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_half(float x) { return __shfl_xor(x, 32); }

// Byte select: result byte i = byte sel[i] of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low 16-bit halves of two words: {lo16(b) : lo16(a)}.
__device__ __forceinline__ uint32_t pack_lo_halves(uint32_t a, uint32_t b) {
  return byte_perm(b, a, 0x05040100u);
}
// High 16-bit halves of two words: {hi16(b) : hi16(a)}.
__device__ __forceinline__ uint32_t pack_hi_halves(uint32_t a, uint32_t b) {
  return byte_perm(b, a, 0x07060302u);
}

}  // namespace fattn
