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
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;

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

// Eight fp32 values as bf16 (RNE) in one 16-byte operand.
__device__ __forceinline__ u32x4_t pack_bf16x8(const float* x) {
  return u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }

__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// acc + lo(w) + hi(w) for a packed bf16 pair w (v_dot2c_f32_bf16 against a
// pair of ones: the bf16 values are exact in fp32, so this sums exactly the
// rounded weights that enter a matrix-core step).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

// Eight fp32 values as a pair of bf16 operands hi + lo, hi = bf16(x) and
// lo = bf16(x - hi): the sum carries about 16 significant bits, so a product
// against an exact bf16 operand split over two matrix-core steps keeps
// near-fp32 accuracy.
__device__ __forceinline__ void split_bf16x8(const float* x, u32x4_t& hi, u32x4_t& lo) {
  hi = pack_bf16x8(x);
  float r[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = x[2 * i] - bf16_lo(hi[i]);
    r[2 * i + 1] = x[2 * i + 1] - bf16_hi(hi[i]);
  }
  lo = pack_bf16x8(r);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_half(float x) { return __shfl_xor(x, 32); }

// max / sum of x over the lane pair (l, l ^ 32), on the VALU (v_permlane32_swap):
// the swap returns {x with the lower half copied up, x with the upper half
// copied down}, so combining the two is symmetric in the pair.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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

// Position of row kk inside a transposed (d-major) LDS tile: bits 2 and 3
// swapped.  Register r of a 32x32 accumulator holds row 8*(r/4) + 4*grp +
// r%4 of its block; after the swap the 8 rows one lane feeds to one operand
// (registers 8t..8t+7) sit at 8 consecutive positions 16t + 8*grp + 0..7, so
// the matching transposed operand is a single 16-byte LDS read.
__device__ __forceinline__ int tr_pos(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// Store a 4-row x 8-column bf16 block (rows r0..r0+3, given as four 16-byte
// row segments) transposed into a d-major LDS tile: column c goes to
// dst[(c0 + c) * stride + tr_pos(r0) .. +3].  r0 must be a multiple of 4.
__device__ __forceinline__ void store_block_transposed(uint16_t* dst, int stride, int c0, int r0,
                                                       const u32x4_t (&rows)[4]) {
  const int pos0 = tr_pos(r0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int w = i >> 1;
    u32x2_t pair;
    if ((i & 1) == 0) {
      pair.x = pack_lo_halves(rows[0][w], rows[1][w]);
      pair.y = pack_lo_halves(rows[2][w], rows[3][w]);
    } else {
      pair.x = pack_hi_halves(rows[0][w], rows[1][w]);
      pair.y = pack_hi_halves(rows[2][w], rows[3][w]);
    }
    *reinterpret_cast<u32x2_t*>(&dst[(c0 + i) * stride + pos0]) = pair;
  }
}

// Ask the scheduler to keep LDS operand reads `lead` reads ahead of the
// matrix-core steps that use them, in a region of `reads` reads that each feed
// `per` consecutive matrix-core steps.  Without it the reads are issued just
// before their use and the LDS latency is exposed on every step.
template <int reads, int per, int lead = 4>
__device__ __forceinline__ void sched_reads_ahead() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  __builtin_amdgcn_sched_group_barrier(kDsRead, lead, 0);
#pragma unroll
  for (int i = 0; i < reads - lead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, per, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, per * lead, 0);
}

// ---------------------------------------------------------------------------
// Buffer unit: global -> LDS copies and range-checked addressing
// ---------------------------------------------------------------------------

// LLVM's raw buffer load into LDS: each lane copies `size` bytes from
// rsrc.base + voffset + soffset + offset to LDS at lds + 16 * lane (lds is
// wave-uniform).  Offsets at or past rsrc.num_records read as zero.
extern "C" __device__ void fattn_llvm_raw_buffer_load_lds(i32x4_t rsrc, lds_u32_t* lds, int size,
                                                          int voffset, int soffset, int offset,
                                                          int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");

// Buffer descriptor for `bytes` bytes at `base` (stride 0, raw addressing).
__device__ __forceinline__ i32x4_t make_buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = (int32_t)(uint32_t)(a & 0xffffffffu);
  r[1] = (int32_t)(uint32_t)((a >> 32) & 0xffffu);
  r[2] = (int32_t)bytes;
  r[3] = 0x00020000;   // gfx9 data format word: raw dword access
  return r;
}

extern "C" __device__ i32x4_t fattn_llvm_raw_buffer_load_v4i32(i32x4_t rsrc, int voffset,
                                                               int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");

// 16 bytes per lane from the buffer at byte `voffset` (zero past num_records).
__device__ __forceinline__ u32x4_t buffer_load_b128(i32x4_t rsrc, int voffset) {
  return __builtin_bit_cast(u32x4_t, fattn_llvm_raw_buffer_load_v4i32(rsrc, voffset, 0, 0));
}

extern "C" __device__ float fattn_llvm_raw_buffer_load_f32(i32x4_t rsrc, int voffset, int soffset,
                                                           int aux)
    __asm("llvm.amdgcn.raw.buffer.load.f32");

// 4 bytes per lane from the buffer at byte `voffset` (zero past num_records).
__device__ __forceinline__ float buffer_load_f32(i32x4_t rsrc, int voffset) {
  return fattn_llvm_raw_buffer_load_f32(rsrc, voffset, 0, 0);
}

// Copy 16 bytes per lane from the buffer at `voffset` into LDS at
// `lds_wave_dst + 16 * lane` (`lds_wave_dst` must be wave-uniform).
__device__ __forceinline__ void buffer_load_lds16(i32x4_t rsrc, void* lds_wave_dst, int voffset) {
  fattn_llvm_raw_buffer_load_lds(rsrc, (lds_u32_t*)lds_wave_dst, 16, voffset, 0, 0, 0);
}

// Wait until this wave's vector-memory operations (including buffer -> LDS
// copies) have completed.
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace fattn
