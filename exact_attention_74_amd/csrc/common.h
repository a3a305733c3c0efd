// Shared device helpers for the gfx950 (CDNA4) attention kernels.
//
// MFMA conventions used throughout (wave64):
//   v_mfma_f32_32x32x16_bf16  A: 32 rows x 16 k, B: 16 k x 32 cols, D: 32x32 fp32.
//   v_mfma_f32_32x32x64_f8f6f4 (e4m3 operands): the same with 64 k.
//   Lane l holds row/col (l % 32) of A/B and a contiguous run of k slots
//   selected by the half-wave h = l / 32; A and B use the same (h, slot) -> k
//   assignment, so any consistent placement of a reduction index into
//   (h, slot) on both operands gives the right dot product.
//   Accumulator: lane l, register v holds D[row = 8*(v/4) + 4*h + v%4][col = l % 32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no running max yet": exp2(x - kNoMax) underflows to 0
// and exp2(kNoMax - kNoMax) = 1, so no inf - inf NaN can arise.
constexpr float kNoMax = -1.0e30f;

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// e4m3 x e4m3 -> fp32, 32x32x64.  Format code 0 = fp8 e4m3 for both operands;
// zero scale operands select the unscaled instruction.
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Both half-waves' values of x in every lane: lo = x of lane l % 32, hi = x of
// lane l % 32 + 32.  One v_permlane32_swap (a VALU lane swap, no LDS round
// trip) exchanges row 1 of its first operand with row 0 of its second; both
// start as x.  Written as assembly because the compiler folds the builtin's
// two results into one when both operands are the same value.  The s_nop
// covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  lo = x;
  hi = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
__device__ __forceinline__ float max_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return lo + hi;
}

// Two fp32 -> packed bf16x2 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Four fp32 -> four e4m3 bytes (round to nearest even), byte i = x_i.
// The first convert's "old" operand only supplies the upper word, which the
// second convert overwrites; passing x0's bits (instead of 0) lets it reuse a
// live register rather than materialise a zero.
__device__ __forceinline__ uint32_t pack_fp8x4(float x0, float x1, float x2, float x3) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __builtin_bit_cast(int, x0), false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, p, true);
  return (uint32_t)p;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace exattn
