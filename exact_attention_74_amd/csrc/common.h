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

#include <type_traits>
#include <utility>

namespace exattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Compile-time loop: f(IC<0>{}), ..., f(IC<N-1>{}) (every index a constant,
// for immediate LDS offsets and per-step wait counts).
template <int V>
using IC = std::integral_constant<int, V>;
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(IC<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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

// Raw buffer descriptor over bytes [off, total) of the region at base (off <
// total).  Loads through it at per-lane offset x read base + off + x when
// off + x < total and return zeros otherwise.  The hardware range check
// applies to the per-lane (VGPR) offset and not to the scalar offset, so a
// tile's start must be carried here, in the descriptor's base and size,
// for rows past the end of the region to read as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t off,
                                                            uint32_t total) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)base + off), (short)0,
                                           total - off, 0x00020000);
}

// Epilogue store of one wave's 32 output rows q0 .. q0 + 31 (BSHD, row pitch
// rs elements, head offset head_off) through the wave's 32-row LDS block ob
// (32 * 2D bytes, free for the wave to overwrite).  The O^T accumulator
// (lane l: row q0 + l % 32, columns 32e + 8g + 4h .. +3, h = l / 32) is
// scaled by inv, rounded to bf16 and written into ob with 16-byte chunk c of
// row r at chunk position c ^ (r % CPR); the rows then leave LDS in 16-byte
// lane reads and global stores, CPR lanes per row, so that every row's 2D
// bytes are written whole by one store instruction rather than in 8-byte
// pieces from 2D / 8 instructions.  Rows at or past N are not stored.
typedef int i32x4_st __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ void store_rows_via_lds(char* ob, const f32x16 (&oacc)[D / 32],
                                                   float inv, __bf16* __restrict__ O,
                                                   int64_t head_off, int64_t rs, int q0, int N,
                                                   int lane) {
  constexpr int RB = 2 * D;   // bytes per row (a multiple of 16 * CPR)
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int li = lane & 31, hh = lane >> 5;
  // Row li, chunk c sits at li * RB + ((c ^ (li % CPR)) * 16): the lane's base
  // address XOR the constant 16 c, so one base register serves every chunk.
  const uint32_t wbase = (uint32_t)(li * RB + (li % CPR) * 16 + 8 * hh);
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      i32x2 pk;
      pk[0] = (int)pack_bf16x2(oacc[e][4 * g + 0] * inv, oacc[e][4 * g + 1] * inv);
      pk[1] = (int)pack_bf16x2(oacc[e][4 * g + 2] * inv, oacc[e][4 * g + 3] * inv);
      *(i32x2*)(ob + (wbase ^ (uint32_t)((4 * e + g) * 16))) = pk;
    }
  // Read-back: lane l takes chunk c = l % CPR of row r = i * RPI + l / CPR.
  // r % CPR = (i * RPI) % CPR + l / CPR with the two terms in disjoint bits,
  // so the chunk position is c ^ (l / CPR) ^ ((i * RPI) % CPR).
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  const int c = lane % CPR, r0 = lane / CPR;
  const uint32_t rbase = (uint32_t)(r0 * RB + ((c ^ r0) * 16));
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const uint32_t x = (uint32_t)(((i * RPI) % CPR) * 16);
    const i32x4_st v = *(const i32x4_st*)(ob + i * RPI * RB + (rbase ^ x));
    const int r = i * RPI + r0;
    if (q0 + r < N) *(i32x4_st*)(O + head_off + (int64_t)(q0 + r) * rs + 8 * c) = v;
  }
}

}  // namespace exattn
