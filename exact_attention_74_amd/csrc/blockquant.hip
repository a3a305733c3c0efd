// FP8 pre-pass for gfx950: optional incoherent processing (random +-1 diagonal
// times a Hadamard matrix, FlashAttention-3 report sections 2.2 / 3.3) fused
// with block quantisation to OCP e4m3.
//
// HBM-bound: one read of the bf16 tensor and one write of the e4m3 codes.  A
// workgroup owns one 128-row x d block of one (b, h); 4 lanes share a row and
// lane r holds the 8-element chunks r, r+4, ..., so each load instruction of
// a row's lanes covers 64 contiguous bytes.  The fast Walsh-Hadamard
// transform runs butterfly strides 1, 2, 4 inside each chunk, 8 and 16 across
// the row's 4 lanes (DPP quad permutes, no LDS traffic) and 32, 64 across the
// lane's chunks; every butterfly is one fp32 add or subtract, in
// increasing-stride order.  The block's amax is
// reduced across the workgroup, then the codes are
// e4m3_rne(y * fp32(448 / amax)).
//
// Fused rotary embedding (FlashAttention-3 report, sections 2.2 and 3.3: the
// quantisation can ride on the memory-bound RoPE pass).  With ROPE != 0 each
// row n is first rotated by the caller's cos/sin tables [N, d/2]: pair
// (a, b) -> (a cos - b sin, a sin + b cos), pairs (2i, 2i+1) (ROPE = 1,
// interleaved) or (i, i + d/2) (ROPE = 2, half-split).  Both pairings fall
// inside one lane's chunks; products and sums are rounded separately (no
// fused multiply-add), the fp32 arithmetic the test oracle emulates.
#include "common.h"
#include "launch.h"

namespace exattn {
namespace {

constexpr int kRows = 128;
constexpr int kThreads = 512;

enum Mode { kQuantBlock = 0, kAmaxOnly = 1, kQuantGiven = 2 };

// Cross-lane butterfly partner within a group of 4 lanes (DPP quad_perm):
// xor 1 -> [1,0,3,2], xor 2 -> [2,3,0,1].
template <int XOR>
__device__ __forceinline__ float quad_xor(float v) {
  constexpr int ctrl = (XOR == 1) ? 0xB1 : 0x4E;
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF,
                                                            0xF, true));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One RoPE pair: (a, b) -> (a c - b s, a s + b c), each product and the sum /
// difference rounded to fp32 on its own (contraction into fma switched off).
__device__ __forceinline__ void rope_pair(float& a, float& b, float c, float s) {
#pragma clang fp contract(off)
  const float ac = a * c, bs = b * s, as = a * s, bc = b * c;
  a = ac - bs;
  b = as + bc;
}

template <int D, bool ROTATE, int MODE, int ROPE>
__global__ __launch_bounds__(kThreads) void blockquant_kernel(const __bf16* __restrict__ X,
                                                              uint8_t* __restrict__ X8,
                                                              float* __restrict__ S,
                                                              const float* __restrict__ signs,
                                                              const float* __restrict__ rcos,
                                                              const float* __restrict__ rsin,
                                                              int H, int N, int nsb, float kconst) {
  constexpr int LPR = 4;                 // lanes per row
  constexpr int EPL = D / LPR;           // elements per lane (64, 32 or 16)
  constexpr int RPP = kThreads / LPR;    // rows per pass
  constexpr int PASSES = kRows / RPP;
  __shared__ float red[kThreads / 64];

  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int rsub = tid / LPR;
  // Without RoPE, workgroups run heads fastest: neighbouring workgroups take
  // the same 128 rows of neighbouring heads, which sit side by side in each
  // BSHD row, so the workgroups in flight read (and write) long contiguous
  // runs.  With RoPE, row blocks run fastest (measured faster there: the
  // workgroups in flight then read different rows of the cos/sin tables).
  int h, sb, b;
  if constexpr (ROPE == 0) {
    h = blockIdx.x % H;
    const int bsb = blockIdx.x / H;
    sb = bsb % nsb;
    b = bsb / nsb;
  } else {
    sb = blockIdx.x % nsb;
    const int bh0 = blockIdx.x / nsb;
    b = bh0 / H;
    h = bh0 - b * H;
  }
  const int bh = b * H + h;
  const int bid = bh * nsb + sb;  // scale slot [b, h, sb]
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = ((int64_t)b * N * H + h) * D;

  // Lane lr of a row holds the 8-element chunks lr, lr+4, lr+8, ... (element
  // 32c + 8lr + k is y[.][c][k]), so the row's 4 lanes read 64 contiguous
  // bytes per load instruction.
  constexpr int NC = EPL / 8;  // chunks per lane
  float y[PASSES][NC][8];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = sb * kRows + p * RPP + rsub;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 xv = {};
      if (row < N) xv = *(const bf16x8*)(X + head_off + (int64_t)row * rs + 32 * c + 8 * lr);
#pragma unroll
      for (int k = 0; k < 8; ++k) y[p][c][k] = (float)xv[k];
    }
  }
  if constexpr (ROPE != 0) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = sb * kRows + p * RPP + rsub;
      if (row < N) {
        const float* cr = rcos + (int64_t)row * (D / 2);
        const float* sr = rsin + (int64_t)row * (D / 2);
        if constexpr (ROPE == 1) {
          // element 32c + 8lr + k, k even, pairs with k + 1: pair 16c + 4lr + k/2
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const f32x4 cv = *(const f32x4*)(cr + 16 * c + 4 * lr);
            const f32x4 sv = *(const f32x4*)(sr + 16 * c + 4 * lr);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              rope_pair(y[p][c][2 * q], y[p][c][2 * q + 1], cv[q], sv[q]);
            }
          }
        } else {
          // element 32c + 8lr + k (c < NC/2) pairs with the same k of chunk c + NC/2
#pragma unroll
          for (int c = 0; c < NC / 2; ++c) {
            const f32x4 c0 = *(const f32x4*)(cr + 32 * c + 8 * lr);
            const f32x4 c1 = *(const f32x4*)(cr + 32 * c + 8 * lr + 4);
            const f32x4 s0 = *(const f32x4*)(sr + 32 * c + 8 * lr);
            const f32x4 s1 = *(const f32x4*)(sr + 32 * c + 8 * lr + 4);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float cs = k < 4 ? c0[k & 3] : c1[k & 3], sn = k < 4 ? s0[k & 3] : s1[k & 3];
              rope_pair(y[p][c][k], y[p][c + NC / 2][k], cs, sn);
            }
          }
        }
      }
    }
  }
  float amax = 0.f;
  if (ROTATE) {
    float sg[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < 8; ++k) sg[c][k] = signs[32 * c + 8 * lr + k];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < 8; ++k) y[p][c][k] *= sg[c][k];
      // strides 1, 2, 4: inside each chunk
#pragma unroll
      for (int st = 1; st < 8; st <<= 1)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((k & st) == 0) {
              const float a = y[p][c][k], b2 = y[p][c][k + st];
              y[p][c][k] = a + b2;
              y[p][c][k + st] = a - b2;
            }
      // strides 8, 16: across the row's 4 lanes.  The lower lane of a pair
      // keeps y + partner, the upper one partner - y: partner + sgn * y with
      // sgn = -1 on the upper lane (one fma, exact sign, one rounding).
      const float sg8 = (lr & 1) ? -1.f : 1.f, sg16 = (lr & 2) ? -1.f : 1.f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < 8; ++k) y[p][c][k] = __builtin_fmaf(sg8, y[p][c][k], quad_xor<1>(y[p][c][k]));
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int k = 0; k < 8; ++k) y[p][c][k] = __builtin_fmaf(sg16, y[p][c][k], quad_xor<2>(y[p][c][k]));
      // strides 32, 64 (, 128): across this lane's chunks
#pragma unroll
      for (int st = 1; st < NC; st <<= 1)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if ((c & st) == 0)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const float a = y[p][c][k], b2 = y[p][c + st][k];
              y[p][c][k] = a + b2;
              y[p][c + st][k] = a - b2;
            }
    }
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(y[p][c][k]));

  // workgroup max
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) amax = fmaxf(amax, red[w]);

  if (MODE == kAmaxOnly) {
    if (tid == 0) S[bid] = amax;
    return;
  }
  if (MODE == kQuantGiven) {
    amax = S[bid];   // tensor-wide amax, broadcast to every slot beforehand
    __syncthreads(); // every thread has read its slot before thread 0 rewrites it
  }
  float r, scale;
  if (amax > 0.f) {
    r = 448.f / amax;
    scale = amax * kconst;
  } else {
    r = 1.f;
    scale = 1.f;
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = sb * kRows + p * RPP + rsub;
    if (row < N) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        i32x2 w;
        w[0] = (int)pack_fp8x4(y[p][c][0] * r, y[p][c][1] * r, y[p][c][2] * r, y[p][c][3] * r);
        w[1] = (int)pack_fp8x4(y[p][c][4] * r, y[p][c][5] * r, y[p][c][6] * r, y[p][c][7] * r);
        *(i32x2*)(X8 + head_off + (int64_t)row * rs + 32 * c + 8 * lr) = w;
      }
    }
  }
  if (tid == 0) S[bid] = scale;
}

// One workgroup: max over all n slots, written back to every slot.
__global__ __launch_bounds__(1024) void max_broadcast_kernel(float* __restrict__ S, int n) {
  __shared__ float red[16];
  float mx = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) mx = fmaxf(mx, S[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) mx = fmaxf(mx, red[w]);
  for (int i = threadIdx.x; i < n; i += 1024) S[i] = mx;
}

template <int D, bool ROTATE, int ROPE>
hipError_t launch(const void* x, void* x8, float* scale, const float* signs, const float* rcos,
                  const float* rsin, int B, int H, int N, int block_rows, hipStream_t stream) {
  const int nsb = (N + kRows - 1) / kRows;
  const int64_t nslots = (int64_t)B * H * nsb;
  const unsigned grid = (unsigned)nslots;
  const float kconst = ROTATE ? (float)(1.0 / (448.0 * __builtin_sqrt((double)D))) : (float)(1.0 / 448.0);
  const __bf16* xp = (const __bf16*)x;
  uint8_t* qp = (uint8_t*)x8;
  if (block_rows != 0) {
    hipLaunchKernelGGL((blockquant_kernel<D, ROTATE, kQuantBlock, ROPE>), dim3(grid),
                       dim3(kThreads), 0, stream, xp, qp, scale, signs, rcos, rsin, H, N, nsb, kconst);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((blockquant_kernel<D, ROTATE, kAmaxOnly, ROPE>), dim3(grid), dim3(kThreads),
                     0, stream, xp, qp, scale, signs, rcos, rsin, H, N, nsb, kconst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(max_broadcast_kernel, dim3(1), dim3(1024), 0, stream, scale, (int)nslots);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((blockquant_kernel<D, ROTATE, kQuantGiven, ROPE>), dim3(grid),
                     dim3(kThreads), 0, stream, xp, qp, scale, signs, rcos, rsin, H, N, nsb, kconst);
  return hipGetLastError();
}

template <int ROPE>
hipError_t dispatch(const void* x, void* x8, float* scale, const float* signs, const float* rcos,
                    const float* rsin, int B, int H, int N, int d, int block_rows,
                    hipStream_t stream) {
  const bool rot = signs != nullptr;
  if (d == 256)
    return rot ? launch<256, true, ROPE>(x, x8, scale, signs, rcos, rsin, B, H, N, block_rows,
                                         stream)
               : launch<256, false, ROPE>(x, x8, scale, signs, rcos, rsin, B, H, N, block_rows,
                                          stream);
  if (d == 128)
    return rot ? launch<128, true, ROPE>(x, x8, scale, signs, rcos, rsin, B, H, N, block_rows,
                                         stream)
               : launch<128, false, ROPE>(x, x8, scale, signs, rcos, rsin, B, H, N, block_rows,
                                          stream);
  return rot ? launch<64, true, ROPE>(x, x8, scale, signs, rcos, rsin, B, H, N, block_rows, stream)
             : launch<64, false, ROPE>(x, x8, scale, signs, rcos, rsin, B, H, N, block_rows,
                                       stream);
}

}  // namespace

hipError_t launch_blockquant(const void* x, void* x8, float* scale, const float* signs, int B, int H,
                             int N, int d, int block_rows, hipStream_t stream) {
  return dispatch<0>(x, x8, scale, signs, nullptr, nullptr, B, H, N, d, block_rows, stream);
}

hipError_t launch_rope_blockquant(const void* x, void* x8, float* scale, const float* signs,
                                  const float* rcos, const float* rsin, bool interleaved, int B,
                                  int H, int N, int d, int block_rows, hipStream_t stream) {
  return interleaved
             ? dispatch<1>(x, x8, scale, signs, rcos, rsin, B, H, N, d, block_rows, stream)
             : dispatch<2>(x, x8, scale, signs, rcos, rsin, B, H, N, d, block_rows, stream);
}

}  // namespace exattn
