// FP8 pre-pass for gfx950: optional incoherent processing (random +-1 diagonal
// times a Hadamard matrix, FlashAttention-3 report sections 2.2 / 3.3) fused
// with block quantisation to OCP e4m3.
//
// HBM-bound: one read of the bf16 tensor and one write of the e4m3 codes.  A
// workgroup owns one 128-row x d block of one (b, h); d/8 lanes share a row,
// each lane holding 8 consecutive elements, so a row is read and written with
// 16-byte (bf16) and 8-byte (e4m3) vector accesses.  The fast Walsh-Hadamard
// transform runs its butterfly strides 1, 2, 4 inside the lane and strides
// 8 .. d/2 across lanes (xor-shuffles within the row's lane group); every
// butterfly is one fp32 add or subtract, in increasing-stride order.  The
// block's amax is reduced across the workgroup, then the codes are
// e4m3_rne(y * fp32(448 / amax)).
#include "common.h"
#include "launch.h"

namespace exattn {
namespace {

constexpr int kRows = 128;
constexpr int kThreads = 256;

enum Mode { kQuantBlock = 0, kAmaxOnly = 1, kQuantGiven = 2 };

template <int D, bool ROTATE, int MODE>
__global__ __launch_bounds__(kThreads) void blockquant_kernel(const __bf16* __restrict__ X,
                                                              uint8_t* __restrict__ X8,
                                                              float* __restrict__ S,
                                                              const float* __restrict__ signs,
                                                              int H, int N, int nsb, float kconst) {
  constexpr int LPR = D / 8;             // lanes per row
  constexpr int RPP = kThreads / LPR;    // rows per pass
  constexpr int PASSES = kRows / RPP;
  __shared__ float red[kThreads / 64];

  const int tid = threadIdx.x;
  const int lr = tid % LPR;
  const int rsub = tid / LPR;
  const int bid = blockIdx.x;
  const int sb = bid % nsb;
  const int bh = bid / nsb;
  const int b = bh / H;
  const int h = bh - b * H;
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = ((int64_t)b * N * H + h) * D;

  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sg[e] = ROTATE ? signs[lr * 8 + e] : 1.f;

  float y[PASSES][8];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = sb * kRows + p * RPP + rsub;
    bf16x8 xv = {};
    if (row < N) xv = *(const bf16x8*)(X + head_off + (int64_t)row * rs + lr * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[p][e] = (float)xv[e];
    if (ROTATE) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[p][e] *= sg[e];
      // strides 1, 2, 4 inside the lane
#pragma unroll
      for (int st = 1; st < 8; st <<= 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if ((e & st) == 0) {
            const float a = y[p][e], c = y[p][e + st];
            y[p][e] = a + c;
            y[p][e + st] = a - c;
          }
        }
      }
      // strides 8 .. D/2 across the lanes of the row
#pragma unroll
      for (int lm = 1; lm < LPR; lm <<= 1) {
        const bool upper = (lr & lm) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float other = __shfl_xor(y[p][e], lm, 64);
          y[p][e] = upper ? (other - y[p][e]) : (y[p][e] + other);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[p][e]));
  }

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
      i32x2 c;
      c[0] = (int)pack_fp8x4(y[p][0] * r, y[p][1] * r, y[p][2] * r, y[p][3] * r);
      c[1] = (int)pack_fp8x4(y[p][4] * r, y[p][5] * r, y[p][6] * r, y[p][7] * r);
      *(i32x2*)(X8 + head_off + (int64_t)row * rs + lr * 8) = c;
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

template <int D, bool ROTATE>
hipError_t launch(const void* x, void* x8, float* scale, const float* signs, int B, int H, int N,
                  int block_rows, hipStream_t stream) {
  const int nsb = (N + kRows - 1) / kRows;
  const int64_t nslots = (int64_t)B * H * nsb;
  const unsigned grid = (unsigned)nslots;
  const float kconst = ROTATE ? (float)(1.0 / (448.0 * __builtin_sqrt((double)D))) : (float)(1.0 / 448.0);
  const __bf16* xp = (const __bf16*)x;
  uint8_t* qp = (uint8_t*)x8;
  if (block_rows != 0) {
    hipLaunchKernelGGL((blockquant_kernel<D, ROTATE, kQuantBlock>), dim3(grid), dim3(kThreads), 0,
                       stream, xp, qp, scale, signs, H, N, nsb, kconst);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((blockquant_kernel<D, ROTATE, kAmaxOnly>), dim3(grid), dim3(kThreads), 0,
                     stream, xp, qp, scale, signs, H, N, nsb, kconst);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(max_broadcast_kernel, dim3(1), dim3(1024), 0, stream, scale, (int)nslots);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((blockquant_kernel<D, ROTATE, kQuantGiven>), dim3(grid), dim3(kThreads), 0,
                     stream, xp, qp, scale, signs, H, N, nsb, kconst);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_blockquant(const void* x, void* x8, float* scale, const float* signs, int B, int H,
                             int N, int d, int block_rows, hipStream_t stream) {
  const bool rot = signs != nullptr;
  if (d == 128)
    return rot ? launch<128, true>(x, x8, scale, signs, B, H, N, block_rows, stream)
               : launch<128, false>(x, x8, scale, signs, B, H, N, block_rows, stream);
  return rot ? launch<64, true>(x, x8, scale, signs, B, H, N, block_rows, stream)
             : launch<64, false>(x, x8, scale, signs, B, H, N, block_rows, stream);
}

}  // namespace exattn
