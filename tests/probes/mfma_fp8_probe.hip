// Test-support probe (not part of the library): the result of the gfx950
// e4m3 x e4m3 -> fp32 MFMA (v_mfma_f32_32x32x64_f8f6f4, the instruction the
// FP8 attention kernel uses for S = K Q^T and O = V^T P^T), chained over KS
// 64-wide k-steps, for many independent 32 x 32 problems.  The FP8 parity
// bound of the tests assumes its deviation from the exact dot product; this
// kernel lets a GPU test measure that deviation.
//
// Problem p: A_p (32 x 64 KS codes, row-major), B_p given as B_p^T (32 x
// 64 KS codes, row-major), D_p = A_p B_p (32 x 32 fp32, row-major).  One
// wave per problem; lane l holds row (A) / column (B) l % 32 and the 32
// k-slots 32 (l / 32) .. +31 of each k-step; accumulator register v of lane
// l is D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int KS>
__global__ __launch_bounds__(64) void mfma_fp8_probe_kernel(const uint8_t* __restrict__ A,
                                                            const uint8_t* __restrict__ BT,
                                                            float* __restrict__ D, int nprob) {
  const int p = blockIdx.x;
  if (p >= nprob) return;
  const int l = threadIdx.x, r = l & 31, h = l >> 5;
  const uint8_t* a = A + (size_t)p * 32 * 64 * KS;
  const uint8_t* bt = BT + (size_t)p * 32 * 64 * KS;
  f32x16 acc = {};
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    const i32x8 fa = *(const i32x8*)(a + r * 64 * KS + 64 * t + 32 * h);
    const i32x8 fb = *(const i32x8*)(bt + r * 64 * KS + 64 * t + 32 * h);
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc, 0, 0, 0, 0, 0, 0);
  }
  float* d = D + (size_t)p * 32 * 32;
#pragma unroll
  for (int v = 0; v < 16; ++v) d[(8 * (v / 4) + 4 * h + v % 4) * 32 + r] = acc[v];
}

// A, BT: device buffers of nprob * 32 * 64 * ks bytes (32-byte aligned);
// D: nprob * 1024 floats.  ks in {1, 2, 4}.  Returns 0 or a HIP error code.
extern "C" int mfma_fp8_probe(const uint8_t* A, const uint8_t* BT, float* D, int nprob, int ks) {
  if (nprob < 1 || (ks != 1 && ks != 2 && ks != 4)) return -1;
  if (ks == 1) hipLaunchKernelGGL(mfma_fp8_probe_kernel<1>, dim3(nprob), dim3(64), 0, 0, A, BT, D, nprob);
  if (ks == 2) hipLaunchKernelGGL(mfma_fp8_probe_kernel<2>, dim3(nprob), dim3(64), 0, 0, A, BT, D, nprob);
  if (ks == 4) hipLaunchKernelGGL(mfma_fp8_probe_kernel<4>, dim3(nprob), dim3(64), 0, 0, A, BT, D, nprob);
  return (int)hipDeviceSynchronize();
}
