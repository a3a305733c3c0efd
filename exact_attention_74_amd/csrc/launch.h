// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C ABI layer before any of these is called; each launcher only enqueues work
// on `stream` and returns the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>

#include <atomic>

namespace exattn {

// Compute units of the current device, queried once per device and cached
// (thread-safe); 0 when the query fails.
inline int current_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      ncu <= 0)
    return 0;
  if (dev < 64) cache[dev].store(ncu, std::memory_order_relaxed);
  return ncu;
}

// Workgroups of `kernel` (block size `threads`, no dynamic LDS) resident on
// one CU at a time, from the runtime's occupancy calculator; queried once per
// kernel (the cache slot is the caller's, one per kernel instance) and 0 when
// the query fails.
template <typename K>
inline int resident_per_cu(K kernel, int threads, std::atomic<int>& cache) {
  const int c = cache.load(std::memory_order_relaxed);
  if (c > 0) return c;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0)
    return 0;
  cache.store(n, std::memory_order_relaxed);
  return n;
}

// Hkv: K/V heads (H a multiple of it); query head h reads K/V head h / (H / Hkv).
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Hkv, int N, int d, bool causal,
                                float softmax_scale, hipStream_t stream, bool same_phase = false);

hipError_t launch_attn_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* sq,
                               const float* sk, const float* sv, void* o, float* lse, int B, int H,
                               int Hkv, int N, int d, bool causal, float softmax_scale,
                               hipStream_t stream);

// Gradients of the bf16 forward; workspace: 2 B H N floats (D, LSE*log2e);
// K/V (and dK/dV) on Hkv heads.
hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                float* workspace, int B, int H, int Hkv, int N, int d,
                                bool causal, float softmax_scale, hipStream_t stream);

// The same with the workspace in the library's fixed per-device scratch
// array (bwd_scratch_bytes() bytes; 8 B H N must fit): no allocation.
hipError_t launch_attn_bwd_bf16_noalloc(const void* q, const void* k, const void* v,
                                        const void* o, const void* dout, const float* lse,
                                        void* dq, void* dk, void* dv, int B, int H, int Hkv,
                                        int N, int d, bool causal, float softmax_scale,
                                        hipStream_t stream);
size_t bwd_scratch_bytes();

hipError_t launch_blockquant(const void* x, void* x8, float* scale, const float* signs, int B, int H,
                             int N, int d, int block_rows, hipStream_t stream);

// blockquant with a rotary embedding first: cos/sin tables [N, d/2] fp32,
// pairs (2i, 2i+1) when interleaved, else (i, i + d/2).
hipError_t launch_rope_blockquant(const void* x, void* x8, float* scale, const float* signs,
                                  const float* rcos, const float* rsin, bool interleaved, int B,
                                  int H, int N, int d, int block_rows, hipStream_t stream);

}  // namespace exattn
