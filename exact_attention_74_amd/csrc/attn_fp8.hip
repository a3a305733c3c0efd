// FP8 (OCP e4m3) exact-attention forward for gfx950, the low-precision scheme
// of the FlashAttention-3 report, section 3.3.
//
// Same decomposition as the bf16 kernel (one workgroup per (b, h, 128 query
// rows), four waves of 32 rows, transposed S^T = K Q^T / O^T = V^T P^T
// formulation) with 128-key blocks, so that every query block and every key
// block coincides with one 128-row quantisation block:
//   * S block scaling: the tile's scalar q_scale * k_scale * softmax_scale *
//     log2(e) multiplies the fp32 accumulator inside the exp2 argument.
//   * P is rounded to e4m3 (v_cvt_pk_fp8_f32) straight from the S^T
//     accumulator: half-wave h, byte slot s of the 64-key k-step u holds key
//     64u + 32*(s/16) + 8*((s%16)/4) + 4h + s%4.
//   * In-LDS V relayout: the fp8 MFMA wants, per lane, 32 consecutive k bytes
//     of one head dim, so the V tile is written to LDS transposed (V^T, key
//     bytes contiguous) with its keys permuted to match the slot order above.
//     Each unit of 16 keys x 16 dims is a 16x16 byte transpose in registers.
//   * V block scales: O is kept in units of the current block's v_scale and
//     rescaled by alpha * v_scale_prev / v_scale_cur when the block changes.
#include "common.h"
#include "launch.h"

namespace exattn {
namespace {

constexpr int kBR = 128;
constexpr int kBC = 128;
constexpr int kQB = 128;  // rows per quantisation block
constexpr int kThreads = 256;

// 16x16 byte transpose: out[j] byte i = in[i] byte j.
__device__ __forceinline__ void transpose16x16(const i32x4 (&in)[16], i32x4 (&out)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int w = j >> 2, sh = 8 * (j & 3);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) v |= (((uint32_t)in[4 * q + t][w] >> sh) & 0xFFu) << (8 * t);
      out[j][q] = (int)v;
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ SQ, const float* __restrict__ SK, const float* __restrict__ SV,
    __bf16* __restrict__ O, float* __restrict__ LSE, int H, int N, float scale_log2, int nqb) {
  constexpr int KP = D + 16;    // bytes
  constexpr int VP = kBC + 16;  // bytes
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kBC * KP];
  __shared__ __attribute__((aligned(16))) uint8_t Vt[D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int hh = lane >> 5;

  const int bid = blockIdx.x;
  const int qb_raw = bid % nqb;
  const int bh = bid / nqb;
  const int qblk = CAUSAL ? (nqb - 1 - qb_raw) : qb_raw;
  const int b = bh / H;
  const int h = bh - b * H;
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = ((int64_t)b * N * H + h) * D;
  const uint8_t* Qh = Q + head_off;
  const uint8_t* Kh = K + head_off;
  const uint8_t* Vh = V + head_off;
  const int nsb = (N + kQB - 1) / kQB;
  const float* sk_bh = SK + (int64_t)bh * nsb;
  const float* sv_bh = SV + (int64_t)bh * nsb;
  const float sq = SQ[(int64_t)bh * nsb + qblk];

  const int q0 = qblk * kBR + wave * 32;
  const int qi = q0 + li;

  // Q^T as the B operand: k-step t covers dims 64t .. 64t+63; half h holds
  // dims 64t + 32h .. +31 of query qi.
  i32x8 qf[D / 64];
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    i32x8 z = {};
    qf[t] = (qi < N) ? *(const i32x8*)(Qh + (int64_t)qi * rs + 64 * t + 32 * hh) : z;
  }

  float m = kNoMax;
  float l = 0.f;
  float sv_prev = 1.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) oacc[e] = f32x16{};

  const int nkb_all = ceil_div(N, kBC);
  const int nkb = CAUSAL ? min(nkb_all, qblk + 1) : nkb_all;

  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * kBC;
    __syncthreads();
#pragma unroll
    for (int c = tid; c < kBC * D / 16; c += kThreads) {
      const int r = c / (D / 16), cc = c % (D / 16);
      i32x4 val = {};
      if (k0 + r < N) val = *(const i32x4*)(Kh + (int64_t)(k0 + r) * rs + cc * 16);
      *(i32x4*)(Ks + r * KP + cc * 16) = val;
    }
    // V^T relayout.  Unit (u, hv, c2, dc): keys 64u + 32c2 + 8g + 4hv + r
    // (g, r in 0..3) x dims 16dc .. 16dc+15, written to V^T rows
    // 16dc .. +15 at byte positions 64u + 32hv + 16c2 + 4g + r.
#pragma unroll
    for (int c = tid; c < (kBC / 64) * 4 * (D / 16); c += kThreads) {
      const int dc = c % (D / 16);
      const int c2 = (c / (D / 16)) & 1;
      const int hv = (c / (D / 8)) & 1;
      const int u = c / (D / 4);
      i32x4 in[16], out[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = k0 + 64 * u + 32 * c2 + 8 * (j >> 2) + 4 * hv + (j & 3);
        i32x4 z = {};
        in[j] = (key < N) ? *(const i32x4*)(Vh + (int64_t)key * rs + dc * 16) : z;
      }
      transpose16x16(in, out);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        *(i32x4*)(Vt + (16 * dc + j) * VP + 64 * u + 32 * hv + 16 * c2) = out[j];
    }
    __syncthreads();

    f32x16 sacc[kBC / 32];
#pragma unroll
    for (int j = 0; j < kBC / 32; ++j) {
      sacc[j] = f32x16{};
#pragma unroll
      for (int t = 0; t < D / 64; ++t) {
        const i32x8 a = *(const i32x8*)(Ks + (j * 32 + li) * KP + 64 * t + 32 * hh);
        sacc[j] = mfma_fp8(a, qf[t], sacc[j]);
      }
    }

    if (k0 + kBC > N || (CAUSAL && k0 + kBC - 1 > q0)) {
#pragma unroll
      for (int j = 0; j < kBC / 32; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + j * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key >= N || (CAUSAL && key > qi)) sacc[j][v] = -INFINITY;
        }
    }

    const float c_tile = scale_log2 * sq * sk_bh[kb];
    const float sv = sv_bh[kb];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBC / 32; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[j][v]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m, mx * c_tile);
    const float alpha = exp2_fast(m - m_new);
    float rsum = 0.f;
#pragma unroll
    for (int j = 0; j < kBC / 32; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2_fast(__builtin_fmaf(sacc[j][v], c_tile, -m_new));
        sacc[j][v] = p;
        rsum += p;
      }
    l = l * alpha + rsum;
    m = m_new;
    const float f = alpha * (sv_prev / sv);
    sv_prev = sv;
#pragma unroll
    for (int e = 0; e < D / 32; ++e) oacc[e] *= f;

    // P^T in e4m3: k-step u, word w holds slots 4w..4w+3 = accumulator
    // block 2u + w/4, registers 4(w%4) .. +3.
    i32x8 pf[kBC / 64];
#pragma unroll
    for (int u = 0; u < kBC / 64; ++u)
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const f32x16& sa = sacc[2 * u + (w >> 2)];
        const int r0 = 4 * (w & 3);
        pf[u][w] = (int)pack_fp8x4(sa[r0], sa[r0 + 1], sa[r0 + 2], sa[r0 + 3]);
      }

#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int u = 0; u < kBC / 64; ++u) {
        const i32x8 a = *(const i32x8*)(Vt + (32 * e + li) * VP + 64 * u + 32 * hh);
        oacc[e] = mfma_fp8(a, pf[u], oacc[e]);
      }
  }

  const float lt = l + xor32(l);
  const float inv = sv_prev / lt;
  if (qi < N) {
    __bf16* orow = O + head_off + (int64_t)qi * rs;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        i32x2 pk;
        pk[0] = (int)pack_bf16x2(oacc[e][4 * g + 0] * inv, oacc[e][4 * g + 1] * inv);
        pk[1] = (int)pack_bf16x2(oacc[e][4 * g + 2] * inv, oacc[e][4 * g + 3] * inv);
        *(i32x2*)(orow + 32 * e + 8 * g + 4 * hh) = pk;
      }
    if (LSE != nullptr && hh == 0) LSE[(int64_t)bh * N + qi] = (m + __log2f(lt)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk,
                  const float* sv, void* o, float* lse, int B, int H, int N, float scale,
                  hipStream_t stream) {
  const int nqb = (N + kBR - 1) / kBR;
  const unsigned grid = (unsigned)((int64_t)B * H * nqb);
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream,
                     (const uint8_t*)q8, (const uint8_t*)k8, (const uint8_t*)v8, sq, sk, sv,
                     (__bf16*)o, lse, H, N, scale * kLog2e, nqb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* sq,
                               const float* sk, const float* sv, void* o, float* lse, int B, int H,
                               int N, int d, bool causal, float softmax_scale, hipStream_t stream) {
  if (d == 128)
    return causal ? launch<128, true>(q8, k8, v8, sq, sk, sv, o, lse, B, H, N, softmax_scale, stream)
                  : launch<128, false>(q8, k8, v8, sq, sk, sv, o, lse, B, H, N, softmax_scale, stream);
  return causal ? launch<64, true>(q8, k8, v8, sq, sk, sv, o, lse, B, H, N, softmax_scale, stream)
                : launch<64, false>(q8, k8, v8, sq, sk, sv, o, lse, B, H, N, softmax_scale, stream);
}

}  // namespace exattn
