// bf16 exact-attention forward for gfx950.
//
// Work decomposition (FA2 query-block parallelism, "Efficient Attention &
// FlashAttention" M4-054): one workgroup per (b, h, block of 128 query rows),
// four waves of 32 query rows each; the key/value sequence is streamed in
// blocks of 64 keys through LDS with the online-softmax recurrence of the
// FlashAttention-3 report, section 3 (running max m, running sum l, one final
// normalisation).
//
// Transposed formulation.  Each wave computes S^T = K Q^T (keys as MFMA rows,
// its 32 queries as MFMA columns), so the accumulator puts every query on one
// lane pair (l, l^32): row max and row sum are in-lane reductions plus one
// cross-half exchange.  The output is accumulated as O^T = V^T P^T, whose
// accumulator again keeps one query per lane, so the per-row rescale factor
// is a lane-local scalar.  P^T is fed to the second MFMA straight from the S^T
// accumulator registers (converted to bf16): with the accumulator layout, the
// 8 k-slots of half-wave h in k-step t hold keys 16t + 8*(s/4) + 4h + s%4, and
// V^T is stored in LDS with its keys permuted the same way (bits 2 and 3 of
// the key index swapped within each group of 16), so no register shuffle is
// needed.  This is the gfx950 counterpart of the report's accumulator-to-
// operand relayout (section 3.3).
#include "common.h"
#include "launch.h"

namespace exattn {
namespace {

constexpr int kBR = 128;  // query rows per workgroup
constexpr int kBC = 64;   // keys per KV block
constexpr int kThreads = 256;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int H, int N, float scale_log2, int nqb) {
  constexpr int KP = D + 8;    // K tile row pitch (elements); +16 B breaks bank aliasing
  constexpr int VP = kBC + 8;  // V^T tile row pitch (elements)
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kBC * KP];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;  // query column of this lane
  const int hh = lane >> 5;  // half-wave

  const int bid = blockIdx.x;
  const int qb_raw = bid % nqb;
  const int bh = bid / nqb;  // b * H + h
  const int qblk = CAUSAL ? (nqb - 1 - qb_raw) : qb_raw;  // heaviest causal blocks first
  const int b = bh / H;
  const int h = bh - b * H;
  const int64_t rs = (int64_t)H * D;  // element stride between sequence positions
  const int64_t head_off = ((int64_t)b * N * H + h) * D;
  const __bf16* Qh = Q + head_off;
  const __bf16* Kh = K + head_off;
  const __bf16* Vh = V + head_off;

  const int q0 = qblk * kBR + wave * 32;  // first query row of this wave
  const int qi = q0 + li;                 // this lane's query row

  // Q^T as the B operand: k-step t covers head dims 16t .. 16t+15, half h
  // holds dims 16t + 8h .. +7 of query qi.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    bf16x8 z = {};
    qf[t] = (qi < N) ? *(const bf16x8*)(Qh + (int64_t)qi * rs + 16 * t + 8 * hh) : z;
  }

  float m = kNoMax;  // running max of scale*log2(e)*s (base-2 domain)
  float l = 0.f;     // running sum over this lane's half of the keys
  f32x16 oacc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) oacc[e] = f32x16{};

  const int nkb_all = ceil_div(N, kBC);
  const int nkb = CAUSAL ? min(nkb_all, ceil_div(min(N, (qblk + 1) * kBR), kBC)) : nkb_all;

  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * kBC;
    __syncthreads();  // previous tiles fully consumed
    // K tile, row-major, 16-byte chunks.
#pragma unroll
    for (int c = tid; c < kBC * D / 8; c += kThreads) {
      const int r = c / (D / 8), cc = c % (D / 8);
      bf16x8 val = {};
      if (k0 + r < N) val = *(const bf16x8*)(Kh + (int64_t)(k0 + r) * rs + cc * 8);
      *(bf16x8*)(Ks + r * KP + cc * 8) = val;
    }
    // V tile, transposed to V^T[d][key'] with key' = key with bits 2,3 swapped
    // inside each group of 16.  A unit is 8 keys x 8 dims: keys
    // {4hb..4hb+3, 8+4hb..8+4hb+3} of one 16-group land contiguously at
    // positions 8hb..8hb+7.
#pragma unroll
    for (int c = tid; c < (kBC / 16) * 2 * (D / 8); c += kThreads) {
      const int dc = c % (D / 8);
      const int hb = (c / (D / 8)) & 1;
      const int g16 = c / (D / 4);
      i32x4 r[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int key = k0 + g16 * 16 + (s < 4 ? 4 * hb + s : 8 + 4 * hb + (s - 4));
        i32x4 z = {};
        r[s] = (key < N) ? *(const i32x4*)(Vh + (int64_t)key * rs + dc * 8) : z;
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int w = dd >> 1;
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        i32x4 out;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          out[u] = (int)__builtin_amdgcn_perm((uint32_t)r[2 * u + 1][w], (uint32_t)r[2 * u][w], sel);
        *(i32x4*)(Vt + (dc * 8 + dd) * VP + g16 * 16 + 8 * hb) = out;
      }
    }
    __syncthreads();

    // S^T = K Q^T for the 64 keys, as two 32x32 accumulators.
    f32x16 sacc[kBC / 32];
#pragma unroll
    for (int j = 0; j < kBC / 32; ++j) {
      sacc[j] = f32x16{};
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 a = *(const bf16x8*)(Ks + (j * 32 + li) * KP + 16 * t + 8 * hh);
        sacc[j] = mfma_bf16(a, qf[t], sacc[j]);
      }
    }

    // Mask keys past the end and (causal) keys after the query.
    if (k0 + kBC > N || (CAUSAL && k0 + kBC - 1 > q0)) {
#pragma unroll
      for (int j = 0; j < kBC / 32; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + j * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key >= N || (CAUSAL && key > qi)) sacc[j][v] = -INFINITY;
        }
    }

    // Online softmax in the base-2 domain.
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBC / 32; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[j][v]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m, mx * scale_log2);
    const float alpha = exp2_fast(m - m_new);
    float rsum = 0.f;
#pragma unroll
    for (int j = 0; j < kBC / 32; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2_fast(__builtin_fmaf(sacc[j][v], scale_log2, -m_new));
        sacc[j][v] = p;
        rsum += p;
      }
    l = l * alpha + rsum;
    m = m_new;
#pragma unroll
    for (int e = 0; e < D / 32; ++e) oacc[e] *= alpha;

    // P^T (bf16) as the B operand: k-step t2 takes accumulator registers
    // 8*(t2%2) .. +7 of block t2/2.
    bf16x8 pb[kBC / 16];
#pragma unroll
    for (int t2 = 0; t2 < kBC / 16; ++t2)
#pragma unroll
      for (int s = 0; s < 8; ++s) pb[t2][s] = (__bf16)sacc[t2 >> 1][8 * (t2 & 1) + s];

    // O^T += V^T P^T.
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int t2 = 0; t2 < kBC / 16; ++t2) {
        const bf16x8 a = *(const bf16x8*)(Vt + (32 * e + li) * VP + 16 * t2 + 8 * hh);
        oacc[e] = mfma_bf16(a, pb[t2], oacc[e]);
      }
  }

  // Epilogue: one normalisation per row, bf16 store, log-sum-exp.
  const float lt = l + xor32(l);
  const float inv = 1.f / lt;
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
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int N, float scale, hipStream_t stream) {
  const int nqb = (N + kBR - 1) / kBR;
  const unsigned grid = (unsigned)((int64_t)B * H * nqb);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, H, N,
                     scale * kLog2e, nqb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int N, int d, bool causal, float softmax_scale,
                                hipStream_t stream) {
  if (d == 128)
    return causal ? launch<128, true>(q, k, v, o, lse, B, H, N, softmax_scale, stream)
                  : launch<128, false>(q, k, v, o, lse, B, H, N, softmax_scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, B, H, N, softmax_scale, stream)
                : launch<64, false>(q, k, v, o, lse, B, H, N, softmax_scale, stream);
}

}  // namespace exattn
