// FP8 (OCP e4m3) exact-attention forward for gfx950: the low-precision scheme
// of the FlashAttention-3 report, section 3.3, on v_mfma_f32_32x32x64_f8f6f4.
//
// Decomposition as in the bf16 kernel: one workgroup of 8 waves per (b, h,
// block of 256 query rows), 32 query rows per wave, two waves per SIMD (head
// dim 256: 4 waves and 128 rows, one wave per SIMD with its 512 registers);
// the keys are streamed 128 at a time, so every key tile is exactly one
// quantisation block and every wave's rows lie in one query block:
//   * S block scaling: the tile's scalar q_scale * k_scale * softmax_scale *
//     log2(e) multiplies the fp32 accumulator inside the exp2 argument.
//   * Transposed formulation S^T = K Q^T and O^T = V^T P^T: every query sits
//     on one lane pair, so row max / row sum are in-lane plus one exchange.
//   * P is rounded to e4m3 (v_cvt_pk_fp8_f32) straight from the S^T
//     accumulator: half-wave h, byte slot s of the 64-key k-step u holds key
//     64u + 32*(s/16) + 8*((s%16)/4) + 4h + s%4.
//   * V relayout in LDS: the V tile stays key-major in LDS and each lane's
//     32-key V^T operand is gathered with four ds_read_b64_tr_b8 transposed
//     reads in exactly the slot order above (the gfx950 counterpart of the
//     report's in-kernel V transpose and byte permute).
//   * V block scales: O is kept in units of the current tile's v_scale and
//     rescaled by alpha * v_scale_prev / v_scale_cur at each tile, together
//     with the online-softmax correction alpha.  The running max follows the
//     report's recurrence exactly (raised at every tile).
// K and V tiles go from HBM/L2 straight into XOR-swizzled LDS with
// buffer_load ... lds, two stages deep, one barrier per tile; reads past the
// end of the sequence return zeros.
#include "common.h"
#include "launch.h"

namespace exattn {
namespace {

constexpr int kBC = 128;  // keys per tile = rows per quantisation block
constexpr int kQB = 128;  // rows per quantisation block

// Waves per workgroup (32 query rows each).
template <int D>
constexpr int waves() { return D > 128 ? 4 : 8; }

typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct Geo8 {
  static constexpr int NW = waves<D>();
  static constexpr int RB = D;                // bytes per key row
  static constexpr int CPR = D / 16;          // 16-byte chunks per row
  static constexpr int RP = 256 / RB;         // rows per 256-byte bank cycle
  static constexpr int TILE = kBC * RB;       // bytes per K or V tile
  static constexpr int STAGE = 2 * TILE;      // K + V
  static constexpr int LOADS = TILE / (1024 * NW);
  // LDS layout: [K0 V0 K1 V1] up to d = 128; [K0 K1 V0 V1] at d = 256, with
  // the V region's base in the read addresses, so that every read offset is a
  // 16-bit immediate.
  static constexpr int VBASE = D > 128 ? 2 * TILE : 0;
  static constexpr int koff(int st) { return D > 128 ? st * TILE : st * STAGE; }
  static constexpr int voff(int st) { return D > 128 ? st * TILE : st * STAGE + TILE; }
  // chunk c of row `row` is stored at chunk position c ^ swz(row).  The V
  // swizzle spreads the eight rows (and two chunks) one transposed read
  // instruction touches per half-wave over distinct banks.
  __device__ static int swz_k(int row) { return (row / RP) % CPR; }
  __device__ static int swz_v(int row) {
    if (D == 256) return 2 * ((row & 3) | (((row >> 3) & 1) << 2));
    if (D == 128) return 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1));
    return 2 * ((row >> 3) & 1);
  }
};

// 16-byte-per-lane copy global -> LDS (lane i's chunk lands at lds_dst + 16 i);
// the scalar offset is 0 because only the per-lane offset is range-checked:
// the tile's position is in the descriptor (tile_rsrc).
__device__ __forceinline__ void copy_to_lds16(__amdgpu_buffer_rsrc_t r, char* lds_dst,
                                              uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, voff, 0, 0, 0);
}

// LDS byte address of a generic pointer into LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Transposed LDS read (ds_read_b64_tr_b8) at LDS address addr + OFF, issued
// as assembly: with the builtin, the compiler's wait-count pass drains vmcnt
// before it (it cannot tell the read from the in-flight buffer_load ... lds
// copies of the next tile), while the tile loop's own vmcnt wait and barrier
// already order them.  The result is valid after lds_wait_v().
template <int OFF>
__device__ __forceinline__ i32x2 read_tr8(uint32_t addr) {
  i32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Waits for every outstanding LDS read, passing the V^T fragments through so
// that no use of them is scheduled before the wait.
template <int NE>
__device__ __forceinline__ void lds_wait_v(i32x8 (&vf)[2][NE]) {
  static_assert(NE == 4 || NE == 2, "four or two 32-dim blocks");
  if constexpr (NE == 4)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vf[0][0]), "+v"(vf[0][1]), "+v"(vf[0][2]), "+v"(vf[0][3]),
                   "+v"(vf[1][0]), "+v"(vf[1][1]), "+v"(vf[1][2]), "+v"(vf[1][3]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(vf[0][0]), "+v"(vf[0][1]), "+v"(vf[1][0]), "+v"(vf[1][1]));
}

// -inf for keys >= N and, when causal, keys after query qi.  k0: first key.
__device__ __forceinline__ void mask_s8(f32x16 (&sacc)[4], int k0, int N, bool causal, int qi,
                                        int hh) {
  const int lim = causal ? min(N, qi + 1) : N;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + j * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
      if (key >= lim) sacc[j][v] = -INFINITY;
    }
}

// V^T operands of stage ST for NE 32-dim blocks, whose read addresses start
// at vaddr (eight transposed reads per block; valid after lds_wait_v).
template <int D, int ST, int NE>
__device__ __forceinline__ void read_vt(const uint32_t* vaddr, i32x8 (&vf)[2][NE]) {
  using G = Geo8<D>;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const uint32_t va = vaddr[e];
    i32x2 r[8];
    r[0] = read_tr8<G::voff(ST) + 0 * G::RB>(va);
    r[1] = read_tr8<G::voff(ST) + 16 * G::RB>(va);
    r[2] = read_tr8<G::voff(ST) + 32 * G::RB>(va);
    r[3] = read_tr8<G::voff(ST) + 48 * G::RB>(va);
    r[4] = read_tr8<G::voff(ST) + 64 * G::RB>(va);
    r[5] = read_tr8<G::voff(ST) + 80 * G::RB>(va);
    r[6] = read_tr8<G::voff(ST) + 96 * G::RB>(va);
    r[7] = read_tr8<G::voff(ST) + 112 * G::RB>(va);
    vf[0][e] = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    vf[1][e] = i32x8{r[4][0], r[4][1], r[5][0], r[5][1], r[6][0], r[6][1], r[7][0], r[7][1]};
  }
}

// Head dim 256: the P.V products are assembly MFMAs on "+v" operands, so O
// (rescaled by the VALU every tile) stays in VGPRs and the compiler's own
// MFMAs (S) take the AGPRs.  The wait states the compiler cannot see are
// explicit: a leading s_nop 1 where an operand was just written by the VALU,
// and o8_fence (24 wait states) between O's MFMAs and the VALU's next use.
template <bool NOP2>
__device__ __forceinline__ void mfma8_v(f32x16& acc, const i32x8& a, const i32x8& b) {
  if constexpr (NOP2)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
template <int D, bool NOP2>
__device__ __forceinline__ void pv8(f32x16& acc, const i32x8& a, const i32x8& b) {
  if constexpr (D > 128) mfma8_v<NOP2>(acc, a, b);
  else acc = mfma_fp8(a, b, acc);
}
template <int D>
__device__ __forceinline__ void o8_fence(f32x16 (&o)[D / 32]) {
  if constexpr (D > 128)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]), "+v"(o[4]), "+v"(o[5]),
                   "+v"(o[6]), "+v"(o[7]));
}


// Software-pipelined interior tiles at head dim 256 (causal: the tiles
// before a block's diagonal): one wave
// per SIMD, so no second wave's MFMAs cover the softmax; instead iteration j
// of a wave issues its MFMAs one per slot, the 16 of S(j+1) = K(j+1) Q^T and
// then the 16 of O^T += V(j)^T P(j)^T, with tile j's softmax (the exponentials,
// the O rescale) and S(j+1)'s row max spread between them (the FlashAttention-3
// report, section 3.2: the next block's S = Q K^T before the current block's
// softmax).  S(j+1) accumulates in AGPRs (assembly MFMAs, Q^T in AGPRs too),
// read by the VALU one value at a time; O stays in VGPRs for the per-tile
// rescale.  Each MFMA's operand is read kLook reads ahead and waited for with
// an exact lgkmcnt count.  The next tiles' sixteen 1 KB copies per wave go
// out one per slot in the first sixteen slots, under the MFMAs (issued
// together after the barrier they stalled the wave for most of a tile's
// softmax; one every two slots lands too late).  Every output element goes
// through the operations of the same-phase tile body in the same order, so
// the results are identical.
namespace fpipe8 {
constexpr int NS = 16;   // S(j+1) MFMAs: key block s % 4, k-step s / 4
constexpr int NP = 16;   // P.V MFMAs: key half u = k / 8, 32-dim block e = k % 8
constexpr int N = NS + NP;
constexpr int kLook = 6;
constexpr int kLast = 2 * NS + 4 * NP - 1;  // reads: 2 per S MFMA, 4 per P.V MFMA
// last read slot s's MFMA needs
constexpr int need(int s) { return s < NS ? 2 * s + 1 : 2 * NS + 4 * (s - NS) + 3; }
// reads issued by the end of slot s (s = -1: the prologue)
constexpr int issued(int s) {
  return s < 0 ? kLook : (need(s) + kLook < kLast ? need(s) + kLook : kLast);
}
// exponential v (0 .. 63, in the same-phase body's order) in slot exp_slot(v):
// P^T half u is complete before its first MFMA (slot NS + 8 u)
constexpr int exp_slot(int v) { return (3 * v) / 8; }
// O^T block e rescaled in slots 2e, 2e + 1 (before its first P.V MFMA)
constexpr int kMax0 = 24;  // S(j+1)'s row max: slots 24 .. 31, eight values each
}  // namespace fpipe8

template <int OFF>
__device__ __forceinline__ i32x4 read_k16(uint32_t addr) {
  i32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// S MFMA on an AGPR accumulator, Q^T from AGPRs; FIRST: the k-step that
// starts the sum (accumulator input 0); NOP2: Q^T may just have been copied
// into the AGPRs.
template <bool FIRST, bool NOP2>
__device__ __forceinline__ void mfma8_sa(f32x16& acc, const i32x8& k, const i32x8& q) {
  if constexpr (FIRST && NOP2)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=a"(acc) : "v"(k), "a"(q));
  else if constexpr (FIRST)
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=a"(acc) : "v"(k), "a"(q));
  else if constexpr (NOP2)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(k), "a"(q));
  else
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(k), "a"(q));
}
// Wait states between S's MFMAs and the VALU's reads of it.
__device__ __forceinline__ void s_fence(f32x16 (&s)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(s[0]), "+a"(s[1]), "+a"(s[2]), "+a"(s[3]));
}

// Causal work runs persistent at every head dim (at d = 256 since S moved to
// the AGPR file: +2% at B4 H16 N8192, +16% at B16 H16 N2048).
template <int D, bool CAUSAL>
constexpr bool persistent8() { return CAUSAL; }

// One workgroup's work item: query block qblk (32 * NW rows) of head bh.
template <int D, bool CAUSAL>
__device__ __forceinline__ void attend_block8(
    char* smem, const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
    const uint8_t* __restrict__ V, const float* __restrict__ SQ, const float* __restrict__ SK,
    const float* __restrict__ SV, __bf16* __restrict__ O, float* __restrict__ LSE, int H, int Hkv,
    int N, float scale_log2, int bh, int qblk) {
  using G = Geo8<D>;
  constexpr int kBR = 32 * G::NW;  // query rows per workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int hh = lane >> 5;

  const int b = bh / H;
  const int h = bh - b * H;
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = ((int64_t)b * N * H + h) * D;
  // Grouped-query attention: H / Hkv consecutive query heads read one K/V head.
  const int bhk = b * Hkv + h / (H / Hkv);
  const int64_t rs_kv = (int64_t)Hkv * D;
  const int64_t kv_off = ((int64_t)b * N * Hkv + h / (H / Hkv)) * D;
  const int nsb = (N + kQB - 1) / kQB;
  const float* sk_bh = SK + (int64_t)bhk * nsb;
  const float* sv_bh = SV + (int64_t)bhk * nsb;

  const int q0 = qblk * kBR + wave * 32;
  const int qi = q0 + li;
  const float sq = (q0 < N) ? SQ[(int64_t)bh * nsb + q0 / kQB] : 0.f;

  // Q^T as the B operand: k-step t covers dims 64t .. 64t+63; half h holds
  // dims 64t + 32h .. +31 of query qi.
  i32x8 qf[D / 64];
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    i32x8 z = {};
    qf[t] = (qi < N) ? *(const i32x8*)(Q + head_off + (int64_t)qi * rs + 64 * t + 32 * hh) : z;
  }

  // This head's K/V rows end at byte nbytes; per-tile descriptors start at the
  // tile's first row and end there, so rows n >= N read as zeros.
  const uint32_t nbytes = (uint32_t)((int64_t)(N - 1) * rs_kv + D);
  const uint8_t* kh = K + kv_off;
  const uint8_t* vh = V + kv_off;
  const uint32_t row_bytes = (uint32_t)rs_kv;
  uint32_t voff_k[G::LOADS], voff_v[G::LOADS];
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    const int chunk = (wave * G::LOADS + i) * 64 + lane;
    const int row = chunk / G::CPR, pos = chunk % G::CPR;
    voff_k[i] = row * row_bytes + (uint32_t)((pos ^ G::swz_k(row)) * 16);
    voff_v[i] = row * row_bytes + (uint32_t)((pos ^ G::swz_v(row)) * 16);
  }
#define LOAD_TILE(stage, k0)                                                                    \
  do {                                                                                          \
    const uint32_t off_ = (uint32_t)(k0) * row_bytes;                                           \
    const __amdgpu_buffer_rsrc_t rk_ = tile_rsrc(kh, off_, nbytes);                             \
    const __amdgpu_buffer_rsrc_t rv_ = tile_rsrc(vh, off_, nbytes);                             \
    _Pragma("unroll") for (int i_ = 0; i_ < G::LOADS; ++i_) {                                   \
      char* dst_ = smem + (wave * G::LOADS + i_) * 1024;                                        \
      copy_to_lds16(rk_, dst_ + G::koff(stage), voff_k[i_]);                                    \
      copy_to_lds16(rv_, dst_ + G::VBASE + G::voff(stage), voff_v[i_]);                         \
    }                                                                                           \
  } while (0)

  // K operand: row li, 16-byte chunks 4t + 2hh and 4t + 2hh + 1.
  int kaddr[D / 64][2];
#pragma unroll
  for (int t = 0; t < D / 64; ++t)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      kaddr[t][c] = li * G::RB + (((4 * t + 2 * hh + c) ^ G::swz_k(li)) * 16);
  // V^T operand, transposed read r of k-step u: source lane 2j + q of group g
  // points at key 64u + 16r + 8(j/4) + 4(g/2) + j%4, dims 32e + 16(g%2) + 8q.
  uint32_t vaddr[D / 32];  // LDS addresses relative to a V buffer (stage offset: immediate)
  {
    const int src = lane & 15, g = lane >> 4;
    const int j = src >> 1, q = src & 1;
    const int kl = 8 * (j >> 2) + 4 * (g >> 1) + (j & 3);
#pragma unroll
    for (int e = 0; e < D / 32; ++e) {
      const int c = 2 * e + (g & 1);
      vaddr[e] = lds_addr(smem) + G::VBASE + kl * G::RB + ((c ^ G::swz_v(kl)) * 16) + 8 * q;
    }
  }

  float m = kNoMax;
  float l = 0.f;
  float sv_prev = 1.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) oacc[e] = f32x16{};

  constexpr int NEH = D / 32 <= 4 ? D / 32 : 4;  // 32-dim blocks of O per half
  constexpr int NHALF = (D / 32) / NEH;
  const int nkb_all = ceil_div(N, kBC);
  const int nkb = CAUSAL ? min(nkb_all, ceil_div(min(N, (qblk + 1) * kBR), kBC)) : nkb_all;

  // Interior tiles (no key past the end, no key after any of the workgroup's
  // query rows) run a copy of the tile body without masking; the few edge
  // tiles at the end run the masked copy.  Tile kb sits in LDS stage kb % 2;
  // both loops take tiles in pairs from an even index, so ST is a
  // compile-time constant and every LDS offset an immediate.
#define TILE_BODY(ST, MASKED)                                                                        \
    const char* kt = smem + G::koff(ST);                                                             \
                                                                                                     \
    i32x8 kf[4][D / 64];                                                                             \
_Pragma("unroll")                                                                                    \
    for (int t = 0; t < D / 64; ++t)                                                                 \
_Pragma("unroll")                                                                                    \
      for (int j = 0; j < 4; ++j) {                                                                  \
        const i32x4 lo = *(const i32x4*)(kt + kaddr[t][0] + j * 32 * G::RB);                         \
        const i32x4 hi = *(const i32x4*)(kt + kaddr[t][1] + j * 32 * G::RB);                         \
        kf[j][t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};                    \
      }                                                                                              \
    f32x16 sacc[4];                                                                                  \
_Pragma("unroll")                                                                                    \
    for (int j = 0; j < 4; ++j) sacc[j] = f32x16{};                                                  \
_Pragma("unroll")                                                                                    \
    for (int t = 0; t < D / 64; ++t)                                                                 \
_Pragma("unroll")                                                                                    \
      for (int j = 0; j < 4; ++j) sacc[j] = mfma_fp8(kf[j][t], qf[t], sacc[j]);                      \
                                                                                                     \
    /* d <= 128, non-causal: the V^T operands are read now, so that the softmax     */           \
    /* covers their latency (in the causal kernel they would not fit the registers) */           \
    i32x8 vf0[2][NEH];                                                                               \
    if constexpr (NHALF == 1 && !CAUSAL) read_vt<D, ST, NEH>(vaddr, vf0);                            \
    if (MASKED) mask_s8(sacc, k0, N, CAUSAL, qi, hh);                                                \
                                                                                                     \
    const float c_tile = scale_log2 * sq * sk_bh[kb];                                                \
    const float sv = sv_bh[kb];                                                                      \
    /* four chains of three-input maxima (v_max3), one per 32-key block */                          \
    float mxj[4];                                                                                    \
_Pragma("unroll")                                                                                    \
    for (int j = 0; j < 4; ++j) {                                                                    \
      mxj[j] = fmaxf(sacc[j][0], sacc[j][1]);                                                        \
_Pragma("unroll")                                                                                    \
      for (int v = 2; v < 16; v += 2) mxj[j] = fmaxf(fmaxf(mxj[j], sacc[j][v]), sacc[j][v + 1]);     \
    }                                                                                                \
    const float mx = max_halves(fmaxf(fmaxf(mxj[0], mxj[1]), fmaxf(mxj[2], mxj[3])));                \
    const float m_new = fmaxf(m, mx * c_tile);                                                       \
    const float alpha = exp2_fast(m - m_new);                                                        \
    m = m_new;                                                                                       \
    const float neg_m = -m;                                                                          \
    float rs4[4] = {0.f, 0.f, 0.f, 0.f}; /* four partial sums: short dependency chains */           \
    i32x8 pf[2];                                                                                     \
_Pragma("unroll")                                                                                    \
    for (int u = 0; u < 2; ++u)                                                                      \
_Pragma("unroll")                                                                                    \
      for (int w = 0; w < 8; ++w) {                                                                  \
        const f32x16& sa = sacc[2 * u + (w >> 2)];                                                   \
        const int r0 = 4 * (w & 3);                                                                  \
        float p[4];                                                                                  \
_Pragma("unroll")                                                                                    \
        for (int i = 0; i < 4; ++i) {                                                                \
          p[i] = exp2_fast(__builtin_fmaf(sa[r0 + i], c_tile, neg_m));                               \
          rs4[i] += p[i];                                                                            \
        }                                                                                            \
        pf[u][w] = (int)pack_fp8x4(p[0], p[1], p[2], p[3]);                                          \
      }                                                                                              \
    l = l * alpha + ((rs4[0] + rs4[1]) + (rs4[2] + rs4[3]));                                         \
    /* hardware reciprocal (1 ulp): the ratio only rescales the fp32 accumulator */                \
    const float f = alpha * (sv_prev * __builtin_amdgcn_rcpf(sv));                                   \
    sv_prev = sv;                                                                                    \
    o8_fence<D>(oacc);                                                                               \
_Pragma("unroll")                                                                                    \
    for (int e = 0; e < D / 32; ++e) oacc[e] *= f;                                                   \
                                                                                                     \
    if constexpr (NHALF == 1 && !CAUSAL) {                                                           \
      /* the early reads: waited for in place (no copy of a register in flight) */                 \
      lds_wait_v(vf0);                                                                               \
_Pragma("unroll")                                                                                    \
      for (int u = 0; u < 2; ++u)                                                                    \
_Pragma("unroll")                                                                                    \
        for (int e = 0; e < NEH; ++e) oacc[e] = mfma_fp8(vf0[u][e], pf[u], oacc[e]);                 \
      static_assert(D <= 128, "early V^T reads at d <= 128 only");                                   \
    } else {                                                                                         \
      /* V^T operands in halves of at most four 32-dim blocks (d = 256: two) */                    \
_Pragma("unroll")                                                                                    \
      for (int hf = 0; hf < NHALF; ++hf) {                                                           \
        i32x8 vf[2][NEH];                                                                            \
        read_vt<D, ST, NEH>(vaddr + hf * NEH, vf);                                                   \
        lds_wait_v(vf);                                                                              \
        static_for<2>([&](auto U_) {                                                                 \
          constexpr int u = decltype(U_)::value;                                                     \
          static_for<NEH>([&](auto E_) {                                                             \
            constexpr int e = decltype(E_)::value;                                                   \
            pv8<D, u == 0 || e == 0>(oacc[hf * NEH + e], vf[u][e], pf[u]);                           \
          });                                                                                        \
        });                                                                                          \
      }                                                                                              \
    }                                                                                                \

#define STEP8(ST, KB, MASKED)                                                                        \
  do {                                                                                               \
    const int kb = (KB);                                                                             \
    const int k0 = kb * kBC;                                                                         \
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                                 \
    __syncthreads(); /* tile kb resident; every wave is done with the other stage */                 \
    if (kb + 1 < nkb) LOAD_TILE((ST) ^ 1, k0 + kBC);                                                 \
    if (!(CAUSAL && k0 > q0 + 31)) { /* else the tile is after all of this wave's rows */            \
      TILE_BODY(ST, MASKED)                                                                          \
    }                                                                                                \
  } while (0)
  const int nkb_int = min(nkb, min(CAUSAL ? qblk * (kBR / kBC) : nkb, N / kBC)) & ~1;

  int kb2 = 0;
  if constexpr (D > 128) {
    if (nkb_int >= 2) {
      namespace P8 = fpipe8;
      const int nint = nkb_int;
      const uint32_t lbase = lds_addr(smem);
      uint32_t kad[D / 64][2];
#pragma unroll
      for (int t = 0; t < D / 64; ++t) {
        kad[t][0] = lbase + (uint32_t)kaddr[t][0];
        kad[t][1] = lbase + (uint32_t)kaddr[t][1];
      }
      auto load_k = [&](int slot, int k0) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(kh, (uint32_t)k0 * row_bytes, nbytes);
#pragma unroll
        for (int i = 0; i < G::LOADS; ++i)
          copy_to_lds16(r, smem + (wave * G::LOADS + i) * 1024 + G::koff(slot), voff_k[i]);
      };
      auto load_v = [&](int slot, int k0) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(vh, (uint32_t)k0 * row_bytes, nbytes);
#pragma unroll
        for (int i = 0; i < G::LOADS; ++i)
          copy_to_lds16(r, smem + (wave * G::LOADS + i) * 1024 + G::VBASE + G::voff(slot), voff_v[i]);
      };
      load_k(0, 0);
      load_v(0, 0);
      load_k(1, kBC);
      // K(0) landed (V(0) and K(1) may still be in flight: S(0) overlaps them)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * G::LOADS) : "memory");
      __builtin_amdgcn_s_barrier();
      f32x16 sA[4], sB[4];
      // S(0) = K(0) Q^T (K slot 0), then its row max
      {
        i32x4 klo[P8::NS], khi[P8::NS];
        auto rd = [&](auto I) __attribute__((always_inline)) {
          constexpr int i = decltype(I)::value, jb = i % 4, t = i / 4;
          klo[i] = read_k16<G::koff(0) + jb * 32 * G::RB>(kad[t][0]);
          khi[i] = read_k16<G::koff(0) + jb * 32 * G::RB>(kad[t][1]);
        };
        constexpr int AHEAD = 4;
        static_for<AHEAD>(rd);
        static_for<P8::NS>([&](auto I) __attribute__((always_inline)) {
          constexpr int i = decltype(I)::value, jb = i % 4, t = i / 4;
          constexpr int nis = (AHEAD + i < P8::NS) ? AHEAD + i : P8::NS;
          asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(klo[i]), "+v"(khi[i]) : "n"(2 * (nis - i - 1)));
          const i32x8 kf = i32x8{klo[i][0], klo[i][1], klo[i][2], klo[i][3],
                                 khi[i][0], khi[i][1], khi[i][2], khi[i][3]};
          mfma8_sa<t == 0, jb == 0>(sA[jb], kf, qf[t]);
          if constexpr (i + AHEAD < P8::NS) rd(IC<i + AHEAD>{});
        });
      }
      s_fence(sA);
      float mx;
      {
        float mxj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          mxj[j] = fmaxf(sA[j][0], sA[j][1]);
#pragma unroll
          for (int v = 2; v < 16; v += 2) mxj[j] = fmaxf(fmaxf(mxj[j], sA[j][v]), sA[j][v + 1]);
        }
        mx = max_halves(fmaxf(fmaxf(mxj[0], mxj[1]), fmaxf(mxj[2], mxj[3])));
      }
      // Softmax of tile kb on S(kb) (cur, AGPRs) up to the rescale factor:
      // the same operations as the same-phase body.
      // Tile kb's block scales were loaded at the end of the previous
      // iteration (prefetch below); their scalar-load wait comes here, right
      // after the barrier, with no LDS read in flight.
      float skp = sk_bh[0], svp = sv_bh[0];
      auto head = [&](int kb, float& c_tile, float& alpha, float& f) __attribute__((always_inline)) {
        (void)kb;
        float skc = skp, svc = svp;
        asm volatile("" : "+s"(skc), "+s"(svc));
        c_tile = scale_log2 * sq * skc;
        const float sv = svc;
        const float m_new = fmaxf(m, mx * c_tile);
        alpha = exp2_fast(m - m_new);
        m = m_new;
        f = alpha * (sv_prev * __builtin_amdgcn_rcpf(sv));
        sv_prev = sv;
      };
      // Iteration j: K slot SK holds K(j+1), V slot SV holds V(j); cur = S(j),
      // nxt receives S(j+1).
      auto iter = [&](auto SK_, auto SV_, f32x16 (&cur)[4], f32x16 (&nxt)[4], int j)
                      __attribute__((always_inline)) {
        constexpr int SK = decltype(SK_)::value, SV = decltype(SV_)::value;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // K(j+1), V(j) landed; every wave is done with K(j), V(j-1)
        // the next tiles' copies go out one per slot in slots 0 .. 15
        const __amdgpu_buffer_rsrc_t rkn = tile_rsrc(kh, (uint32_t)min(j + 2, nint - 1) * kBC * row_bytes, nbytes);
        const __amdgpu_buffer_rsrc_t rvn = tile_rsrc(vh, (uint32_t)(j + 1) * kBC * row_bytes, nbytes);
        const bool kn = j + 2 < nint;
        float c_tile, alpha, f;
        head(j, c_tile, alpha, f);
        const float neg_m = -m;
        o8_fence<D>(oacc);  // P.V(j-1) -> the rescale
        float rs4[4] = {0.f, 0.f, 0.f, 0.f};
        float pe[64];
        i32x8 pf[2];
        i32x4 klo[P8::NS], khi[P8::NS];
        i32x2 vr[P8::NP][4];
        float mxj[4];
        auto issue = [&](auto R_) __attribute__((always_inline)) {
          constexpr int r = decltype(R_)::value;
          if constexpr (r < 2 * P8::NS) {
            constexpr int i = r / 2, jb = i % 4, t = i / 4;
            if constexpr (r % 2 == 0) klo[i] = read_k16<G::koff(SK) + jb * 32 * G::RB>(kad[t][0]);
            else khi[i] = read_k16<G::koff(SK) + jb * 32 * G::RB>(kad[t][1]);
          } else {
            constexpr int k = (r - 2 * P8::NS) / 4, q = (r - 2 * P8::NS) % 4, u = k / 8, e = k % 8;
            vr[k][q] = read_tr8<G::voff(SV) + 16 * (4 * u + q) * G::RB>(vaddr[e]);
          }
        };
        static_for<P8::N>([&](auto S_) __attribute__((always_inline)) {
          constexpr int s = decltype(S_)::value;
          if constexpr (s == 0) {
            static_for<P8::kLook + 1>([&](auto K_) __attribute__((always_inline)) {
              issue(IC<decltype(K_)::value>{});
            });
          }
          constexpr int W = P8::issued(s - 1) - P8::need(s);
          static_assert(W >= 0 && W <= 15, "wait count");
          if constexpr (s < P8::NS) {
            constexpr int jb = s % 4, t = s / 4;
            asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(klo[s]), "+v"(khi[s]) : "n"(W));
            const i32x8 kf = i32x8{klo[s][0], klo[s][1], klo[s][2], klo[s][3],
                                   khi[s][0], khi[s][1], khi[s][2], khi[s][3]};
            mfma8_sa<t == 0, jb == 0>(nxt[jb], kf, qf[t]);
          } else {
            constexpr int k = s - P8::NS, u = k / 8, e = k % 8;
            asm volatile("s_waitcnt lgkmcnt(%4)"
                         : "+v"(vr[k][0]), "+v"(vr[k][1]), "+v"(vr[k][2]), "+v"(vr[k][3])
                         : "n"(W));
            const i32x8 vf = i32x8{vr[k][0][0], vr[k][0][1], vr[k][1][0], vr[k][1][1],
                                   vr[k][2][0], vr[k][2][1], vr[k][3][0], vr[k][3][1]};
            mfma8_v<true>(oacc[e], vf, pf[u]);
          }
          constexpr int first = P8::issued(s - 1) + 1;
          static_for<P8::issued(s) - P8::issued(s - 1)>([&](auto K_) __attribute__((always_inline)) {
            issue(IC<first + decltype(K_)::value>{});
          });
          if constexpr (s < 2 * G::LOADS) {
            constexpr int i = s % G::LOADS;
            if constexpr (s < G::LOADS) {
              if (kn) copy_to_lds16(rkn, smem + (wave * G::LOADS + i) * 1024 + G::koff(SV), voff_k[i]);
            } else {
              copy_to_lds16(rvn, smem + (wave * G::LOADS + i) * 1024 + G::VBASE + G::voff(SK), voff_v[i]);
            }
          }
          // O^T block e = s / 2 rescaled (half of it per slot)
          if constexpr (s < 16) {
            constexpr int e = s / 2, h0 = 8 * (s % 2);
#pragma unroll
            for (int v = h0; v < h0 + 8; ++v) oacc[e][v] *= f;
          }
          // exponentials of S(j), in the same-phase body's order
          static_for<64>([&](auto V_) __attribute__((always_inline)) {
            constexpr int v = decltype(V_)::value;
            if constexpr (P8::exp_slot(v) == s) {
              constexpr int u = v / 32, w = (v % 32) / 4, i = v % 4;
              constexpr int blk = 2 * u + (w >> 2), r0 = 4 * (w & 3);
              pe[v] = exp2_fast(__builtin_fmaf(cur[blk][r0 + i], c_tile, neg_m));
              rs4[i] += pe[v];
              if constexpr (i == 3) {
                pf[u][w] = (int)pack_fp8x4(pe[v - 3], pe[v - 2], pe[v - 1], pe[v]);
                asm volatile("" : "+v"(rs4[0]), "+v"(rs4[1]), "+v"(rs4[2]), "+v"(rs4[3]), "+v"(pf[u][w]));
              } else {
                asm volatile("" : "+v"(pe[v]));
              }
            }
          });
          // S(j+1)'s row max, eight values per slot
          if constexpr (s >= P8::kMax0) {
            constexpr int b = (s - P8::kMax0) / 2, h = 8 * ((s - P8::kMax0) % 2);
            if constexpr (s == P8::kMax0) s_fence(nxt);
            float x = h == 0 ? fmaxf(nxt[b][0], nxt[b][1]) : fmaxf(mxj[b], fmaxf(nxt[b][h], nxt[b][h + 1]));
#pragma unroll
            for (int v = h + 2; v < h + 8; v += 2) x = fmaxf(fmaxf(x, nxt[b][v]), nxt[b][v + 1]);
            mxj[b] = x;
            asm volatile("" : "+v"(mxj[b]));
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        l = l * alpha + ((rs4[0] + rs4[1]) + (rs4[2] + rs4[3]));
        mx = max_halves(fmaxf(fmaxf(mxj[0], mxj[1]), fmaxf(mxj[2], mxj[3])));
        skp = sk_bh[j + 1];  // the next tile's scales (tile j + 1 <= nint - 1 exists)
        svp = sv_bh[j + 1];
      };
      int j = 0;
      for (; j + 2 < nint - 1; j += 2) {
        iter(IC<1>{}, IC<0>{}, sA, sB, j);
        iter(IC<0>{}, IC<1>{}, sB, sA, j + 1);
      }
      iter(IC<1>{}, IC<0>{}, sA, sB, nint - 2);
      // The last interior tile: softmax of S(nint-1) (in sB) and its P.V, V in
      // slot (nint-1) % 2 = 1.
      {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        float c_tile, alpha, f;
        head(nint - 1, c_tile, alpha, f);
        const float neg_m = -m;
        float rs4[4] = {0.f, 0.f, 0.f, 0.f};
        i32x8 pf[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const f32x16& sa = sB[2 * u + (w >> 2)];
            const int r0 = 4 * (w & 3);
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              p[i] = exp2_fast(__builtin_fmaf(sa[r0 + i], c_tile, neg_m));
              rs4[i] += p[i];
            }
            pf[u][w] = (int)pack_fp8x4(p[0], p[1], p[2], p[3]);
          }
        l = l * alpha + ((rs4[0] + rs4[1]) + (rs4[2] + rs4[3]));
        o8_fence<D>(oacc);
#pragma unroll
        for (int e = 0; e < D / 32; ++e) oacc[e] *= f;
        constexpr int NEH = 4;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          i32x8 vf[2][NEH];
          read_vt<D, 1, NEH>(vaddr + hf * NEH, vf);
          lds_wait_v(vf);
          static_for<2>([&](auto U_) {
            constexpr int u = decltype(U_)::value;
            static_for<NEH>([&](auto E_) {
              constexpr int e = decltype(E_)::value;
              pv8<D, true>(oacc[hf * NEH + e], vf[u][e], pf[u]);
            });
          });
        }
      }
      __syncthreads();  // every wave is done with the pipelined loop's tiles
      kb2 = nint;
    }
  }
  if (kb2 < nkb) LOAD_TILE(0, kb2 * kBC);
  for (; kb2 < nkb_int; kb2 += 2) {
    STEP8(0, kb2, false);
    STEP8(1, kb2 + 1, false);
  }
  for (; kb2 < nkb; kb2 += 2) {
    STEP8(0, kb2, true);
    if (kb2 + 1 < nkb) STEP8(1, kb2 + 1, true);
  }
#undef STEP8
#undef LOAD_TILE
#undef TILE_BODY

  // Epilogue.  Non-causal: bf16 rows stored whole through LDS (every wave is
  // done with the K/V tiles after the barrier; each wave takes 32 * 2D bytes
  // of them).  Causal: stored from the accumulator layout directly (the staged
  // store measured 3% slower in the persistent causal kernel).
  const float lt = sum_halves(l);
  const float inv = sv_prev / lt;
  o8_fence<D>(oacc);
  if constexpr (!CAUSAL) {
    static_assert(G::NW * 32 * 2 * D <= 2 * G::STAGE, "the output rows are staged in the tile buffers");
    __syncthreads();
    store_rows_via_lds<D>(smem + wave * 32 * (2 * D), oacc, inv, O, head_off, rs, q0, N, lane);
    if (qi < N && LSE != nullptr && hh == 0) LSE[(int64_t)bh * N + qi] = (m + __log2f(lt)) * kLn2;
  } else {
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
}

// Non-causal: one workgroup per (b, h, query block); with xcd_remap the
// query heads of one K/V head run on one XCD, and XCD x takes the K/V head
// groups x, x + 8, ...
// Causal: as the bf16 kernel, persistent slots over units of
// two query blocks (nqb-1-p, p) of equal total cost when nunits > 0, one
// workgroup per block (heaviest first) when nunits == 0.  (The report's
// section 5.1 lists the persistent kernel as not yet joined with its FP8
// kernel; here both forwards share the schedule.)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * waves<D>(), 1) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ SQ, const float* __restrict__ SK, const float* __restrict__ SV,
    __bf16* __restrict__ O, float* __restrict__ LSE, int H, int Hkv, int N, float scale_log2,
    int nqb, int xcd_remap, int nunits) {
  using G = Geo8<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * G::STAGE];
  if constexpr (!persistent8<D, CAUSAL>()) {
    // With xcd_remap, XCD x (the hardware deals workgroups round robin) takes
    // the K/V head groups x, x + 8, ..., all query blocks of a group together.
    const int L = blockIdx.x;
    int bh, qb;
    if (xcd_remap) {
      const int g = H / Hkv, x = L & 7, j = L >> 3, rem = j % (g * nqb);
      bh = ((j / (g * nqb)) * 8 + x) * g + rem / nqb;
      qb = rem % nqb;
    } else {
      bh = L / nqb;
      qb = L % nqb;
    }
    attend_block8<D, CAUSAL>(smem, Q, K, V, SQ, SK, SV, O, LSE, H, Hkv, N, scale_log2, bh,
                             CAUSAL ? nqb - 1 - qb : qb);
  } else {
    const int npair = (nqb + 1) / 2;
    const int nslot = nunits > 0 ? nunits : (int)gridDim.x;
    int s = blockIdx.x, second = 0;
#pragma nounroll
    while (s < nslot) {
      // Work items per query head: units (pairs) or single blocks; with
      // xcd_remap, slot s stays on XCD s % 8, which takes the K/V head groups
      // x, x + 8, ... as above.
      const int per = nunits > 0 ? npair : nqb;
      int bh, item, qblk, last = 1;
      if (xcd_remap) {
        const int g = H / Hkv, x = s & 7, j = s >> 3, rem = j % (g * per);
        bh = ((j / (g * per)) * 8 + x) * g + rem / per;
        item = rem % per;
      } else {
        bh = s / per;
        item = s % per;
      }
      if (nunits > 0) {
        qblk = second ? item : nqb - 1 - item;
        last = second || item == nqb - 1 - item;
      } else {
        qblk = nqb - 1 - item;
      }
      attend_block8<D, CAUSAL>(smem, Q, K, V, SQ, SK, SV, O, LSE, H, Hkv, N, scale_log2, bh, qblk);
      if (last) {
        second = 0;
        s += gridDim.x;
      } else {
        second = 1;
      }
      __syncthreads();  // every wave is done with this block's LDS tiles
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk,
                  const float* sv, void* o, float* lse, int B, int H, int Hkv, int N,
                  float scale, hipStream_t stream) {
  constexpr int kBR = 32 * waves<D>();
  const int nqb = (N + kBR - 1) / kBR;
  int64_t grid = (int64_t)B * H * nqb;
  int64_t nunits = 0;
  if constexpr (persistent8<D, CAUSAL>()) {
    const int64_t units = (int64_t)B * H * ((nqb + 1) / 2);
    static std::atomic<int> resident{0};
    const int ncu = current_cu_count();
    const int per_cu = resident_per_cu(attn_fwd_fp8_kernel<D, CAUSAL>, 64 * waves<D>(), resident);
    if (ncu <= 0 || per_cu <= 0) return hipErrorInvalidDevice;
    const int64_t slots = (int64_t)ncu * per_cu;  // resident workgroups
    // persistent only with more blocks than CUs and when the equal units
    // fill the slots in whole rounds (last round at least 90% full)
    const int64_t rounds = (units + slots - 1) / slots;
    if (grid > ncu && (units <= slots || units * 10 >= rounds * slots * 9)) {
      nunits = units;
      grid = units < slots ? units : slots;
    }
  }
  // the K/V head groups (B * Hkv of them) split evenly over the 8 XCDs, and a
  // persistent grid a multiple of 8 (each slot stays on one XCD)
  const int remap = (((int64_t)B * Hkv) % 8 == 0 && grid % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(64 * waves<D>()), 0,
                     stream, (const uint8_t*)q8, (const uint8_t*)k8, (const uint8_t*)v8, sq, sk, sv,
                     (__bf16*)o, lse, H, Hkv, N, scale * kLog2e, nqb, remap, (int)nunits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* sq,
                               const float* sk, const float* sv, void* o, float* lse, int B, int H,
                               int Hkv, int N, int d, bool causal, float softmax_scale,
                               hipStream_t stream) {
  if (d == 256)
    return causal ? launch<256, true>(q8, k8, v8, sq, sk, sv, o, lse, B, H, Hkv, N, softmax_scale, stream)
                  : launch<256, false>(q8, k8, v8, sq, sk, sv, o, lse, B, H, Hkv, N, softmax_scale, stream);
  if (d == 128)
    return causal ? launch<128, true>(q8, k8, v8, sq, sk, sv, o, lse, B, H, Hkv, N, softmax_scale, stream)
                  : launch<128, false>(q8, k8, v8, sq, sk, sv, o, lse, B, H, Hkv, N, softmax_scale, stream);
  return causal ? launch<64, true>(q8, k8, v8, sq, sk, sv, o, lse, B, H, Hkv, N, softmax_scale, stream)
                : launch<64, false>(q8, k8, v8, sq, sk, sv, o, lse, B, H, Hkv, N, softmax_scale, stream);
}

}  // namespace exattn
