// bf16 exact-attention gradients (dQ, dK, dV) for gfx950.
//
// The backward pass of the FlashAttention-3 report (section 3.4) keeps FA-2's
// strategy: P is recomputed from Q, K and the saved log-sum-exp instead of
// being stored.  Per (b, h), with O and dO the forward output and its
// gradient:
//   D_i = sum_c dO[i, c] O[i, c]
//   P   = exp(scale Q K^T - LSE)            (causal: 0 for key > query)
//   dV  = P^T dO
//   dS  = P * (dO V^T - D)                   (D per query row)
//   dQ  = scale dS K,   dK = scale dS^T Q
//
// Three kernels, launched in order on one stream:
//   bwd_prep   D and LSE * log2(e) per query row, into the caller's workspace.
//   bwd_dkdv   one workgroup per (b, h, 128 keys); each wave keeps its 32 keys'
//              K^T and V^T in registers and streams 64-row Q and dO tiles
//              (with their LSE and D) through LDS.  S = Q K^T and dP = dO V^T
//              put one key on each MFMA column, so P and dS go straight from
//              the accumulator into dV^T += dO^T P and dK^T += Q^T dS as the
//              B operand, with dO^T and Q^T gathered by transposed LDS reads
//              in the accumulator's row order (the forward's P^T relayout,
//              with keys and queries exchanged).
//   bwd_dq     one workgroup per (b, h, 128 queries), the forward kernel's
//              layout: S^T = K Q^T and dP^T = V dO^T with Q^T, dO^T in
//              registers, then dQ^T += K^T dS^T from transposed reads of K.
// dQ gets its own kernel instead of fp32 atomics across key blocks: S and dP
// are computed twice (seven matrix products instead of five) and every
// result is deterministic.
//
// LDS tiles are 64 rows, copied by buffer_load ... lds (rows past the end of
// the sequence read as zeros) and double-buffered, as in the forward.  A tile
// that is read both row-wise (ds_read_b128, an A operand) and transposed
// (ds_read_b64_tr_b16) uses the chunk swizzle swz_b, free of bank conflicts
// for both patterns.
#include <mutex>

#include "common.h"
#include "exattn.h"
#include "launch.h"
#include "lds_tile.h"

namespace exattn {
namespace {

constexpr int kNWb = 4;           // waves per workgroup (both gradient kernels)
constexpr int kRowsB = 32 * kNWb;  // query rows (dQ) or key rows (dK, dV) per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_wait_f4(f32x4 (&a)[4], f32x4 (&b)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                 "+v"(b[2]), "+v"(b[3]));
}

template <int OFF>
__device__ __forceinline__ f32x4 read_f4(uint32_t addr) {
  f32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Transposed-read A-operand fragments for the 32 rows [32 J, 32 J + 32) of the
// tile at LDS offset OFF (swizzle swz_b): frag[T][e] covers rows 32 J + 16 T ..
// +15 (k) and d-rows 32 e .. 32 e + 31, in the accumulator's row order (row
// 16 T + 8 (s / 4) + 4 h + s % 4 in k-slot s of half-wave h).  Rows + 8 and
// + 24 sit at the address XOR 32 (swz_b(row + 8) = swz_b(row) ^ 2).
template <int D, int OFF, int J>
__device__ __forceinline__ void read_tr_frags(const uint32_t (&taddr)[D / 32],
                                              bf16x8 (&frag)[2][D / 32]) {
  using G = Geo<D>;
#pragma unroll
  for (int e = 0; e < D / 32; ++e) {
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      constexpr int R0 = 32 * J;
      const bf16x4 lo = T == 0 ? read_tr16<OFF + (R0 + 0) * G::RB>(taddr[e])
                               : read_tr16<OFF + (R0 + 16) * G::RB>(taddr[e]);
      const bf16x4 hi = T == 0 ? read_tr16<OFF + (R0 + 8) * G::RB>(taddr[e] ^ 32u)
                               : read_tr16<OFF + (R0 + 24) * G::RB>(taddr[e] ^ 32u);
      frag[T][e] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
}

// S-type product over the NF fragments of a group of row reads just issued
// (one ds_read_b128 each, in order t = 0 .. NF-1): each MFMA waits only for
// its own fragment, since LDS reads complete in issue order.
template <int NF>
__device__ __forceinline__ f32x16 mfma_rows_counted(bf16x8 (&f)[NF], const bf16x8 (&b)[NF]) {
  f32x16 acc = {};
  static_for<NF>([&](auto T) __attribute__((always_inline)) {
    constexpr int t = decltype(T)::value;
    wait_lds<NF - 1 - t>(f[t]);
    acc = mfma_bf16(f[t], b[t], acc);
  });
  return acc;
}

// acc[e] += frag[T][e] x b[T] (T = 0, 1) for the fragments read_tr_frags has
// just issued (two reads per (T, e), e-major), each MFMA waiting only for its
// own two reads; per accumulator the order stays T = 0, 1.
template <int NE>
__device__ __forceinline__ void mfma_tr_counted(bf16x8 (&frag)[2][NE], const bf16x8 (&b)[2],
                                                f32x16 (&acc)[NE]) {
  static_for<NE>([&](auto E) __attribute__((always_inline)) {
    constexpr int e = decltype(E)::value;
    static_for<2>([&](auto TT) __attribute__((always_inline)) {
      constexpr int T = decltype(TT)::value;
      wait_lds<4 * NE - 2 - (4 * e + 2 * T)>(frag[T][e]);
      acc[e] = mfma_bf16(frag[T][e], b[T], acc[e]);
    });
  });
}

// The same eight products for NE = 4 as one block of assembly on accumulators
// held in AGPRs (dV^T and dK^T stay in the AGPR file for the whole kernel, so
// the S and dP products and the softmax keep the 256 VGPRs).  Each MFMA waits
// only for its own two reads (LDS reads complete in issue order); the leading
// s_nop gives the two wait states an MFMA needs after a VALU write of its B
// operand.  Back-to-back products on one accumulator need no wait states.
__device__ __forceinline__ void mfma_tr_agpr4(bf16x8 (&f)[2][4], const bf16x8 (&b)[2],
                                              f32x16 (&acc)[4]) {
  asm volatile(
      "s_waitcnt lgkmcnt(14)\n\t"
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %12, %0\n\t"
      "s_waitcnt lgkmcnt(12)\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %13, %0\n\t"
      "s_waitcnt lgkmcnt(10)\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %6, %12, %1\n\t"
      "s_waitcnt lgkmcnt(8)\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %7, %13, %1\n\t"
      "s_waitcnt lgkmcnt(6)\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %8, %12, %2\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %9, %13, %2\n\t"
      "s_waitcnt lgkmcnt(2)\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %10, %12, %3\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %11, %13, %3"
      : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3])
      : "v"(f[0][0]), "v"(f[1][0]), "v"(f[0][1]), "v"(f[1][1]), "v"(f[0][2]), "v"(f[1][2]),
        "v"(f[0][3]), "v"(f[1][3]), "v"(b[0]), "v"(b[1]));
}

// Wait states between the AGPR accumulators' last MFMA (or their zeroing
// writes) and any other instruction that touches them.
__device__ __forceinline__ void agpr_fence(f32x16 (&a)[4], f32x16 (&b)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(b[0]), "+a"(b[1]),
                 "+a"(b[2]), "+a"(b[3]));
}

// Read stream of the software-pipelined head-dim-128 tile body: per 32-query
// block, 56 LDS reads in this order
//   [0, 8)   Q row fragments (A operands of S = Q K^T, one per MFMA)
//   [8, 12)  LSE * log2(e) of the block's rows
//   [12, 20) dO row fragments (A operands of dP = dO V^T)
//   [20, 24) D of the block's rows
//   [24, 40) dO^T transposed halves (two per dV^T MFMA)
//   [40, 56) Q^T transposed halves (two per dK^T MFMA)
// and 32 MFMA slots: S (8), dP (8), dV^T (8), dK^T (8).  Slot s needs the
// stream up to need(s).  A prologue issues reads 0 .. kLook; slot s issues,
// right after its MFMA, the reads up to issued(s) = need(s) + kLook, so at
// slot s's wait the reads up to issued(s - 1) are in flight and the wait is
// lgkmcnt(issued(s - 1) - need(s)) (LDS reads complete in issue order).  The
// LSE and D reads precede the first dP and dV reads, so the waits of those
// slots cover them too.  Each slot runs: wait, MFMA, the reads ahead, then
// its VALU work: an MFMA's first cycles after issue take LDS and scalar
// instructions better than VALU ones (measured: 16 slots of MFMA + 5 VALU +
// one read took 932 cycles with the VALU right after the MFMA, 812 with the
// read first).
namespace pipe128 {
constexpr int kRPB = 56;
constexpr int kLast = 2 * kRPB - 1;  // two blocks per 64-row tile
constexpr int kLook = 8;
constexpr int need(int s) {
  return (s / 32) * kRPB + ((s % 32) < 8    ? (s % 32)
                            : (s % 32) < 16 ? 12 + (s % 32 - 8)
                            : (s % 32) < 24 ? 24 + 2 * (s % 32 - 16) + 1
                                            : 40 + 2 * (s % 32 - 24) + 1);
}
constexpr int issued(int s) {
  return s < 0 ? kLook : (need(s) + kLook < kLast ? need(s) + kLook : kLast);
}
static_assert(issued(63) == kLast, "every read is issued");
}  // namespace pipe128

template <int N>
__device__ __forceinline__ void wait_lds_pair(bf16x4& a, bf16x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void wait_lds_rows(bf16x8& x, f32x4 (&r)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%5)"
               : "+v"(x), "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3])
               : "n"(N));
}
template <int N>
__device__ __forceinline__ void wait_lds_pair_rows(bf16x4& a, bf16x4& b, f32x4 (&r)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%6)"
               : "+v"(a), "+v"(b), "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3])
               : "n"(N));
}

// acc += a x b on an AGPR accumulator (one dV^T or dK^T product); NOP2 puts
// the two wait states an MFMA needs after a VALU write of its B operand.
template <bool NOP2>
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (NOP2)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// LDS address of this lane's transposed-read source in a tile at LDS byte
// address `base` (rows key-major, chunk swizzle swz_b): row 4 hv + j, chunk
// 4 e + 2 (g % 2) + q / 2, half q % 2.
template <int D>
__device__ __forceinline__ void tr_addresses(uint32_t base, int lane, uint32_t (&taddr)[D / 32]) {
  using G = Geo<D>;
  const int src = lane & 15, g = lane >> 4;
  const int j = src >> 2, q = src & 3, hv = g >> 1;
  const int row = 4 * hv + j;
#pragma unroll
  for (int e = 0; e < D / 32; ++e) {
    const int c = 4 * e + 2 * (g & 1) + (q >> 1);
    taddr[e] = base + row * G::RB + ((c ^ G::swz_b(row)) * 16) + (q & 1) * 8;
  }
}

// Global -> LDS copy offsets of this lane's chunks of a 64-row tile, for a
// layout with chunk swizzle SWZ (0: swz_k, 1: swz_b).
template <int D, int LOADS, int SWZ>
__device__ __forceinline__ void copy_offsets(int wave, int lane, uint32_t row_bytes,
                                             uint32_t (&voff)[LOADS]) {
  using G = Geo<D>;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int chunk = (wave * LOADS + i) * 64 + lane;
    const int row = chunk / G::CPR, pos = chunk % G::CPR;
    const int sw = SWZ ? G::swz_b(row) : G::swz_k(row);
    voff[i] = row * row_bytes + (uint32_t)((pos ^ sw) * 16);
  }
}

// ---------------------------------------------------------------------------
// D_i = sum_c dO[i, c] O[i, c] and LSE_i * log2(e); D / 8 lanes per row.
// Rows are taken in [B, H, N] order (the order of D and the LSE), so a
// workgroup's D and LSE stores are contiguous and coalesced; each row's O and
// dO reads are whole rows of the BSHD tensors (2 D bytes each).
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const __bf16* __restrict__ O,
                                                       const __bf16* __restrict__ dO,
                                                       const float* __restrict__ LSE,
                                                       float* __restrict__ Drow,
                                                       float* __restrict__ L2, int H, int N,
                                                       int64_t rows) {
  constexpr int LPR = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;  // [B, H, N] index
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (idx < rows) {
    const int64_t n = idx % N, bh = idx / N;
    const int64_t h = bh % H, b = bh / H;
    const int64_t r = (b * N + n) * H + h;  // BSHD row
    const bf16x8 o = *(const bf16x8*)(O + r * D + 8 * c);
    const bf16x8 g = *(const bf16x8*)(dO + r * D + 8 * c);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf((float)o[i], (float)g[i], acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m, 64);
  if (idx < rows && c == 0) {
    Drow[idx] = acc;
    L2[idx] = LSE[idx] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dQ: the forward kernel's layout.  Stage: K tile (swz_b: read as the S^T A
// operand and transposed for K^T), V tile (swz_k: read as the dP^T A operand).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kNWb, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Drow,
    __bf16* __restrict__ dQ, int H, int Hkv, int N, float scale_log2, float scale, int nqb,
    int xcd_remap) {
  using G = Geo<D>;
  constexpr int NF = D / 16, NE = D / 32;
  constexpr int LOADS = G::TILE / (1024 * kNWb);
  __shared__ __attribute__((aligned(1024))) char smem[2 * G::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  int L = blockIdx.x;
  if (xcd_remap) L = (L & 7) * (gridDim.x >> 3) + (L >> 3);
  const int qb_raw = L % nqb, bh = L / nqb;
  const int qblk = CAUSAL ? (nqb - 1 - qb_raw) : qb_raw;  // heaviest causal blocks first
  const int b = bh / H, h = bh - b * H;
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = ((int64_t)b * N * H + h) * D;
  const int q0 = qblk * kRowsB + wave * 32;
  const int qi = q0 + li;

  // Q^T and dO^T as B operands: k-step t, half h -> dims 16 t + 8 h .. +7.
  bf16x8 qf[NF], gf[NF];
#pragma unroll
  for (int t = 0; t < NF; ++t) {
    const bf16x8 z = {};
    qf[t] = qi < N ? *(const bf16x8*)(Q + head_off + (int64_t)qi * rs + 16 * t + 8 * hh) : z;
    gf[t] = qi < N ? *(const bf16x8*)(dO + head_off + (int64_t)qi * rs + 16 * t + 8 * hh) : z;
  }
  const float lse2 = qi < N ? L2[(int64_t)bh * N + qi] : 0.f;
  const float dd = qi < N ? Drow[(int64_t)bh * N + qi] : 0.f;

  // K/V head of this query head (grouped-query attention: H / Hkv per group)
  const int64_t rs_kv = (int64_t)Hkv * D;
  const int64_t kv_off = ((int64_t)b * N * Hkv + h / (H / Hkv)) * D;
  // Descriptors over the head's K/V rows (ending at byte nbytes); the tile's
  // position goes into the range-checked per-lane offset, so rows n >= N read
  // as zeros.
  const uint32_t nbytes = (uint32_t)(((int64_t)(N - 1) * rs_kv + D) * 2);
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(K + kv_off, 0, nbytes);
  const __amdgpu_buffer_rsrc_t rv = tile_rsrc(V + kv_off, 0, nbytes);
  const uint32_t row_bytes = (uint32_t)(rs_kv * 2);
  uint32_t voff_k[LOADS], voff_v[LOADS];
  copy_offsets<D, LOADS, 1>(wave, lane, row_bytes, voff_k);
  copy_offsets<D, LOADS, 0>(wave, lane, row_bytes, voff_v);
  auto load_tile = [&](int stage, int k0) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)k0 * row_bytes;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      char* dst = smem + stage * G::STAGE + (wave * LOADS + i) * 1024;
      copy_to_lds16(rk, dst, voff_k[i] + off);
      copy_to_lds16(rv, dst + G::TILE, voff_v[i] + off);
    }
  };

  // Row-read addresses: key row li, k-step t at (a0 ^ 32 t) (the swizzle XORs
  // only chunk bits, so the k-step moves bits 5-7 of the address).
  const uint32_t base = lds_addr(smem);
  const uint32_t ka0 = base + li * G::RB + ((hh ^ G::swz_b(li)) * 16);
  const uint32_t va0 = base + G::TILE + li * G::RB + ((hh ^ G::swz_k(li)) * 16);
  uint32_t taddr[NE];
  tr_addresses<D>(base, lane, taddr);

  f32x16 dqacc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) dqacc[e] = f32x16{};

  auto tile = [&](auto st, auto masked, int k0) __attribute__((always_inline)) {
    constexpr int ST = decltype(st)::value;
    constexpr bool MASKED = decltype(masked)::value != 0;
    static_for<2>([&](auto JH) __attribute__((always_inline)) {
      constexpr int jh = decltype(JH)::value;
      bf16x8 f[NF];
      static_for<NF>([&](auto T) __attribute__((always_inline)) {
        constexpr int t = decltype(T)::value;
        f[t] = read_b128<ST * G::STAGE + jh * 32 * G::RB>(ka0 ^ (uint32_t)(32 * t));
      });
      const f32x16 sacc = mfma_rows_counted<NF>(f, qf);
      static_for<NF>([&](auto T) __attribute__((always_inline)) {
        constexpr int t = decltype(T)::value;
        f[t] = read_b128<ST * G::STAGE + jh * 32 * G::RB>(va0 ^ (uint32_t)(32 * t));
      });
      const f32x16 dpacc = mfma_rows_counted<NF>(f, gf);
      bf16x8 ktf[2][NE];
      read_tr_frags<D, ST * G::STAGE, jh>(taddr, ktf);
      // P^T and dS^T; element v holds key k0 + 32 jh + 8 (v / 4) + 4 h + v % 4.
      bf16x8 dsb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = exp2_fast(__builtin_fmaf(sacc[v], scale_log2, -lse2));
        if (MASKED) {
          const int key = k0 + 32 * jh + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key >= N || (CAUSAL && key > qi)) p = 0.f;
        }
        dsb[v >> 3][v & 7] = (__bf16)(p * (dpacc[v] - dd));
      }
      mfma_tr_counted<NE>(ktf, dsb, dqacc);
    });
  };

  const int nkb_all = ceil_div(N, kBC);
  const int nkb = CAUSAL ? min(nkb_all, ceil_div(min(N, (qblk + 1) * kRowsB), kBC)) : nkb_all;
  const int nkb_int = min(nkb, CAUSAL ? qblk * (kRowsB / kBC) : N / kBC) & ~1;
#define STEP(ST_, KB, MASKED_)                                                                   \
  do {                                                                                          \
    const int kb_ = (KB);                                                                       \
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                           \
    __syncthreads(); /* tile kb_ resident; every wave is done with the other stage */           \
    if (kb_ + 1 < nkb) load_tile((ST_) ^ 1, (kb_ + 1) * kBC);                                   \
    if (!(CAUSAL && kb_ * kBC > q0 + 31)) tile(IC<ST_>{}, IC<MASKED_>{}, kb_ * kBC);            \
  } while (0)
  load_tile(0, 0);
  int kb = 0;
  for (; kb < nkb_int; kb += 2) {
    STEP(0, kb, 0);
    STEP(1, kb + 1, 0);
  }
  for (; kb < nkb; kb += 2) {
    STEP(0, kb, 1);
    if (kb + 1 < nkb) STEP(1, kb + 1, 1);
  }
#undef STEP
  // dQ rows stored whole through LDS (every wave is done with the tiles after
  // the barrier; each wave takes 32 * 2D bytes of them).
  static_assert(kNWb * 32 * 2 * D <= 2 * G::STAGE, "the dQ rows are staged in the tile buffers");
  __syncthreads();
  store_rows_via_lds<D>(smem + wave * 32 * (2 * D), dqacc, scale, dQ, head_off, rs, q0, N, lane);
}

// ---------------------------------------------------------------------------
// dK, dV.  LDS: [2 stages x (LSE*log2e[64], D[64])] then 2 stages x (Q tile,
// dO tile), both tiles swz_b (read row-wise and transposed).
// Head dim 64: two waves per SIMD (at most 250 VGPRs, every MFMA in VGPR
// form).  Head dim 128: one wave per SIMD; dV^T and dK^T (128 registers)
// live in the AGPR file, accumulated by assembly MFMAs, so that K^T, V^T, the
// fragments and the softmax keep the 256 VGPRs, and the unmasked tiles run
// the software-pipelined body tile_pipe.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kNWb, D == 64 ? 2 : 1) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Drow,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int H, int Hkv, int N, float scale_log2,
    float scale, int nkb, int xcd_remap) {
  using G = Geo<D>;
  constexpr int NF = D / 16, NE = D / 32;
  constexpr int LOADS = G::TILE / (1024 * kNWb);
  constexpr int ROWV = 1024;  // bytes of per-row vectors (2 stages x 2 x 64 floats)
  __shared__ __attribute__((aligned(1024))) char smem[ROWV + 2 * G::STAGE];
  char* tiles = smem + ROWV;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  int L = blockIdx.x;
  if (xcd_remap) L = (L & 7) * (gridDim.x >> 3) + (L >> 3);
  // One workgroup per (b, K/V head, 128 keys); it accumulates the gradients
  // of all H / Hkv query heads that read this K/V head.
  const int kblk = L % nkb, bhk = L / nkb;  // causal: low key blocks see the most queries
  const int b = bhk / Hkv, hk = bhk - b * Hkv;
  const int grp = H / Hkv;
  const int64_t rs = (int64_t)H * D, rs_kv = (int64_t)Hkv * D;
  const int64_t kv_off = ((int64_t)b * N * Hkv + hk) * D;
  const int k0w = kblk * kRowsB + wave * 32;  // this wave's first key
  const int kj = k0w + li;                    // this lane's key (MFMA column)

  // K^T and V^T as B operands: k-step t, half h -> dims 16 t + 8 h .. +7 of key kj.
  bf16x8 kt[NF], vt[NF];
#pragma unroll
  for (int t = 0; t < NF; ++t) {
    const bf16x8 z = {};
    kt[t] = kj < N ? *(const bf16x8*)(K + kv_off + (int64_t)kj * rs_kv + 16 * t + 8 * hh) : z;
    vt[t] = kj < N ? *(const bf16x8*)(V + kv_off + (int64_t)kj * rs_kv + 16 * t + 8 * hh) : z;
  }

  // Descriptors over a head's Q and dO rows (ending at byte nbytes) and its
  // LSE and D vectors (4 N bytes); the tile's position goes into the
  // range-checked per-lane offset, so rows n >= N read as zeros.
  const uint32_t nbytes = (uint32_t)(((int64_t)(N - 1) * rs + D) * 2);
  // Q, dO, LSE and D of query head h (set per head of the group)
  __amdgpu_buffer_rsrc_t rq, rg, rl, rd;
  auto set_head = [&](int h) __attribute__((always_inline)) {
    const int64_t head_off = ((int64_t)b * N * H + h) * D;
    const int64_t bh = (int64_t)b * H + h;
    rq = tile_rsrc(Q + head_off, 0, nbytes);
    rg = tile_rsrc(dO + head_off, 0, nbytes);
    rl = tile_rsrc(L2 + bh * N, 0, (uint32_t)N * 4);
    rd = tile_rsrc(Drow + bh * N, 0, (uint32_t)N * 4);
  };
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  uint32_t voff[LOADS];
  copy_offsets<D, LOADS, 1>(wave, lane, row_bytes, voff);
  auto load_tile = [&](int stage, int i0) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)i0 * row_bytes;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      char* dst = tiles + stage * G::STAGE + (wave * LOADS + i) * 1024;
      copy_to_lds16(rq, dst, voff[i] + off);
      copy_to_lds16(rg, dst + G::TILE, voff[i] + off);
    }
    // 64 floats of LSE*log2e (wave 0) and of D (wave 1), lanes 0-15; lane i's
    // 16 bytes land at 16 i, and D follows LSE.  The descriptor is chosen by
    // the wave index (a scalar), so it stays in scalar registers.
    if (wave < 2 && lane < 16)
      copy_to_lds16(wave == 0 ? rl : rd, smem + stage * 512 + wave * 256,
                    (uint32_t)i0 * 4 + (uint32_t)lane * 16);
  };

  const uint32_t base = lds_addr(tiles);
  const uint32_t qa0 = base + li * G::RB + ((hh ^ G::swz_b(li)) * 16);  // row li, k-step t at ^ 32 t
  const uint32_t la0 = lds_addr(smem) + hh * 16;
  uint32_t taddr[NE];
  tr_addresses<D>(base, lane, taddr);

  f32x16 dvacc[NE], dkacc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) dvacc[e] = dkacc[e] = f32x16{};
  if constexpr (NE == 4) agpr_fence(dvacc, dkacc);

  auto tile = [&](auto st, auto masked, int i0) __attribute__((always_inline)) {
    constexpr int ST = decltype(st)::value;
    constexpr bool MASKED = decltype(masked)::value != 0;
    static_for<2>([&](auto JQ) __attribute__((always_inline)) {
      constexpr int jq = decltype(JQ)::value;
      const int iq0 = i0 + 32 * jq;
      if (MASKED && CAUSAL && iq0 + 31 < k0w) return;  // every query before every key of this wave
      bf16x8 f[NF];
      static_for<NF>([&](auto T) __attribute__((always_inline)) {
        constexpr int t = decltype(T)::value;
        f[t] = read_b128<ST * G::STAGE + jq * 32 * G::RB>(qa0 ^ (uint32_t)(32 * t));
      });
      const f32x16 sacc = mfma_rows_counted<NF>(f, kt);
      static_for<NF>([&](auto T) __attribute__((always_inline)) {
        constexpr int t = decltype(T)::value;
        f[t] = read_b128<ST * G::STAGE + G::TILE + jq * 32 * G::RB>(qa0 ^ (uint32_t)(32 * t));
      });
      const f32x16 dpacc = mfma_rows_counted<NF>(f, vt);
      // LSE*log2e and D of this lane's 16 query rows 32 jq + 8 g + 4 h + (0..3).
      f32x4 l4[4], d4[4];
      static_for<4>([&](auto Gi) __attribute__((always_inline)) {
        constexpr int g = decltype(Gi)::value;
        l4[g] = read_f4<ST * 512 + (32 * jq + 8 * g) * 4>(la0);
        d4[g] = read_f4<ST * 512 + 256 + (32 * jq + 8 * g) * 4>(la0);
      });
      lds_wait_f4(l4, d4);
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = exp2_fast(__builtin_fmaf(sacc[v], scale_log2, -l4[v >> 2][v & 3]));
        if (MASKED) {
          const int q = iq0 + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (q >= N || (CAUSAL && kj > q)) p = 0.f;
        }
        pb[v >> 3][v & 7] = (__bf16)p;
        dsb[v >> 3][v & 7] = (__bf16)(p * (dpacc[v] - d4[v >> 2][v & 3]));
      }
      bf16x8 tf[2][NE];
      read_tr_frags<D, ST * G::STAGE + G::TILE, jq>(taddr, tf);  // dO^T
      if constexpr (NE == 4) mfma_tr_agpr4(tf, pb, dvacc);
      else mfma_tr_counted<NE>(tf, pb, dvacc);
      read_tr_frags<D, ST * G::STAGE, jq>(taddr, tf);  // Q^T
      if constexpr (NE == 4) mfma_tr_agpr4(tf, dsb, dkacc);
      else mfma_tr_counted<NE>(tf, dsb, dkacc);
    });
  };

  // Head dim 128, unmasked tiles: the tile's two 32-query blocks as one
  // software pipeline of 64 MFMA slots (see pipe128).  P of a block is
  // computed two rows at a time under its dP products and dS under its dV^T
  // products, about five VALU instructions per MFMA; each slot ends in a
  // scheduling barrier so that this interleave is kept, and each slot's VALU
  // results are pinned in place by an empty assembly use.  The arithmetic and
  // its order are those of the tile body above.
  auto tile_pipe = [&](auto st, int i0) __attribute__((always_inline)) {
    constexpr int ST = decltype(st)::value;
    (void)i0;
    bf16x8 fq[2][8], fg[2][8];
    f32x4 l4[2][4], d4[2][4];
    bf16x4 tlo[2][8], thi[2][8], qlo[2][8], qhi[2][8];
    f32x16 sacc[2], dpacc[2];
    float pr[2][16], fa[2][16], dd[2][16], dsv[2][16];
    uint32_t pw[2][8], dw[2][8];
    auto issue = [&](auto P_) __attribute__((always_inline)) {
      constexpr int P = decltype(P_)::value;
      constexpr int b = P / pipe128::kRPB, q = P % pipe128::kRPB;
      if constexpr (q < 8) {
        fq[b][q] = read_b128<ST * G::STAGE + b * 32 * G::RB>(qa0 ^ (uint32_t)(32 * q));
      } else if constexpr (q < 12) {
        l4[b][q - 8] = read_f4<ST * 512 + (32 * b + 8 * (q - 8)) * 4>(la0);
      } else if constexpr (q < 20) {
        fg[b][q - 12] =
            read_b128<ST * G::STAGE + G::TILE + b * 32 * G::RB>(qa0 ^ (uint32_t)(32 * (q - 12)));
      } else if constexpr (q < 24) {
        d4[b][q - 20] = read_f4<ST * 512 + 256 + (32 * b + 8 * (q - 20)) * 4>(la0);
      } else {
        constexpr bool isq = q >= 40;
        constexpr int r = isq ? q - 40 : q - 24;
        constexpr int k = r / 2, half = r % 2, e = k / 2, T = k % 2;
        constexpr int OFF = ST * G::STAGE + (isq ? 0 : G::TILE) + (32 * b + 16 * T + 8 * half) * G::RB;
        const bf16x4 v = read_tr16<OFF>(half ? (taddr[e] ^ 32u) : taddr[e]);
        if constexpr (isq) {
          if constexpr (half) qhi[b][k] = v; else qlo[b][k] = v;
        } else {
          if constexpr (half) thi[b][k] = v; else tlo[b][k] = v;
        }
      }
    };
    auto join = [](const bf16x4& lo, const bf16x4& hi) __attribute__((always_inline)) {
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto words = [](const uint32_t* w) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]});
    };
    static_for<64>([&](auto S_) __attribute__((always_inline)) {
      constexpr int s = decltype(S_)::value;
      constexpr int b = s / 32, j = s % 32, ph = j / 8, i = j % 8;
      // reads for later slots are issued right after this slot's MFMA (they
      // fill its operand-fetch cycles, which VALU instructions cannot use)
      constexpr int first = pipe128::issued(s - 1) + 1;  // (slot 0: after the prologue's)
      auto issue_ahead = [&]() __attribute__((always_inline)) {
        static_for<pipe128::issued(s) - pipe128::issued(s - 1)>([&](auto K_) __attribute__((always_inline)) {
          issue(IC<first + decltype(K_)::value>{});
        });
      };
      if constexpr (s == 0) {  // prologue: the first kLook + 1 reads
        static_for<pipe128::kLook + 1>([&](auto K_) __attribute__((always_inline)) {
          issue(IC<decltype(K_)::value>{});
        });
      }
      constexpr int W = pipe128::issued(s - 1) - pipe128::need(s);
      static_assert(W >= 0, "this slot's reads were issued by earlier slots");
      if constexpr (ph == 0) {  // S = Q K^T
        wait_lds<W>(fq[b][i]);
        sacc[b] = mfma_bf16(fq[b][i], kt[i], i == 0 ? f32x16{} : sacc[b]);
        __builtin_amdgcn_sched_barrier(0);
        issue_ahead();
      } else if constexpr (ph == 1) {  // dP = dO V^T; P two rows per slot
        if constexpr (i == 0) wait_lds_rows<W>(fg[b][0], l4[b]);
        else wait_lds<W>(fg[b][i]);
        dpacc[b] = mfma_bf16(fg[b][i], vt[i], i == 0 ? f32x16{} : dpacc[b]);
        __builtin_amdgcn_sched_barrier(0);  // the MFMA issues before the VALU that waits on S
        issue_ahead();
        // exp2 arguments of the next slot's rows, exponentials of this slot's,
        // bf16 pair of the previous slot's: no instruction waits on a result
        // of its own slot.
        static_for<2>([&](auto U_) __attribute__((always_inline)) {
          constexpr int u = decltype(U_)::value;
          if constexpr (i == 0)
            fa[b][u] = __builtin_fmaf(sacc[b][u], scale_log2, -l4[b][0][u]);
          if constexpr (i < 7) {
            constexpr int v = 2 * i + 2 + u;
            fa[b][v] = __builtin_fmaf(sacc[b][v], scale_log2, -l4[b][v >> 2][v & 3]);
          }
          pr[b][2 * i + u] = exp2_fast(fa[b][2 * i + u]);
        });
        if constexpr (i >= 1) pw[b][i - 1] = pack_bf16x2(pr[b][2 * i - 2], pr[b][2 * i - 1]);
        asm volatile("" : "+v"(pr[b][2 * i]), "+v"(pr[b][2 * i + 1]));
        if constexpr (i < 7) asm volatile("" : "+v"(fa[b][2 * i + 2]), "+v"(fa[b][2 * i + 3]));
        if constexpr (i >= 1) asm volatile("" : "+v"(pw[b][i - 1]));
      } else if constexpr (ph == 2) {  // dV^T += dO^T P; dS two rows per slot
        if constexpr (i == 0) wait_lds_pair_rows<W>(tlo[b][i], thi[b][i], d4[b]);
        else wait_lds_pair<W>(tlo[b][i], thi[b][i]);
        mfma_agpr<i <= 1>(dvacc[i / 2], join(tlo[b][i], thi[b][i]), words(&pw[b][4 * (i % 2)]));
        __builtin_amdgcn_sched_barrier(0);  // the MFMA issues before the VALU that waits on dP
        issue_ahead();
        if constexpr (i == 0) {
          pw[b][7] = pack_bf16x2(pr[b][14], pr[b][15]);
          asm volatile("" : "+v"(pw[b][7]));
        }
        static_for<2>([&](auto U_) __attribute__((always_inline)) {
          constexpr int u = decltype(U_)::value;
          if constexpr (i == 0) dd[b][u] = dpacc[b][u] - d4[b][0][u];
          if constexpr (i < 7) {
            constexpr int v = 2 * i + 2 + u;
            dd[b][v] = dpacc[b][v] - d4[b][v >> 2][v & 3];
          }
          dsv[b][2 * i + u] = pr[b][2 * i + u] * dd[b][2 * i + u];
        });
        if constexpr (i >= 1) dw[b][i - 1] = pack_bf16x2(dsv[b][2 * i - 2], dsv[b][2 * i - 1]);
        asm volatile("" : "+v"(dsv[b][2 * i]), "+v"(dsv[b][2 * i + 1]));
        if constexpr (i < 7) asm volatile("" : "+v"(dd[b][2 * i + 2]), "+v"(dd[b][2 * i + 3]));
        if constexpr (i >= 1) asm volatile("" : "+v"(dw[b][i - 1]));
      } else {  // dK^T += Q^T dS
        wait_lds_pair<W>(qlo[b][i], qhi[b][i]);
        mfma_agpr<i <= 1>(dkacc[i / 2], join(qlo[b][i], qhi[b][i]), words(&dw[b][4 * (i % 2)]));
        __builtin_amdgcn_sched_barrier(0);
        issue_ahead();
        if constexpr (i == 0) {
          __builtin_amdgcn_sched_barrier(0);
          dw[b][7] = pack_bf16x2(dsv[b][14], dsv[b][15]);
          asm volatile("" : "+v"(dw[b][7]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Query tiles: causal starts at the tile holding the workgroup's first key.
  // The tiles run in three loops of whole pairs (stage 0, stage 1) so that the
  // hot middle loop holds one copy of the unmasked tile body and no branch
  // that the accumulators' registers would have to be reconciled across:
  //   head   [qt0, qt_lo)   causal only: the two tiles that hold the
  //                         workgroup's keys (masked; waves skip what lies
  //                         entirely before their keys)
  //   middle [qt_lo, qt_hi) unmasked: no query past N, none before a key
  //   tail   [qt_hi, nqt)   masked: the rest, including a ragged last tile
  const int nqt = ceil_div(N, kBC);
  const int qt0 = CAUSAL ? (kblk * kRowsB) / kBC : 0;
  static_assert(kRowsB == 2 * kBC, "the causal head is one pair of tiles");
  const int qt_lo = CAUSAL ? min(nqt, qt0 + 2) : qt0;
  const int n_full = N / kBC;
  const int qt_hi = n_full > qt_lo ? qt_lo + ((n_full - qt_lo) & ~1) : qt_lo;
#define STEP(ST_, QT, MASKED_)                                                                   \
  do {                                                                                          \
    const int qt_ = (QT);                                                                       \
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                           \
    __syncthreads(); /* tile qt_ resident; every wave is done with the other stage */           \
    if (qt_ + 1 < nqt) load_tile((ST_) ^ 1, (qt_ + 1) * kBC);                                   \
    const int i0_ = qt_ * kBC;                                                                  \
    if constexpr (NE == 4 && !(MASKED_)) tile_pipe(IC<ST_>{}, i0_);                              \
    else if (!(MASKED_) || !(CAUSAL && i0_ + kBC - 1 < k0w)) tile(IC<ST_>{}, IC<MASKED_>{}, i0_); \
  } while (0)
  for (int g = 0; g < grp; ++g) {
    set_head(hk * grp + g);
    // every wave is done with the previous head's tiles before stage 0 is refilled
    if (g > 0) __syncthreads();
    load_tile(0, qt0 * kBC);
    int qt = qt0;
    for (; qt < qt_lo; qt += 2) {
      STEP(0, qt, 1);
      if (qt + 1 < nqt) STEP(1, qt + 1, 1);
    }
    for (; qt < qt_hi; qt += 2) {
      STEP(0, qt, 0);
      STEP(1, qt + 1, 0);
    }
    for (; qt < nqt; qt += 2) {
      STEP(0, qt, 1);
      if (qt + 1 < nqt) STEP(1, qt + 1, 1);
    }
  }
#undef STEP
  // dK and dV rows stored whole through LDS (every wave is done with the
  // tiles after the barrier; each wave takes 2 * 32 * 2D bytes of them).
  static_assert(kNWb * 2 * 32 * 2 * D <= 2 * G::STAGE, "the dK/dV rows are staged in the tile buffers");
  if constexpr (NE == 4) agpr_fence(dvacc, dkacc);
  __syncthreads();
  char* ob = tiles + wave * 2 * 32 * (2 * D);
  store_rows_via_lds<D>(ob, dkacc, scale, dK, kv_off, rs_kv, k0w, N, lane);
  store_rows_via_lds<D>(ob + 32 * (2 * D), dvacc, 1.f, dV, kv_off, rs_kv, k0w, N, lane);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float* ws, int B, int H,
                      int Hkv, int N, float scale, hipStream_t stream) {
  const int64_t rows = (int64_t)B * N * H;
  float* drow = ws;
  float* l2 = ws + rows;
  constexpr int RPB = 256 / (D / 8);  // rows per prep block
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, (const __bf16*)o, (const __bf16*)dout, lse, drow, l2, H, N, rows);
  const int nb = (N + kRowsB - 1) / kRowsB;
  const int64_t grid_kv = (int64_t)B * Hkv * nb;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)grid_kv), dim3(64 * kNWb), 0,
                     stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                     (const __bf16*)dout, l2, drow, (__bf16*)dk, (__bf16*)dv, H, Hkv, N,
                     scale * kLog2e, scale, nb, (grid_kv % 8 == 0) ? 1 : 0);
  const int64_t grid = (int64_t)B * H * nb;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(64 * kNWb), 0, stream,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, l2,
                     drow, (__bf16*)dq, H, Hkv, N, scale * kLog2e, scale, nb,
                     (grid % 8 == 0) ? 1 : 0);
  return hipGetLastError();
}

// Fixed device scratch for callers that cannot allocate (the no-allocation
// gradient entry point): it takes the place of the caller's workspace (D and
// LSE * log2(e), 8 B H N bytes).  One copy per GPU, resident until the
// process ends; its device address is looked up once per device.
constexpr size_t kScratchBytes = EXATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
float* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];

}  // namespace

size_t bwd_scratch_bytes() { return kScratchBytes; }

hipError_t launch_attn_bwd_bf16_noalloc(const void* q, const void* k, const void* v,
                                        const void* o, const void* dout, const float* lse,
                                        void* dq, void* dk, void* dv, int B, int H, int Hkv,
                                        int N, int d, bool causal, float softmax_scale,
                                        hipStream_t stream) {
  if ((size_t)8 * B * H * N > kScratchBytes) return hipErrorInvalidValue;  // checked by the caller
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // The symbol's device address, taken with this device current (each GPU
  // holds its own copy of the array); the host-side name is not a device
  // address and is never passed to a kernel.
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_status[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  });
  if (g_scratch_status[dev] != hipSuccess) return g_scratch_status[dev];
  if (g_scratch_ptr[dev] == nullptr) return hipErrorInvalidSymbol;
  return launch_attn_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, g_scratch_ptr[dev], B, H, Hkv, N,
                              d, causal, softmax_scale, stream);
}

hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                float* workspace, int B, int H, int Hkv, int N, int d,
                                bool causal, float softmax_scale, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_bwd<128, true>(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Hkv, N,
                                          softmax_scale, stream)
                  : launch_bwd<128, false>(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Hkv, N,
                                           softmax_scale, stream);
  return causal ? launch_bwd<64, true>(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Hkv, N,
                                       softmax_scale, stream)
                : launch_bwd<64, false>(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, Hkv, N,
                                        softmax_scale, stream);
}

}  // namespace exattn
