// bf16 exact-attention forward for gfx950.
//
// Work decomposition (FA2 query-block parallelism, "Efficient Attention &
// FlashAttention" M4-054): one workgroup per (b, h, block of query rows);
// each wave owns 32 query rows and two waves share a SIMD.  Long sequences use
// 8-wave workgroups (256 rows; one per CU, so a K/V tile in LDS serves 256
// rows), short ones 4-wave workgroups (128 rows; two per CU, so one
// workgroup's start-up and epilogue overlap the other's key tiles).  The
// key/value sequence is streamed in blocks of 64 keys with the online-softmax
// recurrence of the FlashAttention-3 report, section 3 (running max m,
// running sum l, one final normalisation).  Causal work runs on
// persistent workgroup slots over pairs of query blocks of equal total cost
// (see the kernel below).  Head dim 256 runs 4-wave workgroups, one wave
// per SIMD, with O in the AGPR file.  The interior key tiles run software-
// pipelined (the next tile's S MFMAs issued between the current tile's
// exponentials, report section 3.2): non-causal everywhere, causal from
// N = 1024; every other case runs the same-phase loop (both waves of a SIMD
// do MFMAs, then both do softmax).
//
// Transposed formulation.  Each wave computes S^T = K Q^T (keys as MFMA rows,
// its 32 queries as MFMA columns), so the accumulator keeps every query on one
// lane pair (l, l^32): row max and row sum are in-lane reductions plus one
// cross-half exchange.  The output is accumulated as O^T = V^T P^T, whose
// accumulator again keeps one query per lane, so the per-row rescale factor is
// a lane-local scalar.  P^T goes to the second MFMA straight from the S^T
// accumulator (converted to bf16): half-wave h, k-slot s of k-step t holds key
// 16t + 8*(s/4) + 4h + s%4, and the V^T operand is gathered with the same key
// order -- the gfx950 counterpart of the report's accumulator-to-operand
// relayout (section 3.3).
//
// Memory pipeline (the report's producer/consumer overlap, section 3.1, done
// the gfx950 way).  K and V tiles go from HBM/L2 straight into LDS with
// buffer_load ... lds (no VGPR staging), two stages deep: the loads of tile
// j+1 are in flight while tile j is consumed; one barrier per tile.  LDS rows
// are XOR-swizzled in 16-byte chunks so that the ds_read_b128 of the K operand
// and the ds_read_b64_tr_b16 transposed reads of the V operand are free of
// bank conflicts; the V tile stays key-major in LDS and the transposed read
// produces V^T fragments directly.  Reads past the end of the sequence come
// back as zeros from the buffer descriptor's range check.  Within a tile, the
// K fragment reads run eight MFMAs ahead of the S MFMAs, and all V^T fragments
// are read before the softmax, whose VALU work then covers their LDS latency.
//
// Rescaling (exact, fewer non-matmul FLOPs: "Efficient Attention &
// FlashAttention", FA2 section).  A row's exp2 offset is raised to its block
// max only when that max exceeds the offset by more than 8 (base 2); P is then
// at most 2^8 and O, l stay consistent with the offset, so O / l and the LSE
// are unchanged while most blocks skip the O rescale entirely.  The decision
// is per row, so a row's arithmetic depends on its own visible keys only.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "lds_tile.h"

namespace exattn {
namespace {

constexpr float kLazy = 8.f;  // rescale threshold (log2 units)

// -inf for keys >= N and, when causal, keys after query qi.  k0: first key.
__device__ __forceinline__ void mask_s(f32x16 (&sacc)[2], int k0, int N, bool causal, int qi,
                                       int hh) {
  const int lim = causal ? min(N, qi + 1) : N;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + j * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
      if (key >= lim) sacc[j][v] = -INFINITY;
    }
}

// In-lane max over this lane's 32 scores (the other half-wave holds the rest).
__device__ __forceinline__ float rowmax(const f32x16 (&s)[2]) {
  float a = fmaxf(s[0][0], s[0][1]), b = fmaxf(s[1][0], s[1][1]);
#pragma unroll
  for (int v = 2; v < 16; v += 2) {
    a = fmaxf(a, fmaxf(s[0][v], s[0][v + 1]));
    b = fmaxf(b, fmaxf(s[1][v], s[1][v + 1]));
  }
  return fmaxf(a, b);
}

// Head dim 256: O^T (128 registers a lane) stays in the AGPR file from its
// zeroing to the epilogue.  Its P.V products are assembly MFMAs on "+a"
// operands (the compiler's own MFMAs write VGPRs, -amdgpu-mfma-vgpr-form), so
// that Q^T, S and the softmax keep the 256 VGPRs and O is never copied
// between the two files in the tile loops.  The compiler does not see the
// MFMAs inside the assembly, so the wait states around them are explicit: a
// leading s_nop 1 for a B operand just written by the VALU, and o_fence (24
// wait states) between the accumulators' MFMAs and any other instruction
// that touches them (the rescale, the epilogue).
template <bool NOP2>
__device__ __forceinline__ void mfma_o(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (NOP2)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int D>
__device__ __forceinline__ void o_fence(f32x16 (&o)[D / 32]) {
  if constexpr (D > 128)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                   "+a"(o[6]), "+a"(o[7]));
}
// O^T[e] += a b; NOP2: b may have been written by the VALU just before.
template <int D, bool NOP2>
__device__ __forceinline__ void pv_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (D > 128) mfma_o<NOP2>(acc, a, b);
  else acc = mfma_bf16(a, b, acc);
}
// O^T *= alpha (the rare lazy-offset raise; at d = 256 through the AGPRs).
template <int D>
__device__ __forceinline__ void o_scale(f32x16 (&o)[D / 32], float alpha) {
  o_fence<D>(o);
#pragma unroll
  for (int e = 0; e < D / 32; ++e) o[e] *= alpha;
  o_fence<D>(o);
}

// One key tile in LDS stage ST: S^T = K Q^T, (masking,) online softmax with
// lazy offset, and O^T += V^T P^T.  smem: the LDS tile buffers; vaddr: LDS
// addresses of this lane's V^T fragment sources in stage 0's V buffer.
template <int D, bool CAUSAL, bool MASKED, int ST>
__device__ __forceinline__ void tile_compute(const char* smem, const uint32_t (&kaddr)[D / 16],
                                             const uint32_t (&vaddr)[D / 32],
                                             const bf16x8 (&qf)[D / 16], f32x16 (&oacc)[D / 32],
                                             float& m, float& l, int k0, int N, int qi, int hh,
                                             float scale_log2) {
  using G = Geo<D>;
  // S^T = K Q^T: two 32-key blocks.  Fragment i = 2t + j (k-step t, block
  // j); the reads run AHEAD fragments ahead of the MFMAs (the loop's barrier
  // has drained this wave's LDS reads, so lgkmcnt counts only these).
  constexpr int NK = 2 * (D / 16);
  constexpr int AHEAD = 8;
  bf16x8 kf[NK];
  auto rd = [&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value, t = i / 2, j = i % 2;
    kf[i] = read_b128<G::koff(ST) + j * 32 * G::RB>(kaddr[t]);
  };
  static_for<AHEAD>(rd);
  f32x16 sacc[2];
  static_for<NK>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value, t = i / 2, j = i % 2;
    constexpr int issued = (AHEAD + i < NK) ? AHEAD + i : NK;
    wait_lds<issued - i - 1>(kf[i]);
    sacc[j] = mfma_bf16(kf[i], qf[t], t == 0 ? f32x16{} : sacc[j]);
    if constexpr (i + AHEAD < NK) rd(IC<i + AHEAD>{});
  });
  // V^T fragments for this tile's P.V, read before the softmax so that the
  // exp/sum work covers their latency.  At d = 256 they come in two halves of
  // four 32-row d-blocks (the second half after the first half's MFMAs), so
  // at most 64 VGPRs of them are live.
  constexpr int NEH = D / 32 <= 4 ? D / 32 : 4;  // d-blocks per half
  constexpr int NHALF = (D / 32) / NEH;
  bf16x8 vf[4][NEH];
  constexpr int VOFF = G::voff(ST);
#define TR_PAIR(T2, E, VA)                                                                       \
  {                                                                                              \
    const bf16x4 lo = read_tr16<VOFF + (16 * (T2)) * G::RB>(VA);                                \
    const bf16x4 hi = read_tr16<VOFF + (16 * (T2) + 8) * G::RB>(VA);                            \
    vf[T2][E] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};                  \
  }
#pragma unroll
  for (int e = 0; e < NEH; ++e) {
    TR_PAIR(0, e, vaddr[e]) TR_PAIR(1, e, vaddr[e]) TR_PAIR(2, e, vaddr[e]) TR_PAIR(3, e, vaddr[e])
  }
  if (MASKED) mask_s(sacc, k0, N, CAUSAL, qi, hh);

  const float mx = max_halves(rowmax(sacc));
  const float mb = mx * scale_log2;
  const bool raise = mb > m + kLazy;  // per row: each row's offset depends on its own keys only
  if (__builtin_amdgcn_ballot_w64(raise) != 0) {
    const float m_new = raise ? mb : m;
    const float alpha = exp2_fast(m - m_new);
    m = m_new;
    l *= alpha;
    o_scale<D>(oacc, alpha);
  }
  const float neg_m = -m;
  float rsum = 0.f;
  bf16x8 pb[4];
#pragma unroll
  for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float p = exp2_fast(__builtin_fmaf(sacc[t2 >> 1][8 * (t2 & 1) + s], scale_log2, neg_m));
      rsum += p;
      pb[t2][s] = (__bf16)p;
    }
  l += rsum;

  // O^T += V^T P^T.
  lds_wait_v(vf);
  static_for<4>([&](auto T2) __attribute__((always_inline)) {
    constexpr int t2 = decltype(T2)::value;
    static_for<NEH>([&](auto E) __attribute__((always_inline)) {
      constexpr int e = decltype(E)::value;
      pv_mfma<D, e == 0>(oacc[e], vf[t2][e], pb[t2]);
    });
  });
  if constexpr (NHALF == 2) {
#pragma unroll
    for (int e = 0; e < NEH; ++e) {
      TR_PAIR(0, e, vaddr[NEH + e]) TR_PAIR(1, e, vaddr[NEH + e])
      TR_PAIR(2, e, vaddr[NEH + e]) TR_PAIR(3, e, vaddr[NEH + e])
    }
    lds_wait_v(vf);
    static_for<4>([&](auto T2) __attribute__((always_inline)) {
      constexpr int t2 = decltype(T2)::value;
      static_for<NEH>([&](auto E) __attribute__((always_inline)) {
        constexpr int e = decltype(E)::value;
        pv_mfma<D, e == 0>(oacc[NEH + e], vf[t2][e], pb[t2]);
      });
    });
  }
#undef TR_PAIR
}

// Software-pipelined interior tiles (non-causal at every head dim and on
// both workgroup sizes; causal from N = 1024, up to a block's diagonal; the
// same-phase loop below serves the edge tiles and every other case).  The FlashAttention-3 report (section 3.2) issues the next block's
// S = Q K^T before the current block's softmax so that the matrix cores work
// while the exponentials run.  Here iteration j of a wave issues its MFMAs one
// per slot: the NS of S(j+1) = K(j+1) Q^T, then the NP of
// O^T += V(j)^T P(j)^T (d = 256: 32 + 32 slots, d = 128: 16 + 16, d = 64:
// 8 + 8).  Between them
// run the VALU work of tile j's softmax and S(j+1)'s row max (the last 8
// slots): exponential v (with its multiply-add and row-sum add) in slot
// exp_slot(v), spread evenly over the slots before the last P^T operand's
// first MFMA (d = 128: about one per slot), and each bf16 pair packed in the
// slot of its second exponential, so every P^T operand is complete before its
// first MFMA (d = 128: measured 0.8% faster than two exponentials in each of
// 16 slots).  Each MFMA's K or V^T fragment is read kLook reads ahead and
// waited for with an exact lgkmcnt count.  K is loaded one tile ahead of V in
// an LDS ring of R slots each (Ring below).  Every output element goes through
// the same operations in the same order as in the same-phase loop, so the
// results are bit-identical to it.
namespace fpipe {
constexpr int kLook = 5;  // LDS reads in flight ahead of the MFMA that needs them
template <int D>
struct Slots {
  static constexpr int NS = 2 * (D / 16);  // S(j+1) MFMAs = K fragments
  static constexpr int NE = D / 32;        // 32-dim blocks of O^T
  static constexpr int NP = 4 * NE;        // P(j).V(j) MFMAs, two V^T half reads each
  static constexpr int N = NS + NP;        // slots per iteration
  static constexpr int kLast = NS + 2 * NP - 1;  // last read index of the iteration
  // Read that slot s's MFMA needs last: K fragment s, or the second V^T half
  // of P.V MFMA s - NS.
  static constexpr int need(int s) { return s < NS ? s : NS + 2 * (s - NS) + 1; }
  // Reads issued by the end of slot s (s = -1: the prologue).
  static constexpr int issued(int s) {
    return s < 0 ? kLook : (need(s) + kLook < kLast ? need(s) + kLook : kLast);
  }
  // Exponential v (0 .. 31) of tile j's P^T: slots 0 .. NS + 3 NE - 1.
  static constexpr int exp_slot(int v) { return (v * (NS + 3 * NE)) / 32; }
  // P^T operand t2 (bf16 pairs 4 t2 .. 4 t2 + 3) is first read in slot
  // NS + t2 NE, so its last exponential must come earlier.
  static constexpr bool exps_in_time() {
    for (int t2 = 0; t2 < 4; ++t2)
      if (exp_slot(8 * t2 + 7) >= NS + t2 * NE) return false;
    return true;
  }
  static_assert(exps_in_time(), "an exponential after its P^T operand's first MFMA");
  static constexpr int kMax0 = N - 8;  // S(j+1)'s row max: slots kMax0 .. N - 1
};
// LDS slots of the pipelined loop.  R = 2: the two stages of the same-phase
// loop ([K0 V0][K1 V1]); the next tile's copies can start only after the
// barrier that frees their slots.  R = 4: [K0 K1 K2 K3][V0 V1 V2 V3] (8
// tiles: 128 KB at d = 128, 64 KB at d = 64); the copies of K(j+3) and V(j+2)
// go out at the end of iteration j, into slots freed two iterations earlier,
// so their issue (a queue of 1 KB copies behind the other waves') overlaps
// the wait at the next barrier instead of following it.  The V^T read addresses carry the V
// region's base (VB), so every immediate offset stays below 64 KB.
template <int D, int R>
struct Ring {
  using G = Geo<D>;
  static constexpr int k(int i) { return R == 2 ? G::koff(i) : i * G::TILE; }
  static constexpr int v(int i) { return R == 2 ? G::voff(i) : i * G::TILE; }
  static constexpr int VB = R == 2 ? 0 : 4 * G::TILE;
  static constexpr int kBytes = R == 2 ? 2 * G::STAGE : 8 * G::TILE;
};
// Ring size: 4 on the 8-wave workgroups (one per CU: their registers leave
// room for no second one); 2 on the 4-wave ones, which share a CU with others
// and would lose occupancy to the larger ring (-4.6% at B16 N1024 d64).
template <int D, int NW>
constexpr int ring() { return NW == 8 ? 4 : 2; }
}  // namespace fpipe

// One workgroup's work item: query block qblk (32 * NW rows) of head bh,
// against every visible key.
// Causal work runs persistent at every head dim (at d = 256 since O moved to
// the AGPR file: the loop around the body no longer spills; +4% at B2 H16
// N8192, +16% at B8 H16 N2048).
template <int D, bool CAUSAL>
constexpr bool persistent() { return CAUSAL; }

template <int D, bool CAUSAL, int NW, bool PIPE>
__device__ __forceinline__ void attend_block(char* smem, const __bf16* __restrict__ Q,
                                             const __bf16* __restrict__ K,
                                             const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                             float* __restrict__ LSE, int H, int Hkv, int N,
                                             float scale_log2, int bh, int qblk) {
  using G = Geo<D>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int li = lane & 31;
  const int hh = lane >> 5;

  const int b = bh / H;
  const int h = bh - b * H;
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = ((int64_t)b * N * H + h) * D;
  // Grouped-query attention: H / Hkv consecutive query heads read one K/V head.
  const int64_t rs_kv = (int64_t)Hkv * D;
  const int64_t kv_off = ((int64_t)b * N * Hkv + h / (H / Hkv)) * D;

  constexpr int kBR = 32 * NW;                       // query rows per workgroup
  static_assert(NW * 32 * 2 * D <= 2 * G::STAGE, "the output rows are staged in the tile buffers");
  constexpr int LOADS = G::TILE / (1024 * NW);        // 1 KB copies per wave per tile
  const int q0 = qblk * kBR + wave * 32;
  const int qi = q0 + li;

  // Q^T as the B operand: k-step t, half h -> dims 16t + 8h .. +7 of query qi.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    bf16x8 z = {};
    qf[t] = (qi < N) ? *(const bf16x8*)(Q + head_off + (int64_t)qi * rs + 16 * t + 8 * hh) : z;
  }

  // This head's K and V rows end at byte nbytes; each tile's copies go
  // through a descriptor that starts at the tile's first row and ends there,
  // so rows n >= N read as zeros.
  const uint32_t nbytes = (uint32_t)(((int64_t)(N - 1) * rs_kv + D) * 2);
  const __bf16* kh = K + kv_off;
  const __bf16* vh = V + kv_off;
  const uint32_t row_bytes = (uint32_t)(rs_kv * 2);

  // Per-lane global byte offsets of the chunks this lane deposits into LDS.
  uint32_t voff_k[LOADS], voff_v[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int chunk = (wave * LOADS + i) * 64 + lane;  // LDS chunk slot within a tile
    const int row = chunk / G::CPR, pos = chunk % G::CPR;
    voff_k[i] = row * row_bytes + (uint32_t)((pos ^ G::swz_k(row)) * 16);
    voff_v[i] = row * row_bytes + (uint32_t)((pos ^ G::swz_v(row)) * 16);
  }
#define LOAD_TILE(stage, k0)                                                                    \
  do {                                                                                          \
    const uint32_t off_ = (uint32_t)(k0) * row_bytes;                                           \
    const __amdgpu_buffer_rsrc_t rk_ = tile_rsrc(kh, off_, nbytes);                             \
    const __amdgpu_buffer_rsrc_t rv_ = tile_rsrc(vh, off_, nbytes);                             \
    _Pragma("unroll") for (int i_ = 0; i_ < LOADS; ++i_) {                                   \
      char* dst_ = smem + (wave * LOADS + i_) * 1024;                                          \
      copy_to_lds16(rk_, dst_ + G::koff(stage), voff_k[i_]);                                    \
      copy_to_lds16(rv_, dst_ + G::VBASE + G::voff(stage), voff_v[i_]);                         \
    }                                                                                           \
  } while (0)

  // LDS byte offsets (within a tile) of this lane's operand fragments.
  uint32_t kaddr[D / 16];  // LDS addresses: K rows li (+32 for the second block), chunk 2t + hh
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    kaddr[t] = lds_addr(smem) + li * G::RB + (((2 * t + hh) ^ G::swz_k(li)) * 16);
  uint32_t vaddr[D / 32];  // transposed-read source: key 4h + j, dims 32e + 16(g%2) + 4q
  {
    const int src = lane & 15, g = lane >> 4;
    const int j = src >> 2, q = src & 3, hv = g >> 1;
    const int row = 4 * hv + j;
#pragma unroll
    for (int e = 0; e < D / 32; ++e) {
      const int c = 4 * e + 2 * (g & 1) + (q >> 1);
      vaddr[e] = lds_addr(smem) + G::VBASE + row * G::RB + ((c ^ G::swz_v(row)) * 16) + (q & 1) * 8;
    }
  }

  float m = kNoMax;  // exp2 offset (base-2 domain), raised lazily
  float l = 0.f;     // running sum over this lane's half of the keys
  f32x16 oacc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e) oacc[e] = f32x16{};
  o_fence<D>(oacc);

  const int nkb_all = ceil_div(N, kBC);
  const int nkb = CAUSAL ? min(nkb_all, ceil_div(min(N, (qblk + 1) * kBR), kBC)) : nkb_all;

  // Interior tiles (no key past the end, no key after any row of this
  // workgroup) need no masking and come first; the few edge tiles follow.
  // Both loops take tiles two at a time from an even tile index, so the LDS
  // stage of every step is a compile-time constant.
  const int nkb_int = min(nkb, CAUSAL ? qblk * (kBR / kBC) : N / kBC) & ~1;
#define STEP(ST_, KB, MASKED)                                                                    \
  do {                                                                                          \
    const int kb_ = (KB);                                                                       \
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                           \
    __syncthreads(); /* tile kb_ resident; every wave is done with the other stage */           \
    if (kb_ + 1 < nkb) LOAD_TILE((ST_) ^ 1, (kb_ + 1) * kBC);                                   \
    if (!(CAUSAL && kb_ * kBC > q0 + 31))                                                       \
      tile_compute<D, CAUSAL, MASKED, ST_>(smem, kaddr, vaddr, qf, oacc, m, l, kb_ * kBC, N, qi, \
                                           hh, scale_log2);                                     \
  } while (0)
  int kb = 0;
  if constexpr (PIPE) {
    using P = fpipe::Slots<D>;
    constexpr int R = fpipe::ring<D, NW>();
    using RG = fpipe::Ring<D, R>;
    // The pipelined loop over the interior tiles 0 .. nkb_int - 1 (an even
    // count, at least two; the edge tiles follow in the loops below).  K(j)
    // sits in K slot j % R and V(j) in V slot j % R, K loaded one tile ahead:
    // iteration j reads K(j+1) and V(j).  R = 2: it starts the copies of
    // K(j+2) and V(j+1) (one per slot in its first slots) after its barrier,
    // which certifies that K(j+1) and V(j) have landed and that every wave is
    // done with the slots of K(j) and V(j-1).  R = 4: it ends by starting the copies of K(j+3) and V(j+2) (of
    // tile nint - 1 again where those are past the interior, so that every
    // iteration has the same copies in flight), and its barrier, fence-free,
    // follows a wait that leaves the last iteration's copies in flight.
    if (nkb_int >= 2) {
      const int nint = nkb_int;
      auto load_k = [&](int slot, int k0) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(kh, (uint32_t)k0 * row_bytes, nbytes);
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
          copy_to_lds16(r, smem + (wave * LOADS + i) * 1024 + RG::k(slot), voff_k[i]);
      };
      auto load_v = [&](int slot, int k0) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(vh, (uint32_t)k0 * row_bytes, nbytes);
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
          copy_to_lds16(r, smem + (wave * LOADS + i) * 1024 + (R == 2 ? G::VBASE : RG::VB) + RG::v(slot),
                        voff_v[i]);
      };
      load_k(0, 0);
      load_v(0, 0);
      load_k(1, kBC);
      if constexpr (R == 4) {
        load_k(2, (nint > 2 ? 2 : nint - 1) * kBC);
        load_v(1, kBC);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * LOADS) : "memory");  // K(0) landed
        __builtin_amdgcn_s_barrier();
        // the V^T read addresses point into the V region for the loop
#pragma unroll
        for (int e = 0; e < D / 32; ++e) vaddr[e] += RG::VB;
      } else {
        // K(0) landed (V(0) and K(1) may still be in flight: S(0) overlaps them)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LOADS) : "memory");
        __builtin_amdgcn_s_barrier();
      }
      // S(0) ahead of the loop, as in the same-phase tile body.
      f32x16 sA[2], sB[2];
      {
        constexpr int NK = P::NS, AHEAD = 8;
        bf16x8 kf[NK];
        auto rd = [&](auto I) __attribute__((always_inline)) {
          constexpr int i = decltype(I)::value, t = i / 2, j = i % 2;
          kf[i] = read_b128<RG::k(0) + j * 32 * G::RB>(kaddr[t]);
        };
        static_for<AHEAD>(rd);
        static_for<NK>([&](auto I) __attribute__((always_inline)) {
          constexpr int i = decltype(I)::value, t = i / 2, j = i % 2;
          constexpr int issued = (AHEAD + i < NK) ? AHEAD + i : NK;
          wait_lds<issued - i - 1>(kf[i]);
          sA[j] = mfma_bf16(kf[i], qf[t], t == 0 ? f32x16{} : sA[j]);
          if constexpr (i + AHEAD < NK) rd(IC<i + AHEAD>{});
        });
      }
      float mx = max_halves(rowmax(sA));
      // The lazy offset of the same-phase body: raised past 8 binades, with
      // the rescale of l and O (after the previous tile's P.V MFMAs).
      auto raise_offset = [&](float mxc) __attribute__((always_inline)) {
        const float mb = mxc * scale_log2;
        const bool raise = mb > m + kLazy;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          const float m_new = raise ? mb : m;
          const float alpha = exp2_fast(m - m_new);
          m = m_new;
          l *= alpha;
          o_scale<D>(oacc, alpha);
        }
      };
      // Iteration j: K slot SK holds K(j+1), V slot SV holds V(j); cur = S(j),
      // nxt receives S(j+1).
      auto iter = [&](auto SK_, auto SV_, f32x16 (&cur)[2], f32x16 (&nxt)[2], int j)
                      __attribute__((always_inline)) {
        constexpr int SK = decltype(SK_)::value, SV = decltype(SV_)::value;
        if constexpr (R == 4) {
          // K(j+1) and V(j) landed, K(j+2) and V(j+1) may still be in flight
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LOADS) : "memory");
          __builtin_amdgcn_s_barrier();
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
        }
        // R = 2: the next tiles' copies go out one per slot in the first slots,
        // under the MFMAs (issued together after the barrier they stalled the
        // wave: at d = 256 sixteen 1 KB copies per wave; +7.6% at d = 256,
        // +6% on the 4-wave workgroups at d = 128)
        const __amdgpu_buffer_rsrc_t rkn =
            tile_rsrc(kh, (uint32_t)min(j + 2, nint - 1) * kBC * row_bytes, nbytes);
        const __amdgpu_buffer_rsrc_t rvn = tile_rsrc(vh, (uint32_t)(j + 1) * kBC * row_bytes, nbytes);
        const bool kn = j + 2 < nint;
        raise_offset(mx);
        const float neg_m = -m;
        float rsum = 0.f;
        uint32_t pw[16];  // P(j)^T as bf16 pairs
        float pe[32];     // its exponentials
        bf16x8 kf[P::NS];
        bf16x4 vlo[P::NP], vhi[P::NP];
        float ma = 0.f, mbx = 0.f;
        // read r of the iteration: K fragment r (r < NS), else half (r - NS) % 2
        // of V^T fragment (r - NS) / 2
        auto issue = [&](auto R_) __attribute__((always_inline)) {
          constexpr int r = decltype(R_)::value;
          if constexpr (r < P::NS) {
            kf[r] = read_b128<RG::k(SK) + (r % 2) * 32 * G::RB>(kaddr[r / 2]);
          } else {
            constexpr int k = (r - P::NS) / 2, half = (r - P::NS) % 2, t2 = k / P::NE,
                          e = k % P::NE;
            const bf16x4 x = read_tr16<RG::v(SV) + (16 * t2 + 8 * half) * G::RB>(vaddr[e]);
            if constexpr (half) vhi[k] = x; else vlo[k] = x;
          }
        };
        static_for<P::N>([&](auto S_) __attribute__((always_inline)) {
          constexpr int s = decltype(S_)::value;
          if constexpr (s == 0) {
            static_for<fpipe::kLook + 1>([&](auto K_) __attribute__((always_inline)) {
              issue(IC<decltype(K_)::value>{});
            });
          }
          constexpr int W = P::issued(s - 1) - P::need(s);
          static_assert(W >= 0 && W <= 15, "wait count");
          if constexpr (s < P::NS) {
            constexpr int t = s / 2, jb = s % 2;
            wait_lds<W>(kf[s]);
            nxt[jb] = mfma_bf16(kf[s], qf[t], t == 0 ? f32x16{} : nxt[jb]);
          } else {
            constexpr int k = s - P::NS, t2 = k / P::NE, e = k % P::NE;
            asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(vlo[k]), "+v"(vhi[k]) : "n"(W));
            const bf16x8 vf = bf16x8{vlo[k][0], vlo[k][1], vlo[k][2], vlo[k][3],
                                     vhi[k][0], vhi[k][1], vhi[k][2], vhi[k][3]};
            const bf16x8 pb = __builtin_bit_cast(
                bf16x8, i32x4{(int)pw[4 * t2], (int)pw[4 * t2 + 1], (int)pw[4 * t2 + 2],
                              (int)pw[4 * t2 + 3]});
            pv_mfma<D, e == 0>(oacc[e], vf, pb);
          }
          constexpr int first = P::issued(s - 1) + 1;
          static_for<P::issued(s) - P::issued(s - 1)>([&](auto K_) __attribute__((always_inline)) {
            issue(IC<first + decltype(K_)::value>{});
          });
          if constexpr (R == 2 && s < 2 * LOADS) {
            constexpr int i = s % LOADS;
            if constexpr (s < LOADS) {
              if (kn) copy_to_lds16(rkn, smem + (wave * LOADS + i) * 1024 + RG::k(SV), voff_k[i]);
            } else {
              copy_to_lds16(rvn, smem + (wave * LOADS + i) * 1024 + G::VBASE + RG::v(SK), voff_v[i]);
            }
          }
          static_for<32>([&](auto E_) __attribute__((always_inline)) {
            constexpr int v = decltype(E_)::value;
            if constexpr (P::exp_slot(v) == s) {
              constexpr int t2 = v / 8, sl = v % 8;
              pe[v] = exp2_fast(__builtin_fmaf(cur[t2 >> 1][8 * (t2 & 1) + sl], scale_log2, neg_m));
              rsum += pe[v];
              if constexpr (v % 2 == 1) {
                pw[v / 2] = pack_bf16x2(pe[v - 1], pe[v]);
                asm volatile("" : "+v"(rsum), "+v"(pw[v / 2]));
              } else {
                asm volatile("" : "+v"(rsum), "+v"(pe[v]));
              }
            }
          });
          if constexpr (s >= P::kMax0) {
            constexpr int r = 2 * (s - P::kMax0);
            if constexpr (s == P::kMax0) {
              ma = fmaxf(nxt[0][0], nxt[0][1]);
              mbx = fmaxf(nxt[1][0], nxt[1][1]);
            } else {
              ma = fmaxf(ma, fmaxf(nxt[0][r], nxt[0][r + 1]));
              mbx = fmaxf(mbx, fmaxf(nxt[1][r], nxt[1][r + 1]));
            }
            asm volatile("" : "+v"(ma), "+v"(mbx));
          }
          // one fence per slot, at its end: a second one between the MFMA and
          // the reads measured 2% slower
          __builtin_amdgcn_sched_barrier(0);
        });
        l += rsum;
        mx = max_halves(fmaxf(ma, mbx));
        if constexpr (R == 4) {
          load_k((SK + 2) % 4, min(j + 3, nint - 1) * kBC);
          load_v((SV + 2) % 4, min(j + 2, nint - 1) * kBC);
        }
      };
      if constexpr (R == 4) {
        // nint - 1 iterations (an odd count), four per trip; iteration j has
        // K slot (j+1) % 4, V slot j % 4, S(j) in sA for even j
        int j = 0;
        for (; j + 4 <= nint - 1; j += 4) {
          iter(IC<1>{}, IC<0>{}, sA, sB, j);
          iter(IC<2>{}, IC<1>{}, sB, sA, j + 1);
          iter(IC<3>{}, IC<2>{}, sA, sB, j + 2);
          iter(IC<0>{}, IC<3>{}, sB, sA, j + 3);
        }
        iter(IC<1>{}, IC<0>{}, sA, sB, j);
        if (j + 1 < nint - 1) {
          iter(IC<2>{}, IC<1>{}, sB, sA, j + 1);
          iter(IC<3>{}, IC<2>{}, sA, sB, j + 2);
        }
      } else {
        for (int j = 0; j + 2 < nint - 1; j += 2) {
          iter(IC<1>{}, IC<0>{}, sA, sB, j);
          iter(IC<0>{}, IC<1>{}, sB, sA, j + 1);
        }
        iter(IC<1>{}, IC<0>{}, sA, sB, nint - 2);
      }
      // The last interior tile's P.V: V(nint-1) in V slot (nint-1) % R,
      // S(nint-1) in sB.
      {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const uint32_t vs = (uint32_t)RG::v((nint - 1) % R);
        // V^T operands in halves of at most four 32-dim blocks (d = 256: two)
        constexpr int NEH = P::NE <= 4 ? P::NE : 4;
        bf16x8 vf[4][NEH];
        auto read_half = [&](auto HF) __attribute__((always_inline)) {
          constexpr int hf = decltype(HF)::value;
#pragma unroll
          for (int e = 0; e < NEH; ++e)
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) {
              const bf16x4 lo = read_tr16<0>(vaddr[hf * NEH + e] + vs + 16 * t2 * G::RB);
              const bf16x4 hi = read_tr16<0>(vaddr[hf * NEH + e] + vs + (16 * t2 + 8) * G::RB);
              vf[t2][e] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        };
        read_half(IC<0>{});
        raise_offset(mx);
        const float neg_m = -m;
        float rsum = 0.f;
        bf16x8 pb[4];
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2)
#pragma unroll
          for (int sl = 0; sl < 8; ++sl) {
            const float pv =
                exp2_fast(__builtin_fmaf(sB[t2 >> 1][8 * (t2 & 1) + sl], scale_log2, neg_m));
            rsum += pv;
            pb[t2][sl] = (__bf16)pv;
          }
        l += rsum;
        static_for<P::NE / NEH>([&](auto HF) __attribute__((always_inline)) {
          constexpr int hf = decltype(HF)::value;
          if constexpr (hf > 0) read_half(HF);
          lds_wait_v(vf);
          static_for<4>([&](auto T2) __attribute__((always_inline)) {
            constexpr int t2 = decltype(T2)::value;
            static_for<NEH>([&](auto E) __attribute__((always_inline)) {
              constexpr int e = decltype(E)::value;
              pv_mfma<D, e == 0>(oacc[hf * NEH + e], vf[t2][e], pb[t2]);
            });
          });
        });
      }
      kb = nint;
      if constexpr (R == 4) {
#pragma unroll
        for (int e = 0; e < D / 32; ++e) vaddr[e] -= RG::VB;
      }
      __syncthreads();  // every wave is done with the loop's slots
    }
  }
  if (kb < nkb) LOAD_TILE(0, kb * kBC);
  for (; kb < nkb_int; kb += 2) {
    STEP(0, kb, false);
    STEP(1, kb + 1, false);
  }
  for (; kb < nkb; kb += 2) {
    STEP(0, kb, true);
    if (kb + 1 < nkb) STEP(1, kb + 1, true);
  }
#undef STEP

#undef LOAD_TILE
  // Epilogue: one normalisation per row, bf16 store, log-sum-exp.  The rows
  // are stored whole through LDS (every wave is done with the K/V tiles after
  // the barrier; each wave takes 32 * 2D bytes of them): 1-8% faster than
  // stores from the accumulator layout, most with many heads at N = 4096,
  // except causal d = 256 (1% slower), which stores directly.
  const float lt = sum_halves(l);
  const float inv = 1.f / lt;
  o_fence<D>(oacc);
  if constexpr (!(CAUSAL && D > 128)) {
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

// NW waves per workgroup (32 query rows each): 8 for long sequences (one
// workgroup per CU, K/V tiles shared by 256 rows), 4 for short ones (two
// workgroups per CU, so one's start-up and epilogue overlap the other's tiles).
//
// Non-causal: one workgroup per (b, h, query block).  With xcd_remap, all
// query blocks of the query heads that share one K/V head run on one XCD
// (their K/V stay in that XCD's L2), and XCD x takes the K/V heads x, x + 8,
// ... (measured 0-2% faster than contiguous ranges of heads per XCD).
//
// Causal, nunits > 0 (a persistent, resident kernel: FlashAttention-3 report,
// section 5.1): unit u = query blocks nqb-1-p and p
// (p = u % npair) of head u / npair, whose visible key counts add up to the
// same for every p, so every unit costs the same.  The grid is one slot per
// workgroup that fits on the GPU; slot s takes units s, s + gridDim.x, ...
// (heavier block of a unit first).  With xcd_remap the units of one head stay
// on one XCD.  Causal, nunits == 0: one workgroup per query block, heaviest
// first, dispatched by the hardware as CUs free up.
template <int D, bool CAUSAL, int NW, bool PIPE>
__global__ __launch_bounds__(64 * NW, D > 128 ? 1 : 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int H, int Hkv, int N, float scale_log2,
    int nqb, int xcd_remap, int nunits) {
  using G = Geo<D>;
  constexpr int kSmem = PIPE ? fpipe::Ring<D, fpipe::ring<D, NW>()>::kBytes : 2 * G::STAGE;
  static_assert(kSmem >= 2 * G::STAGE, "the same-phase stages fit");
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];
  if constexpr (!persistent<D, CAUSAL>()) {
    const int L = blockIdx.x;
    int bh, qb;
    if (xcd_remap) {
      // The hardware deals workgroups to the 8 XCDs round robin (L % 8).
      // XCD x takes the K/V head groups x, x + 8, ... (a group: the H / Hkv
      // query heads that read one K/V head), all query blocks of a group
      // together, so a group's K/V stays in one XCD's L2 and the groups an
      // XCD runs at a time are not neighbours in memory.
      const int g = H / Hkv;
      const int per_group = g * nqb;
      const int x = L & 7, j = L >> 3;
      const int rem = j % per_group;
      bh = ((j / per_group) * 8 + x) * g + rem / nqb;
      qb = rem % nqb;
    } else {
      bh = L / nqb;
      qb = L % nqb;
    }
    attend_block<D, CAUSAL, NW, PIPE>(smem, Q, K, V, O, LSE, H, Hkv, N, scale_log2, bh,
                                CAUSAL ? nqb - 1 - qb : qb);
  } else {
    // One call site for both causal modes (a second inlined copy of the
    // block would not fit the registers).
    const int npair = (nqb + 1) / 2;
    const int nslot = nunits > 0 ? nunits : (int)gridDim.x;
    int s = blockIdx.x, second = 0;  // unit (or block) slot; which block of the unit
#pragma nounroll
    while (s < nslot) {
      // Work items per query head: units (pairs) or single blocks.  With
      // xcd_remap, slot s runs on XCD s % 8 (the grid is a multiple of 8),
      // which takes the K/V head groups x, x + 8, ... as in the non-causal
      // kernel.
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
      attend_block<D, CAUSAL, NW, PIPE>(smem, Q, K, V, O, LSE, H, Hkv, N, scale_log2, bh, qblk);
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

template <int D, bool CAUSAL, int NW, bool PIPE>
hipError_t launch_nw(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                     int Hkv, int N, float scale, hipStream_t stream) {
  constexpr int kBR = 32 * NW;
  const int nqb = (N + kBR - 1) / kBR;
  int64_t grid = (int64_t)B * H * nqb;
  int64_t nunits = 0;
  if constexpr (persistent<D, CAUSAL>()) {
    const int64_t units = (int64_t)B * H * ((nqb + 1) / 2);
    static std::atomic<int> resident{0};
    const int ncu = current_cu_count();
    const int per_cu = resident_per_cu(attn_fwd_bf16_kernel<D, CAUSAL, NW, PIPE>, 64 * NW, resident);
    if (ncu <= 0 || per_cu <= 0) return hipErrorInvalidDevice;
    // At most two slots per CU: at d = 64 three 4-wave workgroups fit, but a
    // third slot per CU measured 2-8% slower on most causal shapes.
    const int64_t slots = (int64_t)ncu * (per_cu < 2 ? per_cu : 2);
    // Blocks no more than the CUs: one workgroup each, all at once (a pair
    // would be the longer path).  Otherwise pairs, if they fill the slots in
    // whole rounds: with a last round less than 90% full, the hardware's own
    // dispatch of the single blocks (heaviest first) packs better.
    const int64_t rounds = (units + slots - 1) / slots;
    if (grid > ncu && (units <= slots || units * 10 >= rounds * slots * 9)) {
      nunits = units;
      grid = units < slots ? units : slots;
    }
  }
  // the K/V head groups (B * Hkv of them) split evenly over the 8 XCDs, and a
  // persistent grid a multiple of 8 (each slot stays on one XCD)
  const int remap = (((int64_t)B * Hkv) % 8 == 0 && grid % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, NW, PIPE>), dim3((unsigned)grid), dim3(64 * NW), 0,
                     stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse,
                     H, Hkv, N, scale * kLog2e, nqb, remap, (int)nunits);
  return hipGetLastError();
}

// Four-wave workgroups win where a workgroup has few key tiles (short
// sequences) or the causal work is uneven; crossover measured on the 16384-
// token sweep (B = 16384 / N): N <= 1024 (d=128) / 2048 (d=64) non-causal,
// N <= 4096 / 8192 causal.
template <int D, bool CAUSAL, bool PIPE = false>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int Hkv, int N, float scale, hipStream_t stream) {
  // d = 256: one wave per SIMD (Q fragments and O take 192 registers), so
  // always four waves, with the pipelined loop (+11.6% at B2 H16 N8192,
  // causal +14%).
  if constexpr (D > 128) {
    return launch_nw<D, CAUSAL, 4, PIPE>(q, k, v, o, lse, B, H, Hkv, N, scale, stream);
  } else {
    const int small_n = (CAUSAL ? 4096 : 1024) * (128 / D);
    // the pipelined loop on the 4-wave workgroups: non-causal at every N;
    // causal from N = 1024 (+2-9% at N = 1024-8192; at N = 512 the blocks
    // have too few interior tiles: -5.5%)
    if (N <= small_n) {
      if (CAUSAL && N < 1024)
        return launch_nw<D, CAUSAL, 4, false>(q, k, v, o, lse, B, H, Hkv, N, scale, stream);
      return launch_nw<D, CAUSAL, 4, PIPE>(q, k, v, o, lse, B, H, Hkv, N, scale, stream);
    }
    return launch_nw<D, CAUSAL, 8, PIPE>(q, k, v, o, lse, B, H, Hkv, N, scale, stream);
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Hkv, int N, int d, bool causal,
                                float softmax_scale, hipStream_t stream, bool same_phase) {
  // The pipelined loop (the same results as the same-phase loop, measured
  // 1-9% faster at d = 64 and 128, 12-14% at d = 256): non-causal at every
  // head dim and workgroup size, causal from N = 1024; same_phase selects the
  // same-phase loop there too, for comparison.
  if (!same_phase && d == 128)
    return causal ? launch<128, true, true>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream)
                  : launch<128, false, true>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream);
  if (!same_phase && d == 64)
    return causal ? launch<64, true, true>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream)
                  : launch<64, false, true>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream);
  if (!same_phase && d == 256)
    return causal ? launch<256, true, true>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream)
                  : launch<256, false, true>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream);
  if (d == 256)
    return causal ? launch<256, true>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream)
                  : launch<256, false>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream);
  if (d == 128)
    return causal ? launch<128, true>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream)
                  : launch<128, false>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream)
                : launch<64, false>(q, k, v, o, lse, B, H, Hkv, N, softmax_scale, stream);
}

}  // namespace exattn
