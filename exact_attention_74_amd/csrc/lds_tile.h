// LDS tile plumbing shared by the bf16 attention kernels (forward and
// gradients): 64-row tiles of a BSHD tensor copied global -> LDS by
// buffer_load ... lds, XOR-swizzled 16-byte chunks, and LDS reads issued as
// assembly with explicit wait counts.
#pragma once

#include "common.h"

namespace exattn {
namespace {

constexpr int kBC = 64;  // rows (keys or queries) per LDS tile

typedef __attribute__((address_space(3))) void lds_void;

template <int D>
struct Geo {
  static constexpr int RB = 2 * D;           // bytes per key row
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RP = RB >= 256 ? 1 : 256 / RB;  // rows per 256-byte bank cycle (>= 1)
  static constexpr int TILE = kBC * RB;      // bytes per K or V tile
  static constexpr int STAGE = 2 * TILE;     // K + V
  // LDS byte offsets of stage st's K and V tiles.  d <= 128: stages are
  // [K V][K V].  d = 256: [K0 K1][V0 V1], with the V region's base (VBASE)
  // carried in the read addresses, so every immediate offset stays below 64 KB.
  static constexpr int VBASE = D > 128 ? 2 * TILE : 0;
  static constexpr int koff(int st) { return D > 128 ? st * TILE : st * STAGE; }
  static constexpr int voff(int st) { return D > 128 ? st * TILE : st * STAGE + TILE; }
  // chunk position of chunk c of row `row`
  __device__ static int swz_k(int row) { return (row / RP) % CPR; }
  __device__ static int swz_v(int row) { return 4 * ((row / RP) % (CPR / 4)); }
  // For a tile read both ways (ds_read_b128 rows and ds_read_b64_tr_b16):
  // swz_v plus (row / 4) % 4 in the low chunk bits.  16 consecutive rows get
  // 16 distinct chunk positions (row reads without bank conflicts), rows 0-3
  // keep swz_v's separation (transposed reads without conflicts), and
  // swz_b(row + 16) = swz_b(row), swz_b(row + 8) = swz_b(row) ^ 2, so the
  // transposed reads of rows + 8 use the address XOR 32 with the same
  // immediate offsets.
  __device__ static int swz_b(int row) { return swz_v(row) + (row / 4) % 4; }
};

// Asynchronous 16-byte-per-lane copy global -> LDS; lane i's chunk lands at
// lds_dst + 16 i (lds_dst is wave-uniform).  The scalar offset is always 0:
// the range check of a raw buffer covers the per-lane offset only, so a tile's
// position goes into the descriptor (tile_rsrc), never into soffset.
__device__ __forceinline__ void copy_to_lds16(__amdgpu_buffer_rsrc_t r, char* lds_dst,
                                              uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, voff, 0, 0, 0);
}

// LDS byte address of a generic pointer into LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Transposed LDS read (ds_read_b64_tr_b16) at LDS address addr + OFF, issued
// as assembly.  With the builtin, the compiler's wait-count pass assumes the
// read may see LDS that an in-flight buffer_load ... lds is writing and drains
// vmcnt first, which ties the next tile's prefetch to this tile's V reads; the
// tile loop's own vmcnt wait and barrier already order the two.  The result is
// valid only after lds_wait_v() has taken it.
template <int OFF>
__device__ __forceinline__ bf16x4 read_tr16(uint32_t addr) {
  bf16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// 16-byte LDS read at addr + OFF, issued as assembly so that the reads of a
// tile can run several MFMAs ahead; waited for with wait_lds<N>().
template <int OFF>
__device__ __forceinline__ bf16x8 read_b128(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Waits until at most N of this wave's LDS reads are outstanding, passing x
// through so that no use of x is scheduled before the wait.
template <int N>
__device__ __forceinline__ void wait_lds(bf16x8& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}

// Waits for every outstanding LDS read, passing the V^T fragments through so
// that no use of them is scheduled before the wait.
template <int NE>
__device__ __forceinline__ void lds_wait_v(bf16x8 (&vf)[4][NE]) {
  static_assert(NE == 4 || NE == 2, "four or two 32-dim blocks");
  if constexpr (NE == 4)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vf[0][0]), "+v"(vf[0][1]), "+v"(vf[0][2]), "+v"(vf[0][3]),
                   "+v"(vf[1][0]), "+v"(vf[1][1]), "+v"(vf[1][2]), "+v"(vf[1][3]),
                   "+v"(vf[2][0]), "+v"(vf[2][1]), "+v"(vf[2][2]), "+v"(vf[2][3]),
                   "+v"(vf[3][0]), "+v"(vf[3][1]), "+v"(vf[3][2]), "+v"(vf[3][3]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vf[0][0]), "+v"(vf[0][1]), "+v"(vf[1][0]), "+v"(vf[1][1]),
                   "+v"(vf[2][0]), "+v"(vf[2][1]), "+v"(vf[3][0]), "+v"(vf[3][1]));
}


}  // namespace
}  // namespace exattn
