// C ABI of libexattn.so: argument validation, then dispatch to the gfx950
// launchers.  Every check runs before the first HIP call, so a rejected call
// launches nothing and touches no output.
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "exattn.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 24;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// A byte range [p, p + n) of device memory; p == NULL (an optional argument
// left out) or n == 0 takes part in no overlap.
struct Span {
  const void* p;
  int64_t n;
};

bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.n <= 0 || b.n <= 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a.p), pb = reinterpret_cast<uintptr_t>(b.p);
  return pa < pb + (uintptr_t)b.n && pb < pa + (uintptr_t)a.n;
}

// True when an output overlaps an input or another output (inputs may share
// memory with each other: they are only read).
bool aliased(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (const Span& i : ins)
      if (overlap(*o, i)) return true;
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlap(*o, *o2)) return true;
  }
  return false;
}

// fp32 scale slots per (b, h) of a sequence of N rows (one per 128 rows).
int64_t scale_blocks(int N) { return ((int64_t)N + 127) / 128; }

// elt: bytes per element of the Q/K/V inputs.  One batch entry of a tensor
// (N x H x d elements) must stay below 2 GiB: kernels address a head's rows
// with 32-bit buffer offsets.
int check_shape(int B, int H, int N, int d, int elt, bool allow_d256 = true) {
  if (B < 0 || H < 0 || N < 0) return EXATTN_ERR_SHAPE;
  if (d != 64 && d != 128 && !(allow_d256 && d == 256)) return EXATTN_ERR_SHAPE;
  if ((int64_t)N >= kMaxN) return EXATTN_ERR_SHAPE;
  if ((int64_t)N * H * d * elt >= (int64_t(1) << 31)) return EXATTN_ERR_SHAPE;
  const int64_t blocks = (int64_t)B * H * (((int64_t)N + 127) / 128);
  if (blocks >= (int64_t(1) << 31)) return EXATTN_ERR_SHAPE;
  return EXATTN_OK;
}

bool good_scale(float s) { return isfinite(s) && s > 0.f; }

// K/V head count: at least 1 (for H > 0) and dividing H.
bool good_heads(int H, int H_kv) { return H_kv > 0 ? H % H_kv == 0 : H == 0 && H_kv == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? EXATTN_OK : EXATTN_ERR_HIP; }

}  // namespace

extern "C" {

int exattn_abi_version(void) { return 9; }

const char* exattn_strerror(int code) {
  switch (code) {
    case EXATTN_OK: return "success";
    case EXATTN_ERR_NULL: return "a required pointer is NULL";
    case EXATTN_ERR_SHAPE:
      return "unsupported shape (negative size, d not in {64,128,256} (backward: {64,128}), too "
             "large, or H not a multiple of H_kv)";
    case EXATTN_ERR_ALIGN: return "pointer not aligned (tensors 16 bytes, scales/LSE 4 bytes)";
    case EXATTN_ERR_VALUE:
      return "invalid value (softmax_scale, causal, block_rows, or an output overlapping an "
             "input or another output)";
    case EXATTN_ERR_HIP: return "HIP error (no device or kernel launch failed)";
    case EXATTN_ERR_SCRATCH:
      return "problem too large for the fixed scratch of the no-allocation entry point "
             "(8 B H N bytes above EXATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

namespace {
int fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int H_kv, int N, int d, int causal, float softmax_scale, void* stream,
             bool same_phase) {
  int rc = check_shape(B, H, N, d, 2);
  if (rc) return rc;
  if (!good_heads(H, H_kv)) return EXATTN_ERR_SHAPE;
  if ((causal != 0 && causal != 1) || !good_scale(softmax_scale)) return EXATTN_ERR_VALUE;
  const int64_t bytes = (int64_t)B * N * H * d * 2;
  const int64_t kv_bytes = (int64_t)B * N * H_kv * d * 2;
  if (bytes == 0) return EXATTN_OK;
  if (!q || !k || !v || !o) return EXATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return EXATTN_ERR_ALIGN;
  if (aliased({{o, bytes}, {lse, (int64_t)B * H * N * 4}}, {{q, bytes}, {k, kv_bytes}, {v, kv_bytes}}))
    return EXATTN_ERR_VALUE;
  return hip_status(exattn::launch_attn_fwd_bf16(q, k, v, o, lse, B, H, H_kv, N, d, causal != 0,
                                                 softmax_scale, (hipStream_t)stream, same_phase));
}
}  // namespace

int attn_fwd_bf16_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int H_kv, int N, int d, int causal, float softmax_scale,
                      void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, H_kv, N, d, causal, softmax_scale, stream, false);
}

int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int N, int d, int causal, float softmax_scale, void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, H, N, d, causal, softmax_scale, stream, false);
}

int attn_fwd_bf16_same_phase(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int N, int d, int causal, float softmax_scale,
                             void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, H, H, N, d, causal, softmax_scale, stream, true);
}

int attn_fwd_fp8_gqa(const void* q8, const void* k8, const void* v8, const float* q_scale,
                     const float* k_scale, const float* v_scale, void* o, float* lse, int B, int H,
                     int H_kv, int N, int d, int causal, float softmax_scale, void* stream) {
  int rc = check_shape(B, H, N, d, 1);
  if (rc) return rc;
  if (!good_heads(H, H_kv)) return EXATTN_ERR_SHAPE;
  if ((causal != 0 && causal != 1) || !good_scale(softmax_scale)) return EXATTN_ERR_VALUE;
  const int64_t in_bytes = (int64_t)B * N * H * d;
  const int64_t kv_bytes = (int64_t)B * N * H_kv * d;
  if (in_bytes == 0) return EXATTN_OK;
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o) return EXATTN_ERR_NULL;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16) ||
      !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      (lse && !aligned(lse, 4)))
    return EXATTN_ERR_ALIGN;
  const int64_t out_bytes = 2 * in_bytes;
  const int64_t sq_bytes = (int64_t)B * H * scale_blocks(N) * 4;
  const int64_t skv_bytes = (int64_t)B * H_kv * scale_blocks(N) * 4;
  if (aliased({{o, out_bytes}, {lse, (int64_t)B * H * N * 4}},
              {{q8, in_bytes}, {k8, kv_bytes}, {v8, kv_bytes}, {q_scale, sq_bytes},
               {k_scale, skv_bytes}, {v_scale, skv_bytes}}))
    return EXATTN_ERR_VALUE;
  return hip_status(exattn::launch_attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B,
                                                H, H_kv, N, d, causal != 0, softmax_scale,
                                                (hipStream_t)stream));
}

int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale,
                 const float* k_scale, const float* v_scale, void* o, float* lse, int B, int H,
                 int N, int d, int causal, float softmax_scale, void* stream) {
  return attn_fwd_fp8_gqa(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, H, N, d, causal,
                          softmax_scale, stream);
}

long long attn_bwd_bf16_workspace_bytes(int B, int H, int N) {
  if (B < 0 || H < 0 || N < 0) return EXATTN_ERR_SHAPE;
  return 8LL * B * H * N;
}

int attn_bwd_bf16_gqa(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* workspace, int B, int H, int H_kv, int N, int d, int causal,
                      float softmax_scale, void* stream) {
  int rc = check_shape(B, H, N, d, 2, /*allow_d256=*/false);
  if (rc) return rc;
  if (!good_heads(H, H_kv)) return EXATTN_ERR_SHAPE;
  if ((causal != 0 && causal != 1) || !good_scale(softmax_scale)) return EXATTN_ERR_VALUE;
  // the per-row prep kernel runs 16 rows per workgroup
  if ((int64_t)B * N * H >= (int64_t(1) << 35)) return EXATTN_ERR_SHAPE;
  const int64_t bytes = (int64_t)B * N * H * d * 2;
  if (bytes == 0) return EXATTN_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return EXATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 4))
    return EXATTN_ERR_ALIGN;
  const int64_t lse_bytes = (int64_t)B * H * N * 4;
  const int64_t ws_bytes = 2 * lse_bytes;
  const int64_t kv_bytes = (int64_t)B * N * H_kv * d * 2;
  // Outputs and workspace must not overlap any input or each other.
  if (aliased({{dq, bytes}, {dk, kv_bytes}, {dv, kv_bytes}, {workspace, ws_bytes}},
              {{q, bytes}, {k, kv_bytes}, {v, kv_bytes}, {o, bytes}, {dout, bytes},
               {lse, lse_bytes}}))
    return EXATTN_ERR_VALUE;
  return hip_status(exattn::launch_attn_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, workspace, B,
                                                 H, H_kv, N, d, causal != 0, softmax_scale,
                                                 (hipStream_t)stream));
}

int attn_bwd_bf16_noalloc(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                          int H, int H_kv, int N, int d, int causal, float softmax_scale,
                          void* stream) {
  int rc = check_shape(B, H, N, d, 2, /*allow_d256=*/false);
  if (rc) return rc;
  if (!good_heads(H, H_kv)) return EXATTN_ERR_SHAPE;
  if ((causal != 0 && causal != 1) || !good_scale(softmax_scale)) return EXATTN_ERR_VALUE;
  if ((int64_t)8 * B * H * N > (int64_t)exattn::bwd_scratch_bytes()) return EXATTN_ERR_SCRATCH;
  const int64_t bytes = (int64_t)B * N * H * d * 2;
  if (bytes == 0) return EXATTN_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return EXATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return EXATTN_ERR_ALIGN;
  const int64_t lse_bytes = (int64_t)B * H * N * 4;
  const int64_t kv_bytes = (int64_t)B * N * H_kv * d * 2;
  if (aliased({{dq, bytes}, {dk, kv_bytes}, {dv, kv_bytes}},
              {{q, bytes}, {k, kv_bytes}, {v, kv_bytes}, {o, bytes}, {dout, bytes},
               {lse, lse_bytes}}))
    return EXATTN_ERR_VALUE;
  return hip_status(exattn::launch_attn_bwd_bf16_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H,
                                                         H_kv, N, d, causal != 0, softmax_scale,
                                                         (hipStream_t)stream));
}

int attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, float* workspace, int B, int H,
                  int N, int d, int causal, float softmax_scale, void* stream) {
  return attn_bwd_bf16_gqa(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, H, N, d, causal,
                           softmax_scale, stream);
}

int blockquant_hadamard(const void* x, void* x8, float* scale, const float* signs, int B, int H,
                        int N, int d, int block_rows, void* stream) {
  int rc = check_shape(B, H, N, d, 2);
  if (rc) return rc;
  if (block_rows != 0 && block_rows != 128) return EXATTN_ERR_VALUE;
  const int64_t n = (int64_t)B * N * H * d;
  if (n == 0) return EXATTN_OK;
  if (!x || !x8 || !scale) return EXATTN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(scale, 4) || (signs && !aligned(signs, 4)))
    return EXATTN_ERR_ALIGN;
  const int64_t s_bytes = (int64_t)B * H * scale_blocks(N) * 4;
  if (aliased({{x8, n}, {scale, s_bytes}}, {{x, 2 * n}, {signs, (int64_t)d * 4}}))
    return EXATTN_ERR_VALUE;
  return hip_status(
      exattn::launch_blockquant(x, x8, scale, signs, B, H, N, d, block_rows, (hipStream_t)stream));
}

int rope_blockquant_hadamard(const void* x, void* x8, float* scale, const float* signs,
                             const float* rope_cos, const float* rope_sin, int rope_interleaved,
                             int B, int H, int N, int d, int block_rows, void* stream) {
  int rc = check_shape(B, H, N, d, 2);
  if (rc) return rc;
  if (block_rows != 0 && block_rows != 128) return EXATTN_ERR_VALUE;
  if (rope_interleaved != 0 && rope_interleaved != 1) return EXATTN_ERR_VALUE;
  const int64_t n = (int64_t)B * N * H * d;
  if (n == 0) return EXATTN_OK;
  if (!x || !x8 || !scale || !rope_cos || !rope_sin) return EXATTN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(scale, 4) || (signs && !aligned(signs, 4)) ||
      !aligned(rope_cos, 16) || !aligned(rope_sin, 16))
    return EXATTN_ERR_ALIGN;
  const int64_t s_bytes = (int64_t)B * H * scale_blocks(N) * 4;
  const int64_t table_bytes = (int64_t)N * (d / 2) * 4;
  if (aliased({{x8, n}, {scale, s_bytes}},
              {{x, 2 * n}, {signs, (int64_t)d * 4}, {rope_cos, table_bytes},
               {rope_sin, table_bytes}}))
    return EXATTN_ERR_VALUE;
  return hip_status(exattn::launch_rope_blockquant(x, x8, scale, signs, rope_cos, rope_sin,
                                                   rope_interleaved != 0, B, H, N, d, block_rows,
                                                   (hipStream_t)stream));
}

}  // extern "C"
