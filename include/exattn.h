/*
 * exattn -- fused exact attention forward for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libexattn.so.  Plain pointers and sizes only.
 *
 * The operation is exact softmax attention,
 *     O = softmax(scale * Q K^T [+ causal mask]) V,
 * computed tile by tile with the online-softmax recurrence (running row max m
 * and row sum l, one final normalisation) so that the N x N score matrix never
 * reaches device memory ("深度解读报告：FlashAttention-3（2024）", zako-mio
 * knowledge base, section 3 and section 3.1-3.2; "Efficient Attention &
 * FlashAttention", talentme M4-054, FA2's query-block parallelism and single
 * final normalisation).  The FP8 entry points implement the report's section
 * 3.3 low-precision scheme: per-block scales on Q, K and V and incoherent
 * processing (Q and K multiplied by a random +-1 diagonal times a Hadamard
 * matrix, which leaves Q K^T unchanged).
 *
 * Conventions shared by every entry point
 *   Layout      Q, K, V and O are BSHD: (batch B, seqlen N, heads H, head dim d),
 *               contiguous, the layout of the FlashAttention-3 Python
 *               interface (0539edu blog on FlashAttention V3, section 4.2).
 *               Element (b, n, h, c) is at ((b*N + n)*H + h)*d + c.
 *   Sizes       B, H, N >= 0 (any of them 0: nothing to do, returns 0 once
 *               the sizes and values are valid; pointers may then be NULL);
 *               d in {64, 128, 256}; the backward takes d in {64, 128} (other
 *               head dims are zero-padded by the caller to the next of these,
 *               keeping softmax_scale = 1/sqrt(d_original); the same blog,
 *               section 3.1); B*H*ceil(N/128) < 2^31; N < 2^24;
 *               N*H*d*(bytes per input element) < 2^31 (one batch entry of
 *               a tensor below 2 GiB: rows are addressed with 32-bit offsets).
 *   Memory      every pointer is device memory owned by the caller; the
 *               library allocates and frees nothing and keeps no state
 *               between calls.  Tensor pointers must be 16-byte aligned
 *               (64-byte alignment is recommended), scale/LSE pointers 4-byte.
 *   Streams     every call is asynchronous on `stream` (a hipStream_t; NULL is
 *               the default stream).  Device faults surface at the caller's
 *               next synchronisation.
 *   Errors      0 on success, a negative EXATTN_ERR_* code otherwise.  All
 *               arguments are validated before any HIP call, in the order
 *               sizes, values, empty problem, NULL, alignment, aliasing; on a validation
 *               error nothing is launched and no output is touched.  No C++
 *               exception crosses the ABI.  Thread-safe.
 *   Aliasing    no output (O, LSE, e4m3 codes, scales, gradients, workspace)
 *               may overlap an input (tensors, scales, signs, RoPE tables) or
 *               another output: EXATTN_ERR_VALUE.  Inputs may overlap each
 *               other.  Sizes are those of the arguments' documented shapes.
 *   Causal      key j is visible to query i iff j <= i.
 *   Outputs     O is bfloat16 (round to nearest even from fp32);
 *               LSE[b, h, i] = ln sum_j exp(scale * q_i . k_j) over visible
 *               keys, fp32, laid out [B, H, N] (the softmax statistic kept for
 *               a backward pass, 0539edu blog section 5.4).  lse may be NULL.
 */
#ifndef EXATTN_H
#define EXATTN_H

#ifdef __cplusplus
extern "C" {
#endif

#define EXATTN_OK 0
#define EXATTN_ERR_NULL (-1)  /* a required pointer is NULL                        */
#define EXATTN_ERR_SHAPE (-2) /* negative size, unsupported d, or too large       */
#define EXATTN_ERR_ALIGN (-3) /* a pointer is not aligned as required             */
#define EXATTN_ERR_VALUE (-4) /* bad softmax_scale/causal/block_rows, or aliasing */
#define EXATTN_ERR_HIP (-5)   /* no HIP device, or a launch failed                */
#define EXATTN_ERR_SCRATCH (-6) /* too large for attn_bwd_bf16_noalloc's scratch */

/* Bytes of the fixed per-GPU scratch array behind attn_bwd_bf16_noalloc. */
#define EXATTN_NOALLOC_SCRATCH_BYTES (16 << 20)

/*
 * bf16 attention forward.
 *   q, k, v      bfloat16 BSHD inputs.
 *   o            bfloat16 BSHD output (must not alias q, k or v).
 *   lse          fp32 [B, H, N] output, or NULL.
 *   causal       0 or 1.
 *   softmax_scale  multiplies Q K^T; finite and > 0 (usually 1/sqrt(d)).
 * The score matrix is never materialised: each workgroup owns a block of
 * query rows of one (b, h) and streams K/V blocks through LDS; each wave
 * software-pipelines the matrix products of the next key block under the
 * softmax of the current one (report section 3.2; see
 * attn_fwd_bf16_same_phase for where it does).
 */
int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, int d, int causal, float softmax_scale, void* stream);

/*
 * attn_fwd_bf16 with the same-phase schedule everywhere: both waves of a SIMD
 * issue a key tile's matrix products, then both run its softmax, one barrier
 * per tile.  attn_fwd_bf16 (and attn_fwd_bf16_gqa) use this schedule causal
 * with N < 1024; in
 * every other case they run the intra-wave pipelined schedule of the
 * FlashAttention-3 report, section 3.2, over a block's interior key tiles:
 * each wave issues the matrix products of S(j+1) = Q K(j+1)^T and of
 * O += P(j) V(j) one at a time between the exponentials and sums of block j's
 * softmax (the last, ragged or diagonal tiles run the same-phase loop).  The two
 * schedules compute every output element with the same operations in the
 * same order, so the results are identical bit for bit; this entry point
 * exists to compare them (the bench line's schedule leg).  Arguments,
 * validation and errors as in attn_fwd_bf16.
 */
int attn_fwd_bf16_same_phase(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int N, int d, int causal, float softmax_scale,
                             void* stream);

/*
 * FP8 (OCP e4m3) attention forward, FlashAttention-3 report section 3.3.
 *   q8, k8, v8   e4m3 codes, BSHD (one byte per element), as written by
 *                blockquant_hadamard (Q and K rotated with the same signs).
 *   q_scale, k_scale, v_scale   fp32 [B, H, ceil(N/128)]: the dequantised value
 *                of element (b, n, h, c) is code * scale[b, h, n / 128].
 *   o, lse, causal, softmax_scale   as in attn_fwd_bf16.
 * Each score tile is scaled by q_scale * k_scale * softmax_scale; the softmax
 * probabilities are rounded to e4m3 for the P.V product; V scales are folded
 * into the output rescaling.  Accumulation is fp32.
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                 const float* q_scale, const float* k_scale, const float* v_scale,
                 void* o, float* lse,
                 int B, int H, int N, int d, int causal, float softmax_scale, void* stream);

/*
 * Grouped-query / multi-query variants (FlashAttention-3 report, section 3.4:
 * MQA and GQA by FA-2's index mapping, so K/V are not duplicated in HBM).
 *   k, v (k8, v8)   BSHD with H_kv heads: [B, N, H_kv, d].
 *   k_scale, v_scale   fp32 [B, H_kv, ceil(N/128)].
 *   H_kv         K/V heads, >= 1, dividing H; query head h attends with K/V
 *                head h / (H / H_kv).  H_kv = H is plain multi-head attention,
 *                H_kv = 1 multi-query attention.
 * Everything else, outputs included (H heads), as in attn_fwd_bf16 and
 * attn_fwd_fp8; those two are these with H_kv = H.  H not a multiple of H_kv
 * (or H_kv < 1 with H > 0) returns EXATTN_ERR_SHAPE.
 */
int attn_fwd_bf16_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int H_kv, int N, int d, int causal, float softmax_scale,
                      void* stream);
int attn_fwd_fp8_gqa(const void* q8, const void* k8, const void* v8,
                     const float* q_scale, const float* k_scale, const float* v_scale,
                     void* o, float* lse,
                     int B, int H, int H_kv, int N, int d, int causal, float softmax_scale,
                     void* stream);

/*
 * Gradients of attn_fwd_bf16 (FlashAttention-3 report, section 3.4: FA-2's
 * recompute strategy, P rebuilt from Q, K and the saved log-sum-exp).
 *   q, k, v      the forward's bfloat16 BSHD inputs.
 *   o, lse       the forward's outputs (bf16 BSHD O and fp32 [B, H, N] LSE,
 *                natural log, as attn_fwd_bf16 writes them).
 *   dout         bfloat16 BSHD gradient of the loss with respect to O.
 *   dq, dk, dv   bfloat16 BSHD outputs: the gradients with respect to q, k, v.
 *   workspace    device memory of attn_bwd_bf16_workspace_bytes(B, H, N) bytes
 *                (fp32, 4-byte aligned), owned by the caller; its contents on
 *                entry do not matter and are overwritten.
 *   causal, softmax_scale   as in the forward call that produced o and lse.
 * With P = exp(scale Q K^T - LSE) and D_i = sum_c dO[i,c] O[i,c] per row:
 * dV = P^T dO, dS = P * (dO V^T - D), dQ = scale dS K, dK = scale dS^T Q.
 * P and dS are rounded to bf16 for the matrix products, which accumulate in
 * fp32.  Outputs must not overlap any input, each other or the workspace
 * (EXATTN_ERR_VALUE).  Three kernels are launched on `stream`.
 */
long long attn_bwd_bf16_workspace_bytes(int B, int H, int N);
int attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, float* workspace,
                  int B, int H, int N, int d, int causal, float softmax_scale, void* stream);
/*
 * The same for grouped-query / multi-query attention: k, v, dk, dv on H_kv
 * heads ([B, N, H_kv, d]; H a multiple of H_kv, query head h reads K/V head
 * h / (H / H_kv)); dk and dv are the sums over each K/V head's group of query
 * heads.  attn_bwd_bf16 is this with H_kv = H.
 */
int attn_bwd_bf16_gqa(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* workspace, int B, int H, int H_kv, int N, int d, int causal,
                      float softmax_scale, void* stream);

/*
 * attn_bwd_bf16_gqa without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, outputs and results are those
 * of attn_bwd_bf16_gqa (H_kv = H for plain multi-head attention); the
 * per-row D and LSE*log2(e) go to a fixed scratch array of
 * EXATTN_NOALLOC_SCRATCH_BYTES bytes held by the library on each GPU until
 * the process ends, so 8 * B * H * N must not exceed it (EXATTN_ERR_SCRATCH
 * otherwise, before any HIP call).  The call allocates nothing.  Every call
 * on one GPU uses that GPU's one scratch array: calls that overlap in time on
 * the same GPU (other streams, other host threads) race and must be
 * serialised by the caller.  The scratch is fully rewritten by each call
 * before it is read, so nothing needs clearing between calls.
 */
int attn_bwd_bf16_noalloc(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          int B, int H, int H_kv, int N, int d, int causal, float softmax_scale,
                          void* stream);

/*
 * FP8 pre-pass: optional incoherent rotation, then block quantisation to e4m3
 * (FlashAttention-3 report, sections 2.2 and 3.3).
 *   x        bfloat16 BSHD input.
 *   x8       e4m3 BSHD output (one byte per element).
 *   scale    fp32 [B, H, ceil(N/128)] output.
 *   signs    d floats, each +1 or -1, device memory; NULL = no rotation.
 *   block_rows  128: one scale per 128-row x d block of each (b, h);
 *               0: one scale for the whole tensor, written to every slot
 *               (the per-tensor baseline).
 * With signs, y = x diag(signs) H_d (Sylvester Hadamard, unnormalised fast
 * Walsh-Hadamard transform, butterfly strides 1, 2, 4, ... in fp32), and the
 * stored scale carries the 1/sqrt(d) of the orthonormal rotation.  Without
 * signs, y = x.  Per block: amax = max |y|; r = 448 / amax (fp32);
 * code = e4m3_rne(y * r); scale = amax / 448 (/ sqrt(d) when rotated).  A block
 * with amax 0 gets scale 1 and all-zero codes.  Dequantised: code * scale
 * approximates x M with M = diag(signs) H_d / sqrt(d), M M^T = I.
 * block_rows = 0 launches three kernels (block amax, global max, quantise);
 * otherwise one.
 */
int blockquant_hadamard(const void* x, void* x8, float* scale, const float* signs,
                        int B, int H, int N, int d, int block_rows, void* stream);

/*
 * The FP8 pre-pass fused with a rotary position embedding (FlashAttention-3
 * report, sections 2.2 and 3.3: quantisation riding on the memory-bound RoPE
 * pass, for Q and K).  As blockquant_hadamard, with each row n of x first
 * rotated pairwise:
 *   (x_a, x_b) -> (x_a cos[n][i] - x_b sin[n][i], x_a sin[n][i] + x_b cos[n][i])
 *   rope_interleaved = 1: pairs (a, b) = (2i, 2i+1);  0: (i, i + d/2).
 *   rope_cos, rope_sin   fp32 [N, d/2] device tables (16-byte aligned), the
 *                caller's frequency schedule and position offset.
 * The rotation is fp32 with every product and sum rounded separately; the
 * quantised values are those of the rotated rows.
 */
int rope_blockquant_hadamard(const void* x, void* x8, float* scale, const float* signs,
                             const float* rope_cos, const float* rope_sin, int rope_interleaved,
                             int B, int H, int N, int d, int block_rows, void* stream);

/* Static, never-NULL description of a return code. */
const char* exattn_strerror(int code);

/* Library ABI version (increments on any signature or semantic change). */
int exattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXATTN_H */
