"""FP8 path on the GPU vs the CPU oracle.

blockquant_hadamard: e4m3 codes bit-exact and scales equal to the oracle's
emulation of the pre-pass (both take the quantise decision in fp32, with the
same butterfly order).

attn_fwd_fp8 (fed the oracle's own codes and scales):
  * per element vs the oracle's FP8 emulation: |o_gpu - o_emul| within the
    bound of tests/fp8_bound.py (bf16 output rounding, a possible one-step
    e4m3 flip of each P lying within the fp32 error of a rounding midpoint,
    fp32 accumulation slack), with the RMS of err/bound <= 0.45;
  * tight norm gate vs the emulation: RMSE(GPU - emulation) <= 0.1 x
    RMSE(emulation - exact);
  * vs exact fp64 attention on the unrotated bf16 inputs: RMSE <= 3e-2 on the
    outlier distribution of the FlashAttention-3 report (section 4.3), and
    below the per-tensor-scaled run without rotation on both outlier
    distributions.  On the x30-outlier workload the measured RMSE is reported
    next to the emulation floor of the scheme (about 9e-2, above 3e-2).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_bound import check_fp8, emulation_with_bound
from gpu_helpers import DEV, err_stats, rows_of, say, to_np

import exact_attention_74_amd as ea

pytestmark = pytest.mark.gpu


def _bf16_host(w):
    return [workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w)]


def _dev_bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16).to(DEV)


def _gpu_quant(x_host, signs, block_rows):
    s = None if signs is None else torch.from_numpy(signs).to(DEV)
    c, sc = ea.blockquant_hadamard(_dev_bf16(x_host), s, block_rows)
    torch.cuda.synchronize()
    return c.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 130, 300, 1024])
@pytest.mark.parametrize("rotate", [True, False])
@pytest.mark.parametrize("block_rows", [128, 0])
def test_blockquant_bit_exact(d, N, rotate, block_rows):
    say(f"blockquant d{d} N{N} rot{rotate} br{block_rows}")
    w = workloads.Workload("bq", 2, 3, N, d, False, seed=40 + N, dist="outlier30")
    x = _bf16_host(w)[0]
    signs = workloads.gen_signs(d) if rotate else None
    c_gpu, s_gpu = _gpu_quant(x, signs, block_rows)
    c_ref, s_ref = oracle.blockquant_hadamard(x, signs, block_rows)
    assert np.array_equal(s_gpu, s_ref), np.abs(s_gpu - s_ref).max()
    assert np.array_equal(c_gpu, c_ref), f"{np.count_nonzero(c_gpu != c_ref)} codes differ"


def test_blockquant_full_size_heads():
    """The fp8 workload's full tensor on the GPU; a few (b, h) heads checked."""
    w = workloads.FP8
    say(w.name + " blockquant")
    x = _bf16_host(w)[0]
    signs = workloads.gen_signs(w.d)
    c_gpu, s_gpu = _gpu_quant(x, signs, 128)
    for b, h in ((0, 0), (1, 7), (3, 15)):
        c_ref, s_ref = oracle.blockquant_hadamard(x[b:b + 1, :, h:h + 1], signs, 128)
        assert np.array_equal(s_gpu[b:b + 1, h:h + 1], s_ref)
        assert np.array_equal(c_gpu[b:b + 1, :, h:h + 1], c_ref)


def test_blockquant_zero_block_and_signs_identity():
    say("blockquant zero block")
    x = workloads.to_bf16_f32(workloads.gen_random((1, 256, 2, 64), 41))
    x[:, :128] = 0.0
    c, s = _gpu_quant(x, workloads.gen_signs(64), 128)
    assert np.all(s[:, :, 0] == 1.0) and not (c[:, :128] & 0x7F).any()
    c_ref, s_ref = oracle.blockquant_hadamard(x, workloads.gen_signs(64), 128)
    assert np.array_equal(c, c_ref) and np.array_equal(s, s_ref)


def _quant_all(q, k, v, signs, block_rows):
    """The oracle's codes and scales for Q, K (rotated if signs) and V."""
    q8, sq = oracle.blockquant_hadamard(q, signs, block_rows)
    k8, sk = oracle.blockquant_hadamard(k, signs, block_rows)
    v8, sv = oracle.blockquant_hadamard(v, None, block_rows)
    return q8, k8, v8, sq, sk, sv


def _gpu_fp8(q8, k8, v8, sq, sk, sv, scale, causal):
    t = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (q8, k8, v8, sq, sk, sv)]
    o, lse = ea.attn_fwd_fp8(*t, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


def _rmse(a, b):
    return float(np.sqrt(np.mean((np.asarray(a, np.float64) - b) ** 2)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [100, 256, 1000])
def test_fp8_attention_vs_emulation_full(causal, d, N):
    _fp8_vs_emulation(causal, d, N)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [384, 640, 1152, 1300])
def test_fp8_d256_pipelined_vs_emulation(causal, N):
    """The pipelined loop of head dim 256 against the emulation.
    Non-causal: one, three and seven iterations over the interior tiles, each
    followed by one whole edge tile (N = 384, 640, 1152), and nine followed by
    a ragged tail (N = 1300).  Causal: the blocks' tiles before their
    diagonal (query blocks 2 and up), then the diagonal and ragged tiles."""
    _fp8_vs_emulation(causal, 256, N)


def _fp8_vs_emulation(causal, d, N):
    w = workloads.Workload(f"fp8_n{N}_d{d}", 2, 3, N, d, causal, seed=50 + N, dist="outlier_sd10")
    say(w.name + ("_causal" if causal else ""))
    q, k, v = _bf16_host(w)
    signs = workloads.gen_signs(d)
    qs = _quant_all(q, k, v, signs, 128)
    o, lse = _gpu_fp8(*qs, w.softmax_scale, causal)
    o_em, l_em, bound = emulation_with_bound(*qs, w.softmax_scale, causal)
    o_ex, l_ex = oracle.naive_attention(q, k, v, w.softmax_scale, causal)
    check_fp8(o, o_em, bound, w.name)
    e_kernel = _rmse(o, o_em)
    e_scheme = _rmse(o_em, o_ex)
    lerr = float(np.abs(lse - l_em).max())
    print(f"{w.name}: rmse(gpu-emul)={e_kernel:.3e} rmse(emul-exact)={e_scheme:.3e} "
          f"rmse(gpu-exact)={_rmse(o, o_ex):.3e} lse(gpu-emul)={lerr:.3e}", flush=True)
    assert e_kernel <= 0.1 * e_scheme
    assert lerr <= 1e-3
    assert np.isfinite(o).all()


@pytest.mark.parametrize("w", [workloads.FP8_PAGE, workloads.FP8], ids=lambda w: w.name)
def test_fp8_full_size_rows_and_baseline(w):
    """Full fp8 workload on the GPU (pre-pass and attention); 128 sampled rows
    in each of four (b, h) heads checked.  Blocks never straddle heads, so the
    oracle quantises just those heads."""
    say(w.name)
    q, k, v = _bf16_host(w)
    signs = workloads.gen_signs(w.d)
    ts = torch.from_numpy(signs).to(DEV)
    tq, tk, tv = (_dev_bf16(x) for x in (q, k, v))

    def gpu_path(sg, br):
        q8, sq = ea.blockquant_hadamard(tq, sg, br)
        k8, sk = ea.blockquant_hadamard(tk, sg, br)
        v8, sv = ea.blockquant_hadamard(tv, None, br)
        o, _ = ea.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, softmax_scale=w.softmax_scale)
        torch.cuda.synchronize()
        return to_np(o)

    o_fa3 = gpu_path(ts, 128)
    o_base = gpu_path(None, 0)
    got_fa3, got_base, ref_ex, ref_em, bounds = [], [], [], [], []
    for b, h in ((0, 0), (1, 5), (2, 10), (3, 15)):
        sl = [x[b:b + 1, :, h:h + 1] for x in (q, k, v)]
        rows = workloads.sample_rows(1, 1, w.N, 128, seed=77 + h)
        o_ex, _ = oracle.naive_attention_rows(*sl, w.softmax_scale, False, rows)
        o_em, _, bd = emulation_with_bound(*_quant_all(*sl, signs, 128), w.softmax_scale, False,
                                           rows=rows)
        i = rows[:, 2]
        got_fa3.append(o_fa3[b, i, h])
        got_base.append(o_base[b, i, h])
        ref_ex.append(o_ex)
        ref_em.append(o_em)
        bounds.append(bd)
    o_fa3, o_base, o_ex, o_em = (np.concatenate(a) for a in (got_fa3, got_base, ref_ex, ref_em))
    check_fp8(o_fa3, o_em, np.concatenate(bounds), w.name)
    e_fa3, e_base, e_em = _rmse(o_fa3, o_ex), _rmse(o_base, o_ex), _rmse(o_em, o_ex)
    e_kernel = _rmse(o_fa3, o_em)
    rel = e_fa3 / float(np.sqrt(np.mean(o_ex ** 2)))
    print(f"{w.name}: rmse fa3-fp8={e_fa3:.3e} (rel {rel:.3e}) per-tensor/no-rotation={e_base:.3e} "
          f"emulation floor={e_em:.3e} gpu-vs-emulation={e_kernel:.3e} "
          f"ratio={e_base / e_fa3:.2f}", flush=True)
    assert e_kernel <= 0.1 * e_em
    assert e_fa3 < e_base
    if w.dist == "outlier_sd10":
        assert e_fa3 <= 3e-2


def test_fp8_lse_vs_exact_normal_inputs():
    w = workloads.Workload("fp8_normal", 1, 4, 2048, 128, False, seed=60)
    say(w.name)
    q, k, v = _bf16_host(w)
    qs = _quant_all(q, k, v, workloads.gen_signs(128), 128)
    o, lse = _gpu_fp8(*qs, w.softmax_scale, False)
    o_ex, l_ex = oracle.naive_attention(q, k, v, w.softmax_scale, False)
    rows = workloads.sample_rows(w.B, w.H, w.N, 256, seed=61)
    o_em, _, bound = emulation_with_bound(*qs, w.softmax_scale, False, rows=rows)
    check_fp8(rows_of(o, rows), o_em, bound, w.name)
    mx, rmse = err_stats(o, o_ex)
    print(f"fp8 normal: max={mx:.3e} rmse={rmse:.3e} lse={np.abs(lse - l_ex).max():.3e}")
    assert rmse <= 3e-3 and np.abs(lse - l_ex).max() <= 5e-2


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_d256_full_size_sampled_rows(causal):
    """Head dim 256 at full size (B2 H8 N8192, the report's 2048-wide model
    at d = 256): GPU pre-pass and attention, 128 sampled rows in each of three
    heads against the emulation and exact attention."""
    w = workloads.Workload("fp8_b2h8n8192d256", 2, 8, 8192, 256, causal, seed=31,
                           dist="outlier_sd10")
    say(w.name + ("_causal" if causal else ""))
    q, k, v = _bf16_host(w)
    signs = workloads.gen_signs(w.d)
    ts = torch.from_numpy(signs).to(DEV)
    tq, tk, tv = (_dev_bf16(x) for x in (q, k, v))
    q8, sq = ea.blockquant_hadamard(tq, ts, 128)
    k8, sk = ea.blockquant_hadamard(tk, ts, 128)
    v8, sv = ea.blockquant_hadamard(tv, None, 128)
    o, lse = ea.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=causal, softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    o, lse = to_np(o), lse.cpu().numpy().astype(np.float64)
    got, ref_ex, ref_em, l_got, l_em, bounds = [], [], [], [], [], []
    for b, h in ((0, 0), (1, 3), (1, 7)):
        sl = [x[b:b + 1, :, h:h + 1] for x in (q, k, v)]
        rows = workloads.sample_rows(1, 1, w.N, 128, seed=91 + h)
        o_ex, _ = oracle.naive_attention_rows(*sl, w.softmax_scale, causal, rows)
        o_em, le, bd = emulation_with_bound(*_quant_all(*sl, signs, 128), w.softmax_scale,
                                            causal, rows=rows)
        i = rows[:, 2]
        got.append(o[b, i, h])
        l_got.append(lse[b, h, i])
        ref_ex.append(o_ex)
        ref_em.append(o_em)
        l_em.append(le)
        bounds.append(bd)
    o, o_ex, o_em = (np.concatenate(a) for a in (got, ref_ex, ref_em))
    check_fp8(o, o_em, np.concatenate(bounds), w.name)
    e_kernel, e_em, e_ex = _rmse(o, o_em), _rmse(o_em, o_ex), _rmse(o, o_ex)
    lerr = float(np.abs(np.concatenate(l_got) - np.concatenate(l_em)).max())
    print(f"{w.name}: rmse gpu-vs-emulation={e_kernel:.3e} emulation floor={e_em:.3e} "
          f"gpu-vs-exact={e_ex:.3e} lse={lerr:.3e}", flush=True)
    assert e_kernel <= 0.1 * e_em
    assert e_ex <= 3e-2
    assert lerr <= 1e-3


@pytest.mark.parametrize("B,H,N,d", [(2, 16, 5000, 128), (3, 5, 3000, 64), (2, 8, 8192, 128),
                                     (4, 16, 4096, 128), (1, 8, 32768, 128)])
def test_fp8_causal_schedules_sampled_rows(B, H, N, d):
    """Causal FP8 work in both schedules.  One workgroup per query block:
    B2 H16 N5000 (its 320 equal-cost block pairs would leave the second round
    of 256 slots a quarter full) and B3 H5 N3000 d64 (180 blocks, fewer than
    the CUs).  Persistent slots over block pairs: B2 H8 N8192 (one round),
    B4 H16 N4096 (two) and the long single request B1 H8 N32768 (512 pairs of
    up to 256 key tiles each).  Sampled rows against the emulation, and a
    second run bit for bit."""
    w = workloads.Workload(f"fp8_causal_sched_b{B}h{H}n{N}d{d}", B, H, N, d, True, seed=70 + N,
                           dist="outlier_sd10")
    say(w.name)
    q, k, v = _bf16_host(w)
    qs = _quant_all(q, k, v, workloads.gen_signs(d), 128)
    o, lse = _gpu_fp8(*qs, w.softmax_scale, True)
    o2, lse2 = _gpu_fp8(*qs, w.softmax_scale, True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    rows = workloads.sample_rows(B, H, N, 384, seed=N + 3)
    o_em, l_em, bound = emulation_with_bound(*qs, w.softmax_scale, True, rows=rows)
    o_ex, _ = oracle.naive_attention_rows(q, k, v, w.softmax_scale, True, rows)
    got = rows_of(o, rows)
    check_fp8(got, o_em, bound, w.name)
    e_kernel, e_scheme = _rmse(got, o_em), _rmse(o_em, o_ex)
    lerr = float(np.abs(lse[rows[:, 0], rows[:, 1], rows[:, 2]] - l_em).max())
    print(f"{w.name}: rmse(gpu-emul)={e_kernel:.3e} rmse(emul-exact)={e_scheme:.3e} "
          f"lse={lerr:.3e}", flush=True)
    assert e_kernel <= 0.1 * e_scheme
    assert lerr <= 1e-3
