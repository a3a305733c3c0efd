"""bf16 attention forward on the GPU vs the fp64 CPU oracle.

Gate (both masks): max-abs error <= 1e-2 and RMSE <= 2e-3 on N(0,1) inputs, the
stated bf16 tolerance.  A tighter internal gate catches kernel bugs that the
stated tolerance would let through.  It bounds each output element by the two
roundings of the bf16 path, each at most 2^-8 relative:
  * P rounded to bf16 before P.V: |error| <= 2^-8 (P|V|)_i.
  * O rounded to bf16 at the end: |error| <= 2^-8 |O|_i.
So the bound is |o - o_ref| <= 2^-8 (|O| + P|V|) (1 + 1e-3) + 1e-5.  The gate
requires every element inside it, the RMS of error/bound <= 0.35 (a rounding
error is rarely near its worst case), and the LSE error <= 2e-5.  One key
masked wrongly moves the LSE by about p_j / sum p, so the LSE gate is
sensitive to masking errors.  The oracle sees the same
bf16-rounded inputs upcast to fp64, so the gate measures the kernel, not the
input rounding.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (DEV, bf16_inputs, err_stats, lse_rows, rows_of, say, to_dev_bf16, to_np)

import exact_attention_74_amd as ea

pytestmark = pytest.mark.gpu

GATE_MAX, GATE_RMSE = 1e-2, 2e-3
INT_NRMS, INT_LSE = 0.35, 2e-5
U_BF16 = 2.0 ** -8


def _check(o, lse, o_ref, lse_ref, tag, o_absv=None):
    """o_absv: the oracle's attention applied to |V| (P|V|), for the rounding bound."""
    mx, rmse = err_stats(o, o_ref)
    lerr = float(np.abs(lse - lse_ref).max())
    ratio = nrms = float("nan")
    if o_absv is not None:
        bound = U_BF16 * (np.abs(o_ref) + o_absv) * (1 + 1e-3) + 1e-5
        r = np.abs(o - o_ref) / bound
        ratio, nrms = float(r.max()), float(np.sqrt(np.mean(r ** 2)))
    print(f"{tag}: max_abs={mx:.3e} rmse={rmse:.3e} lse_max={lerr:.3e} "
          f"err/bound max={ratio:.3f} rms={nrms:.3f}", flush=True)
    assert mx <= GATE_MAX and rmse <= GATE_RMSE, (mx, rmse)
    assert lerr <= INT_LSE, lerr
    if o_absv is not None:
        assert ratio <= 1.0 and nrms <= INT_NRMS, (ratio, nrms)


def _run(dev_qkv, causal, scale):
    o, lse = ea.attn_fwd_bf16(*dev_qkv, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_full_parity(causal):
    w = workloads.TINY_CAUSAL if causal else workloads.TINY
    say(w.name)
    host, dev = bf16_inputs(w)
    o, lse = _run(dev, causal, w.softmax_scale)
    o_ref, lse_ref = oracle.naive_attention(*host, w.softmax_scale, causal)
    absv, _ = oracle.naive_attention(host[0], host[1], np.abs(host[2]), w.softmax_scale, causal)
    _check(o, lse, o_ref, lse_ref, w.name, absv)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 37, 64, 129, 1000])
def test_ragged_full_parity(causal, d, N):
    """Several query/key tiles with a ragged tail (N not a multiple of 64/128)."""
    w = workloads.Workload(f"ragged_n{N}_d{d}", 2, 3, N, d, causal, seed=11 + N)
    say(w.name + ("_causal" if causal else ""))
    host, dev = bf16_inputs(w)
    o, lse = _run(dev, causal, w.softmax_scale)
    o_ref, lse_ref = oracle.naive_attention(*host, w.softmax_scale, causal)
    absv, _ = oracle.naive_attention(host[0], host[1], np.abs(host[2]), w.softmax_scale, causal)
    _check(o, lse, o_ref, lse_ref, w.name, absv)


@pytest.mark.parametrize("N,d,causal", [(1025, 128, False), (1500, 128, False), (2100, 64, False),
                                         (4097, 128, True), (8300, 64, True)])
def test_ragged_eight_wave_path(N, d, causal):
    """Lengths just past the short-sequence crossover take the 8-wave
    workgroups (256 query rows); ragged tails of 1 to 63 keys."""
    w = workloads.Workload(f"ragged8_n{N}_d{d}", 1, 3, N, d, causal, seed=31 + N)
    say(w.name + ("_causal" if causal else ""))
    host, dev = bf16_inputs(w)
    o, lse = _run(dev, causal, w.softmax_scale)
    if N <= 2100:
        o_ref, lse_ref = oracle.naive_attention(*host, w.softmax_scale, causal)
        absv, _ = oracle.naive_attention(host[0], host[1], np.abs(host[2]), w.softmax_scale, causal)
        _check(o, lse, o_ref, lse_ref, w.name, absv)
    else:
        rows = workloads.sample_rows(w.B, w.H, w.N, 512, seed=N)
        # the last rows of every head (the ragged q-block) are always checked
        tail = np.array([(0, h, n) for h in range(w.H) for n in range(N - 5, N)])
        rows = np.concatenate([rows, tail])
        o_ref, l_ref = oracle.naive_attention_rows(*host, w.softmax_scale, causal, rows)
        absv, _ = oracle.naive_attention_rows(host[0], host[1], np.abs(host[2]), w.softmax_scale,
                                              causal, rows)
        _check(rows_of(o, rows), lse_rows(lse, rows), o_ref, l_ref, w.name, absv)


@pytest.mark.parametrize("causal", [False, True])
def test_d96_zero_padded(causal):
    """d=96 zero-padded to 128 with scale 1/sqrt(96) equals d=96 attention."""
    w = workloads.Workload("pad96", 2, 4, 700, 128, causal, seed=21, d_logical=96)
    say(w.name)
    host, dev = bf16_inputs(w)
    o, lse = _run(dev, causal, w.softmax_scale)
    q, k, v = (x[..., :96] for x in host)
    o_ref, lse_ref = oracle.naive_attention(q, k, v, 1 / math.sqrt(96), causal)
    absv, _ = oracle.naive_attention(q, k, np.abs(v), 1 / math.sqrt(96), causal)
    _check(o[..., :96], lse, o_ref, lse_ref, w.name, absv)
    assert np.all(o[..., 96:] == 0.0)


@pytest.mark.parametrize("w", [workloads.MID, workloads.MID_CAUSAL, workloads.LONG],
                         ids=lambda w: w.name)
def test_full_size_sampled_rows(w):
    say(w.name)
    host, dev = bf16_inputs(w)
    o, lse = _run(dev, w.causal, w.softmax_scale)
    rows = workloads.sample_rows(w.B, w.H, w.N, 1024, seed=w.seed + 100)
    o_ref, l_ref = oracle.naive_attention_rows(*host, w.softmax_scale, w.causal, rows)
    absv, _ = oracle.naive_attention_rows(host[0], host[1], np.abs(host[2]), w.softmax_scale,
                                          w.causal, rows)
    _check(rows_of(o, rows), lse_rows(lse, rows), o_ref, l_ref, w.name, absv)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


@pytest.mark.parametrize("w", workloads.sweep(False) + workloads.sweep(True), ids=lambda w: w.name)
def test_sweep_sampled_rows(w):
    """All 36 configurations of the 16384-token sweep (N 512..16k x d 64, 96
    padded to 128, 128 x both masks), 512 sampled rows each."""
    say(w.name)
    host, dev = bf16_inputs(w)
    o, lse = _run(dev, w.causal, w.softmax_scale)
    rows = workloads.sample_rows(w.B, w.H, w.N, 512, seed=w.N)
    dl = w.d_logical or w.d
    q, k, v = (x[..., :dl] for x in host)
    o_ref, l_ref = oracle.naive_attention_rows(q, k, v, w.softmax_scale, w.causal, rows)
    absv, _ = oracle.naive_attention_rows(q, k, np.abs(v), w.softmax_scale, w.causal, rows)
    _check(rows_of(o, rows)[:, :dl], lse_rows(lse, rows), o_ref, l_ref, w.name, absv)


@pytest.mark.parametrize("B,H,N,d", [(2, 16, 5000, 128), (2, 16, 8192, 128), (3, 5, 3000, 128),
                                     (1, 7, 2500, 64), (4, 16, 4096, 128)])
def test_causal_schedules_sampled_rows(B, H, N, d):
    """Causal work runs persistent (workgroup slots take equal-cost pairs of
    query blocks) when there are more blocks than CUs and the pairs fill the
    slots in whole rounds, else one workgroup per query block.  Per-block:
    B2 H16 N5000 (320 pairs on 256 slots) and B1 H7 N2500 d64 (140 blocks);
    persistent: the others (several rounds, fewer pairs than slots).
    Sampled rows against the oracle, and a second run bit for bit."""
    w = workloads.Workload(f"causal_sched_b{B}h{H}n{N}d{d}", B, H, N, d, True, seed=40 + N)
    say(w.name)
    host, dev = bf16_inputs(w)
    o, lse = _run(dev, True, w.softmax_scale)
    o2, lse2 = _run(dev, True, w.softmax_scale)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    rows = workloads.sample_rows(B, H, N, 768, seed=N + 1)
    o_ref, l_ref = oracle.naive_attention_rows(*host, w.softmax_scale, True, rows)
    absv, _ = oracle.naive_attention_rows(host[0], host[1], np.abs(host[2]), w.softmax_scale,
                                          True, rows)
    _check(rows_of(o, rows), lse_rows(lse, rows), o_ref, l_ref, w.name, absv)


def test_causal_row0_equals_v0_bitwise():
    w = workloads.Workload("row0", 2, 4, 300, 128, True, seed=31)
    say(w.name)
    host, dev = bf16_inputs(w)
    o, _ = ea.attn_fwd_bf16(*dev, causal=True)
    assert torch.equal(o[:, 0], dev[2][:, 0])


def test_identical_value_rows():
    w = workloads.Workload("vrows", 1, 2, 513, 64, False, seed=32)
    say(w.name)
    host, dev = bf16_inputs(w)
    row = workloads.to_bf16_f32(workloads.gen_random((64,), 33))
    v = np.broadcast_to(row, host[2].shape).copy()
    o, _ = ea.attn_fwd_bf16(dev[0], dev[1], to_dev_bf16(v), causal=False)
    torch.cuda.synchronize()
    assert np.abs(to_np(o) - row).max() <= 4e-3 * max(1.0, np.abs(row).max())


def test_causal_prefix_independence_bitwise():
    w = workloads.Workload("prefix", 1, 2, 640, 128, True, seed=34)
    say(w.name)
    host, dev = bf16_inputs(w)
    o1, l1 = ea.attn_fwd_bf16(*dev, causal=True)
    k2, v2 = host[1].copy(), host[2].copy()
    k2[:, 300:] += 3.0
    v2[:, 300:] *= -2.0
    o2, l2 = ea.attn_fwd_bf16(dev[0], to_dev_bf16(k2), to_dev_bf16(v2), causal=True)
    assert torch.equal(o1[:, :300], o2[:, :300])
    assert torch.equal(l1[:, :, :300], l2[:, :, :300])
    assert not torch.equal(o1[:, 300:], o2[:, 300:])


def test_deterministic_bitwise():
    w = workloads.Workload("determinism", 2, 8, 2048, 128, False, seed=35)
    say(w.name)
    _, dev = bf16_inputs(w)
    o1, l1 = ea.attn_fwd_bf16(*dev)
    o2, l2 = ea.attn_fwd_bf16(*dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_lse_none_and_stream():
    """lse=NULL is accepted at the ABI, and work goes to the caller's stream."""
    w = workloads.Workload("stream", 1, 2, 256, 64, False, seed=36)
    say(w.name)
    host, dev = bf16_inputs(w)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o = torch.empty_like(dev[0])
        rc = ea.lib().attn_fwd_bf16(dev[0].data_ptr(), dev[1].data_ptr(), dev[2].data_ptr(),
                                    o.data_ptr(), None, 1, 2, 256, 64, 0, 0.125, s.cuda_stream)
    s.synchronize()
    assert rc == 0
    o_ref, _ = oracle.naive_attention(*host, 0.125, False)
    mx, rmse = err_stats(to_np(o), o_ref)
    assert mx <= GATE_MAX and rmse <= GATE_RMSE


def test_empty_problem_is_noop():
    say("empty")
    z = torch.empty((0, 128, 2, 64), dtype=torch.bfloat16, device=DEV)
    o, lse = ea.attn_fwd_bf16(z, z, z)
    assert o.shape == z.shape and lse.numel() == 0


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 100, 129, 700])
def test_d256_full_parity(causal, N):
    """Head dim 256 (four one-wave-per-SIMD waves per workgroup; V^T fragments in
    two halves); ragged N over several query and key tiles."""
    w = workloads.Workload(f"d256_n{N}", 2, 2, N, 256, causal, seed=500 + N)
    say(w.name + ("_causal" if causal else ""))
    host, dev = bf16_inputs(w)
    o, lse = _run(dev, causal, w.softmax_scale)
    o_ref, lse_ref = oracle.naive_attention(*host, w.softmax_scale, causal)
    absv, _ = oracle.naive_attention(host[0], host[1], np.abs(host[2]), w.softmax_scale, causal)
    _check(o, lse, o_ref, lse_ref, w.name, absv)


@pytest.mark.parametrize("causal", [False, True])
def test_d256_full_size_sampled_rows(causal):
    w = workloads.Workload("d256_b1h8n8192", 1, 8, 8192, 256, causal, seed=77)
    say(w.name + ("_causal" if causal else ""))
    host, dev = bf16_inputs(w)
    o, lse = _run(dev, causal, w.softmax_scale)
    rows = workloads.sample_rows(w.B, w.H, w.N, 384, seed=78)
    o_ref, l_ref = oracle.naive_attention_rows(*host, w.softmax_scale, causal, rows)
    absv, _ = oracle.naive_attention_rows(host[0], host[1], np.abs(host[2]), w.softmax_scale,
                                          causal, rows)
    _check(rows_of(o, rows), lse_rows(lse, rows), o_ref, l_ref, w.name, absv)


def _default_vs_same_phase(dev, causal, scale):
    o, lse = ea.attn_fwd_bf16(*dev, causal=causal, softmax_scale=scale)
    o0, lse0 = ea.attn_fwd_bf16_same_phase(*dev, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, lse0), "the two schedules differ"
    return to_np(o), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("N,d", [(128, 128), (129, 64), (640, 64), (1000, 128), (1025, 128),
                                 (1088, 128), (1100, 128), (1500, 128), (2048, 128), (2049, 64),
                                 (2112, 64), (2500, 64), (128, 256), (191, 256), (640, 256),
                                 (1000, 256)])
def test_pipelined_full_parity(N, d):
    """The pipelined loop (S(j+1) MFMAs between the exponentials of tile j),
    which attn_fwd_bf16 runs non-causal on 4-wave (short N, and d = 256 with O
    in the AGPR file) and 8-wave workgroups: every element against the oracle,
    and the outputs bit-identical to the same-phase schedule's.  N = 128 is
    the shortest pipelined run (one pair of tiles); N = 640, 1088 and 2112
    leave an odd whole tile after the pipelined pairs, the others a ragged
    tail of 1 to 63 keys."""
    w = workloads.Workload(f"pipe_n{N}_d{d}", 1, 3, N, d, False, seed=41 + N)
    say(w.name)
    host, dev = bf16_inputs(w)
    o, lse = _default_vs_same_phase(dev, False, w.softmax_scale)
    o_ref, lse_ref = oracle.naive_attention(*host, w.softmax_scale, False)
    absv, _ = oracle.naive_attention(host[0], host[1], np.abs(host[2]), w.softmax_scale, False)
    _check(o, lse, o_ref, lse_ref, w.name, absv)


@pytest.mark.parametrize("N", [300, 640, 1000])
def test_pipelined_causal_d256_full_parity(N):
    """Causal head dim 256: the pipelined loop over each block's tiles
    before its diagonal (blocks 1 and up), the same-phase loop over the
    diagonal and ragged tiles; every element against the oracle, and
    bit-identical to the same-phase schedule."""
    w = workloads.Workload(f"pipe_c_n{N}_d256", 1, 3, N, 256, True, seed=43 + N)
    say(w.name)
    host, dev = bf16_inputs(w)
    o, lse = _default_vs_same_phase(dev, True, w.softmax_scale)
    o_ref, lse_ref = oracle.naive_attention(*host, w.softmax_scale, True)
    absv, _ = oracle.naive_attention(host[0], host[1], np.abs(host[2]), w.softmax_scale, True)
    _check(o, lse, o_ref, lse_ref, w.name, absv)


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 16, 8192, 128, False), (2, 4, 8192, 128, True),
                                            (1, 3, 5000, 128, True), (1, 2, 8300, 64, True),
                                            (1, 4, 1024, 128, False),
                                            (1, 3, 3000, 64, False), (1, 3, 3000, 128, True),
                                            (1, 2, 700, 256, True), (2, 8, 8192, 256, False),
                                            (2, 8, 8192, 256, True), (2, 8, 4000, 256, True),
                                            (2, 4, 700, 128, True), (2, 4, 1500, 64, True),
                                            (2, 2, 1, 128, False)])
def test_schedules_sampled_rows(B, H, N, d, causal):
    """The bench shapes B2 H16 N8192 (d = 128) and B2 H8 N8192 (d = 256, both
    masks), d = 64 N = 3000, causal N = 5000, 8192 (d = 128), 8300 (d = 64)
    and 700, 4000 (d = 256; 4000: persistent slots, ragged), and the 4-wave
    causal workgroups at N = 3000 (d = 128) and 1500 (d = 64) through the
    pipelined loop (sampled rows against the oracle; causal blocks run it up
    to their diagonal), and the shapes that run the same-phase loop under both
    entry points (causal N < 1024, one token): bit-identical."""
    w = workloads.Workload(f"sched_b{B}h{H}n{N}d{d}", B, H, N, d, causal, seed=7 + N)
    say(w.name + ("_causal" if causal else ""))
    host, dev = bf16_inputs(w)
    o, lse = _default_vs_same_phase(dev, causal, w.softmax_scale)
    rows = workloads.sample_rows(B, H, N, 256, seed=N)
    o_ref, l_ref = oracle.naive_attention_rows(*host, w.softmax_scale, causal, rows)
    absv, _ = oracle.naive_attention_rows(host[0], host[1], np.abs(host[2]), w.softmax_scale,
                                          causal, rows)
    _check(rows_of(o, rows), lse_rows(lse, rows), o_ref, l_ref, w.name, absv)
