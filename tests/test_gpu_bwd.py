"""bf16 attention gradients on the GPU vs the fp64 oracle ([FA3-report]
section 3.4: FA-2's recompute strategy).

The forward runs first (attn_fwd_bf16 gives O and LSE, as a caller would have
them); attn_bwd_bf16 then returns dQ, dK, dV.  The oracle differentiates the
exact fp64 forward on the same bf16-rounded inputs.

Gate, derived from the roundings of the bf16 path (U = 2^-8 bounds one bf16
rounding, as in the forward tests; products accumulate in fp32):
  * P rounded to bf16 for dV = P^T dO:   |err dV| <= U (|dV| + P^T |dO|)
  * O arrives rounded to bf16, so D_i = sum dO O is off by at most
    dD_i = U sum_c |dO_ic O_ic|; dS = P (dP - D) rounded to bf16:
    |err dS_ij| <= U |dS_ij| + P_ij dD_i = e_ij
  * dQ = scale dS K, dK = scale dS^T Q, each rounded to bf16 at the end:
    |err dQ| <= U |dQ| + scale e |K|,  |err dK| <= U |dK| + scale e^T |Q|
Every element must lie inside its bound (times 1 + 1e-3, plus 1e-6 of the
largest gradient for fp32 summation), the RMS of err/bound must stay below
0.35 (a rounding error is rarely at its worst case), and the normalised RMSE
(RMSE / RMS of the exact gradient) must stay below 1e-2 wherever that RMS is
not negligible (at N = 1 the exact dQ and dK are zero).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, say, to_np

import exact_attention_74_amd as ea

pytestmark = pytest.mark.gpu

U = 2.0 ** -8
GATE_NRMSE, GATE_RATIO_RMS = 1e-2, 0.35


def _inputs(B, N, H, d, seed):
    w = workloads.Workload("bwd", B, H, N, d, False, seed=seed)
    q, k, v = (workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w))
    do = workloads.to_bf16_f32(workloads.gen_random((B, N, H, d), seed + 1000))
    return q, k, v, do


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(DEV)


def _gpu(q, k, v, do, causal, scale):
    qd, kd, vd, dod = (_dev(x) for x in (q, k, v, do))
    o, lse = ea.attn_fwd_bf16(qd, kd, vd, causal=causal, softmax_scale=scale)
    dq, dk, dv = ea.attn_bwd_bf16(qd, kd, vd, o, lse, dod, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return to_np(dq), to_np(dk), to_np(dv), to_np(o)


def _bounds(q, k, v, do, o_bf16, scale, causal):
    """Per-element bounds (dQ, dK, dV) of the bf16 path, from the exact P, dS."""
    qh, kh, vh, doh, oh = (np.transpose(np.asarray(x, np.float64), (0, 2, 1, 3))
                           for x in (q, k, v, do, o_bf16))
    B, H, N, d = qh.shape
    out = [np.empty((B, H, N, d)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            s = scale * (qh[b, h] @ kh[b, h].T)
            if causal:
                s[np.triu_indices(N, 1)] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = p @ vh[b, h]
            dd = np.sum(doh[b, h] * o, axis=1)
            ds = p * (doh[b, h] @ vh[b, h].T - dd[:, None])
            dq, dk, dv = scale * ds @ kh[b, h], scale * ds.T @ qh[b, h], p.T @ doh[b, h]
            e = U * np.abs(ds) + p * (U * np.sum(np.abs(doh[b, h] * oh[b, h]), axis=1))[:, None]
            out[0][b, h] = U * np.abs(dq) + scale * e @ np.abs(kh[b, h])
            out[1][b, h] = U * np.abs(dk) + scale * e.T @ np.abs(qh[b, h])
            out[2][b, h] = U * (np.abs(dv) + p.T @ np.abs(doh[b, h]))
    return [np.transpose(x, (0, 2, 1, 3)) for x in out]


def _check(got, ref, bounds, tag):
    for name, g, r, bd in zip(("dQ", "dK", "dV"), got, ref, bounds):
        err = np.abs(g - r)
        tol = bd * (1 + 1e-3) + 1e-6 * np.abs(r).max()
        ratio = err / tol
        rms_ref = float(np.sqrt(np.mean(r ** 2)))
        nrmse = float(np.sqrt(np.mean(err ** 2)) / rms_ref) if rms_ref > 1e-3 else 0.0
        print(f"{tag} {name}: max_abs={err.max():.3e} nrmse={nrmse:.3e} "
              f"err/bound max={ratio.max():.3f} rms={np.sqrt(np.mean(ratio ** 2)):.3f}", flush=True)
        assert np.isfinite(g).all()
        assert ratio.max() <= 1.0, (name, float(ratio.max()))
        assert np.sqrt(np.mean(ratio ** 2)) <= GATE_RATIO_RMS, name
        assert nrmse <= GATE_NRMSE, (name, nrmse)


@pytest.mark.parametrize("causal", [False, True])
# N = 192 and 320 at d = 128: an odd number of whole 64-row query tiles, so
# the dK/dV kernel's unmasked middle loop (whole pairs) ends one tile early
# and the last whole tile goes through the masked tail; 640 likewise at d = 64.
@pytest.mark.parametrize("N,d", [(1, 64), (37, 128), (64, 64), (129, 128), (192, 128), (256, 64),
                                  (300, 128), (320, 128), (640, 64), (1000, 64), (1000, 128)])
def test_bwd_full_parity(causal, N, d):
    tag = f"bwd_n{N}_d{d}" + ("_causal" if causal else "")
    say(tag)
    q, k, v, do = _inputs(2, N, 3, d, seed=300 + N + d)
    scale = d ** -0.5
    dq, dk, dv, o = _gpu(q, k, v, do, causal, scale)
    ref = oracle.attention_backward(q, k, v, do, scale, causal)
    _check((dq, dk, dv), ref, _bounds(q, k, v, do, o, scale, causal), tag)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_full_size_heads(causal):
    """B2 H16 N4096 d128 on the GPU; two whole heads checked against the oracle
    (every key's gradient needs every query)."""
    B, N, H, d = 2, 4096, 16, 128
    tag = f"bwd_b{B}h{H}n{N}d{d}" + ("_causal" if causal else "")
    say(tag)
    q, k, v, do = _inputs(B, N, H, d, seed=41)
    scale = d ** -0.5
    dq, dk, dv, o = _gpu(q, k, v, do, causal, scale)
    heads = np.array([[0, 0], [1, 13]])
    ref = oracle.attention_backward_heads(q, k, v, do, scale, causal, heads)
    for r, (b, h) in enumerate(heads):
        sl = lambda x: x[b:b + 1, :, h:h + 1, :]  # noqa: E731
        got = [x[b, :, h, :][None, :, None, :] for x in (dq, dk, dv)]
        refr = [x[r][None, :, None, :] for x in ref]
        bd = _bounds(sl(q), sl(k), sl(v), sl(do), sl(o), scale, causal)
        _check(got, refr, bd, f"{tag} head ({b},{h})")


def test_bwd_deterministic_and_workspace():
    q, k, v, do = _inputs(1, 700, 4, 128, seed=5)
    qd, kd, vd, dod = (_dev(x) for x in (q, k, v, do))
    o, lse = ea.attn_fwd_bf16(qd, kd, vd, causal=True)
    nbytes = ea.lib().attn_bwd_bf16_workspace_bytes(1, 4, 700)
    assert nbytes == 8 * 4 * 700
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    a = ea.attn_bwd_bf16(qd, kd, vd, o, lse, dod, causal=True, workspace=ws)
    b = ea.attn_bwd_bf16(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_empty_is_noop():
    z = torch.zeros((0, 16, 2, 64), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((0, 2, 16), dtype=torch.float32, device=DEV)
    dq, dk, dv = ea.attn_bwd_bf16(z, z, z, z, lse, z)
    torch.cuda.synchronize()
    assert dq.numel() == 0


@pytest.mark.parametrize("H,Hkv,N,d,causal", [(4, 2, 300, 128, False), (4, 2, 300, 128, True),
                                               (6, 1, 500, 64, True), (8, 2, 1000, 128, False)])
def test_bwd_gqa_full_parity(H, Hkv, N, d, causal):
    """Grouped-query gradients: dK, dV of a K/V head sum over its group.  The
    bound is the per-query-head bound (K/V written out per head) summed over
    the group."""
    tag = f"bwd_gqa_h{H}kv{Hkv}_n{N}_d{d}" + ("_causal" if causal else "")
    say(tag)
    w = workloads.Workload("bwdg", 2, H, N, d, False, seed=600 + N + H)
    q = workloads.to_bf16_f32(workloads.gen_qkv(w)[0])
    k, v = (workloads.to_bf16_f32(x) for x in workloads.gen_qkv_gqa(2, N, H, Hkv, d, 610 + N)[1:])
    do = workloads.to_bf16_f32(workloads.gen_random((2, N, H, d), 620 + N))
    scale = d ** -0.5
    qd, kd, vd, dod = (_dev(x) for x in (q, k, v, do))
    o, lse = ea.attn_fwd_bf16_gqa(qd, kd, vd, causal=causal, softmax_scale=scale)
    dq, dk, dv = ea.attn_bwd_bf16(qd, kd, vd, o, lse, dod, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    got = [to_np(x) for x in (dq, dk, dv)]
    assert got[1].shape == k.shape and got[2].shape == v.shape
    ref = oracle.attention_backward(q, k, v, do, scale, causal)
    r = H // Hkv
    kr, vr = (np.repeat(x, r, axis=2) for x in (k, v))
    bq, bk, bv = _bounds(q, kr, vr, do, to_np(o), scale, causal)
    B_, N_ = bk.shape[0], bk.shape[1]
    bk = bk.reshape(B_, N_, Hkv, r, d).sum(axis=3)
    bv = bv.reshape(B_, N_, Hkv, r, d).sum(axis=3)
    _check(got, ref, (bq, bk, bv), tag)
