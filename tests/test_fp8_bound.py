"""The FP8 parity bound (tests/fp8_bound.py) on the CPU.

An fp32 evaluation of the FP8 forward's recurrence (scores, running max,
exp2, e4m3 P, fp32 accumulation with per-tile rescale, bf16 output), written
here in numpy float32 in the kernel's order, must stay inside the bound the
GPU tests apply; and the bound must be tight enough that a wrong element (one key
dropped) falls outside it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_bound import U_BF16, e4m3_flip_step, emulation_with_bound

QB = 128


def fp32_forward(q8, k8, v8, sq, sk, sv, scale, causal):
    """O (bf16-rounded, as float64) of the FP8 forward evaluated in float32."""
    f32 = np.float32
    qv, kv, vv = (oracle.e4m3_decode(x).astype(f32) for x in (q8, k8, v8))
    B, N, H, d = qv.shape
    Hkv = kv.shape[2]
    o = np.zeros((B, N, H, d))
    c0 = f32(scale * (1.0 / math.log(2.0)))
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            for r0 in range(0, N, QB):
                qi = np.arange(r0, min(N, r0 + QB))
                m = np.full(len(qi), f32(-1e30))
                l = np.zeros(len(qi), f32)
                acc = np.zeros((len(qi), d), f32)
                svp = f32(1.0)
                for j, k0 in enumerate(range(0, N, QB)):
                    keys = np.arange(k0, min(N, k0 + QB))
                    if causal and k0 > qi.max():
                        break
                    s = (qv[b, qi, h] @ kv[b, keys, g].T).astype(f32)
                    if causal:
                        s[keys[None, :] > qi[:, None]] = -np.inf
                    ct = f32(f32(c0 * f32(sq[b, h, r0 // QB])) * f32(sk[b, g, j]))
                    mn = np.maximum(m, (s.max(axis=1) * ct).astype(f32))
                    alpha = np.exp2((m - mn).astype(f32)).astype(f32)
                    p = np.exp2((s * ct - mn[:, None]).astype(f32)).astype(f32)
                    pq = oracle.e4m3_decode(oracle.e4m3_encode(p)).astype(f32)
                    l = (l * alpha + p.sum(axis=1, dtype=f32)).astype(f32)
                    svc = f32(sv[b, g, j])
                    fct = (alpha * f32(svp / svc)).astype(f32)
                    acc = (acc * fct[:, None] + (pq @ vv[b, keys, g]).astype(f32)).astype(f32)
                    svp, m = svc, mn
                out = (acc * (svp / l)[:, None]).astype(f32)
                o[b, qi, h] = torch.from_numpy(out).to(torch.bfloat16).double().numpy()
    return o


def _case(N, d, causal, dist, seed):
    w = workloads.Workload("b", 1, 2, N, d, causal, seed=seed, dist=dist)
    q, k, v = (workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w))
    signs = workloads.gen_signs(d)
    q8, sq = oracle.blockquant_hadamard(q, signs, 128)
    k8, sk = oracle.blockquant_hadamard(k, signs, 128)
    v8, sv = oracle.blockquant_hadamard(v, None, 128)
    return (q8, k8, v8, sq, sk, sv), w.softmax_scale


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,dist", [(300, 64, "outlier_sd10"), (260, 128, "outlier30"),
                                      (129, 128, "normal")])
def test_fp32_evaluation_inside_bound(N, d, causal, dist):
    args, scale = _case(N, d, causal, dist, 300 + N)
    o_em, _, bound = emulation_with_bound(*args, scale, causal)
    o32 = fp32_forward(*args, scale, causal)
    r = np.abs(o32 - o_em) / bound
    assert r.max() <= 1.0, r.max()
    assert np.sqrt(np.mean(r ** 2)) <= 0.45


def test_bound_rejects_a_dropped_key_and_a_shifted_p():
    args, scale = _case(256, 64, False, "outlier_sd10", 77)
    o_em, _, bound = emulation_with_bound(*args, scale, False)
    q8, k8, v8, sq, sk, sv = args
    # key 17 left out of every row
    k8b = k8.copy()
    k8b[:, 17] = oracle.e4m3_encode(np.full(k8.shape[-1], -448.0))  # its score -> very negative
    o_drop = fp32_forward(q8, k8b, v8, sq, sk, sv, scale, False)
    assert (np.abs(o_drop - o_em) / bound).max() > 1.0
    # typical elements are bounded within a few bf16 roundings of |O|
    assert np.median(bound / (U_BF16 * np.abs(o_em) + 1e-9)) < 8.0


def test_flip_step_only_near_midpoints():
    mags = np.sort(oracle.e4m3_decode_table()[:127])
    assert not e4m3_flip_step(mags[1:], np.full(126, 1e-3)).any()   # exact values never flip
    mids = 0.5 * (mags[1:] + mags[:-1])
    st = e4m3_flip_step(mids[1:], np.full(125, 1e-9))
    np.testing.assert_array_equal(st, (mags[1:] - mags[:-1])[1:])
    assert e4m3_flip_step(np.array([0.0, 500.0]), np.array([1.0, 1.0])).sum() == 0.0
