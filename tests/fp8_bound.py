"""Per-element bound on |O_gpu - O_emulation| for the FP8 forward.

The oracle's FP8 emulation takes every step of the FP8 path in fp64 (scores,
exp, the running max) and rounds P to e4m3 against the running max, as the
kernel does.  The kernel takes the same steps in fp32; the two results differ
only by:

  1. O rounded to bf16 at the end:                <= 2^-8 |O|.
  2. P_gpu = P_emul (1 + eta) before the e4m3 rounding, with eta bounded from
     the arithmetic of each score: the e4m3 MFMA's dot product (on gfx950 its
     result is not the fp32-rounded exact sum: it deviates by up to 2^-14.9 of
     sum |q_k k_k| in a probe of 64-wide k-steps; EPS_MFMA = 2^-13 is taken,
     and tests/test_gpu_mfma_precision.py checks it on the device), the
     tile's scale product, the running max, the fused multiply-add and exp2.  Where P_emul lies within eta of a rounding
     midpoint the two roundings may pick neighbouring e4m3 values: a change of
     one e4m3 spacing in that P, times |V| sv, over l.
  3. The P.V MFMA (the same EPS_MFMA of sum P|V| per k-step), fp32
     accumulation of O and l over the keys, the per-tile rescale factors
     (exp2 of the max difference, the V-scale ratio by reciprocal) and the
     final division: relative slack kappa on sum P|V|sv / l, and kappa_l
     (including the largest eta, which moves l) on |O|.

Test infrastructure: reads the oracle's emulation through its observer hook
and adds no arithmetic to it.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

U_BF16 = 2.0 ** -8
U32 = 2.0 ** -23          # one fp32 rounding, allowing truncation
EPS_MFMA = 2.0 ** -13     # e4m3 MFMA dot product: |error| <= EPS_MFMA sum |a_k b_k|
LOG2E = 1.0 / math.log(2.0)
_MAGS = np.sort(oracle.e4m3_decode_table()[:127])  # non-negative e4m3 values, 0 .. 448


def e4m3_flip_step(p: np.ndarray, eta: np.ndarray) -> np.ndarray:
    """The spacing of the two e4m3 values around p where p lies within
    eta * p of their midpoint (an e4m3 rounding of p (1 +- eta) may return
    either), else 0.  p >= 0; values above 448 saturate and never flip."""
    p = np.asarray(p, np.float64)
    i = np.clip(np.searchsorted(_MAGS, p, side="left"), 1, len(_MAGS) - 1)
    lo, hi = _MAGS[i - 1], _MAGS[i]
    near = np.abs(p - 0.5 * (lo + hi)) <= eta * p
    return np.where(near & (p > 0) & (p <= 448.0), hi - lo, 0.0)


def emulation_with_bound(q8, k8, v8, sq, sk, sv, scale: float, causal: bool, rows=None):
    """(O, LSE, bound) of the oracle's FP8 emulation, O and bound shaped like
    O (BSHD, or [R, d] for ``rows``)."""
    qv, kv, vv = (oracle.e4m3_decode(x) for x in (q8, k8, v8))
    d = qv.shape[3]
    sq, sk, sv = (np.asarray(x, np.float64) for x in (sq, sk, sv))
    state = {}

    def observe(b, h, g, qi, keys, s, m_new, p, alpha):
        st = state.setdefault((b, h, int(qi[0]), len(qi)), {
            "qi": qi, "flip": 0.0, "abs": 0.0, "l": 0.0, "eta": np.zeros(len(qi)),
            "dalpha": np.zeros(len(qi)), "nk": 0, "nb": 0})
        vis = np.isfinite(s)
        # exponent of the kernel's exp2, in log2 units, and its absolute error
        cq = scale * LOG2E * sq[b, h, qi // oracle.fp8.QBLOCK]
        c = cq[:, None] * sk[b, g, keys // oracle.fp8.QBLOCK][None, :]
        qk_abs = np.abs(qv[b, qi, h, :]) @ np.abs(kv[b, keys, g, :]).T
        t = np.where(vis, s, 0.0) * LOG2E
        mm = (m_new * LOG2E)[:, None]
        dx = c * EPS_MFMA * qk_abs + (np.abs(t) + np.abs(mm)) * 4 * U32 + np.abs(t - mm) * U32
        eta = np.where(vis, math.log(2.0) * dx + 2 * U32, 0.0)
        step = e4m3_flip_step(p, eta)
        pq = oracle.e4m3_decode(oracle.e4m3_encode(p))
        vabs = np.abs(vv[b, keys, g, :]) * sv[b, g, keys // oracle.fp8.QBLOCK][:, None]
        a = alpha[:, None]
        st["flip"] = a * st["flip"] + step @ vabs
        st["abs"] = a * st["abs"] + pq @ vabs
        st["l"] = alpha * st["l"] + p.sum(axis=1)
        st["eta"] = np.maximum(st["eta"], eta.max(axis=1))
        # the tile's rescale of O: exp2(m - m') (its argument rounded from
        # two fp32 maxima, then exp2) and the V-scale ratio (reciprocal and
        # two products); exact 0 on the first block, exact 1 when m' = m
        live = (alpha > 0) & (alpha < 1)
        m_old = m_new + np.log(np.where(live, alpha, 1.0))
        st["dalpha"] += np.where(live, (np.abs(m_old) + np.abs(m_new)) * 2 * U32, 0.0) + 4 * U32
        st["nk"] += int(vis.any(axis=0).sum())
        st["nb"] += 1

    o, lse = oracle.fp8_attention_emulation(q8, k8, v8, sq, sk, sv, scale, causal, rows=rows,
                                            observer=observe)
    bound = np.zeros_like(o)
    if rows is not None:
        rows = np.asarray(rows, np.int64)
        where = {(int(b), int(h), int(i)): r for r, (b, h, i) in enumerate(rows)}
    for (b, h, _, _), st in state.items():
        kappa = EPS_MFMA + (st["nk"] + 4 * st["nb"] + 16) * U32 + st["dalpha"]
        kappa_l = st["eta"] + (st["nk"] + 4 * st["nb"] + 8) * U32 + st["dalpha"]
        l = st["l"][:, None]
        for j, i in enumerate(st["qi"]):
            if rows is None:
                oi = o[b, i, h]
            else:
                oi = o[where[(b, h, int(i))]]
            bd = (U_BF16 * (1 + kappa_l[j]) + kappa_l[j]) * np.abs(oi) + \
                (st["flip"][j] + kappa[j] * st["abs"][j]) / l[j]
            if rows is None:
                bound[b, i, h] = bd
            else:
                bound[where[(b, h, int(i))]] = bd
    bound += 1e-7 * float(np.abs(o).max())
    return o, lse, bound


def check_fp8(o_gpu, o_em, bound, tag: str, rms_gate: float = 0.45):
    """Every element inside its bound (x (1 + 1e-3)); RMS of err / bound below
    rms_gate (bf16 rounding alone gives about 0.4 against 2^-8 |O|, the other
    terms only widen the bound).  Returns (max ratio, RMS ratio)."""
    r = np.abs(np.asarray(o_gpu, np.float64) - o_em) / bound
    mx, rms = float(r.max()), float(np.sqrt(np.mean(r ** 2)))
    worst = np.unravel_index(int(np.argmax(r)), r.shape)
    print(f"{tag}: err/bound max={mx:.3f} (at {worst}) rms={rms:.3f}", flush=True)
    assert mx <= 1.0 + 1e-3, (mx, worst)
    assert rms <= rms_gate, rms
    return mx, rms
