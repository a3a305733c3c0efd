"""Gradients of exact attention, fp64: the definition (test infrastructure).

Test infrastructure only (see the package docstring).

The backward pass of [FA3-report] section 3.4 keeps FA-2's strategy: it
recomputes the score block from Q, K and the saved log-sum-exp instead of
storing P, and does five matrix products per block (2.5 times the forward's
two); [FA3-blog] section 5.4 is the reminder that the softmax statistics must
be kept (or recomputed) for it.  What is computed is the plain derivative of
the forward definition.  For one (b, h), with O = P V and the loss gradient
dO:

    P    = softmax(scale Q K^T [causal])        (exactly, from LSE)
    D_i  = sum_c dO[i, c] O[i, c]
    dV   = P^T dO
    dP   = dO V^T
    dS   = P * (dP - D)                          (elementwise; D per row)
    dQ   = scale dS K
    dK   = scale dS^T Q

(dS is the gradient with respect to the scores S = scale Q K^T that enter
the softmax; its rows sum to zero because the rows of P sum to one.)

With K and V on H_kv heads (grouped-query attention, [FA3-report] section
3.4), query head h reads K/V head h // (H // H_kv), so the gradient of a K/V
head is the sum of the per-query-head gradients of its group.
"""
from __future__ import annotations

import numpy as np

from .attention import _heads, kv_head


def _probs(qh, kh, scale, causal):
    s = scale * (qh @ kh.T)
    if causal:
        n, m = s.shape
        s[np.arange(m)[None, :] > np.arange(n)[:, None]] = -np.inf
    mx = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - mx)
    return e / np.sum(e, axis=1, keepdims=True)


def attention_backward(q, k, v, do, scale: float, causal: bool):
    """(dQ, dK, dV) as fp64 BSHD arrays for inputs q, k, v and output gradient
    do (BSHD; k, v may have H_kv heads, H a multiple of H_kv)."""
    qh, kh, vh, doh = _heads(q), _heads(k), _heads(v), _heads(do)
    B, H, N, d = qh.shape
    Hkv = kh.shape[1]
    dq = np.empty_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            p = _probs(qh[b, h], kh[b, g], scale, causal)
            o = p @ vh[b, g]
            dd = np.sum(doh[b, h] * o, axis=1)
            dv[b, g] += p.T @ doh[b, h]
            dp = doh[b, h] @ vh[b, g].T
            ds = p * (dp - dd[:, None])
            dq[b, h] = scale * (ds @ kh[b, g])
            dk[b, g] += scale * (ds.T @ qh[b, h])
    back = lambda x: np.transpose(x, (0, 2, 1, 3))  # noqa: E731
    return back(dq), back(dk), back(dv)


def attention_backward_heads(q, k, v, do, scale: float, causal: bool, heads):
    """The same for selected query heads only: ``heads`` is an int array
    [R, 2] of (b, h) pairs.  Returns fp64 arrays [R, N, d]: dQ of query head
    (b, h), and dK, dV of the K/V head (b, g) it reads, g = h // (H // H_kv),
    which are the sums over all query heads of that group (large workloads are
    checked on a few whole heads: every key's gradient needs every query)."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    heads = np.asarray(heads, np.int64)
    R, N, d = heads.shape[0], q.shape[1], q.shape[3]
    H, Hkv = q.shape[2], k.shape[2]
    r = H // Hkv
    out = [np.empty((R, N, d)) for _ in range(3)]
    for i, (b, h) in enumerate(heads):
        g = kv_head(int(h), H, Hkv)
        # the group's query heads with their one K/V head (grouped-query, H_kv = 1)
        qs = np.asarray(q[b:b + 1, :, g * r:(g + 1) * r, :], np.float64)
        dos = np.asarray(do[b:b + 1, :, g * r:(g + 1) * r, :], np.float64)
        ks = np.asarray(k[b:b + 1, :, g:g + 1, :], np.float64)
        vs = np.asarray(v[b:b + 1, :, g:g + 1, :], np.float64)
        dq, dk, dv = attention_backward(qs, ks, vs, dos, scale, causal)
        out[0][i] = dq[0, :, h - g * r, :]
        out[1][i] = dk[0, :, 0, :]
        out[2][i] = dv[0, :, 0, :]
    return tuple(out)
