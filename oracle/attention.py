"""Exact softmax attention in fp64: the definition, and the tiled recurrence.

Test infrastructure only (see the package docstring).  Nothing here is shared
with, or imported by, the HIP library.

Definition ([FA3-report] section 3, "FlashAttention computes the same
mathematics, only the execution changes"): for every batch b and head h, with
Q, K, V the (N x d) slices of the BSHD tensors,

    S   = scale * Q K^T              (causal: S[i, j] = -inf for j > i)
    m_i = max_j S[i, j]
    P   = exp(S - m) / sum_j exp(S - m)
    O   = P V
    LSE_i = m_i + ln sum_j exp(S[i, j] - m_i)

The log-sum-exp is the softmax statistic kept for the backward pass ([FA3-blog]
section 5.4).

Grouped-query and multi-query attention ([FA3-report] section 3.4, which keeps
FA-2's index mapping for MQA/GQA): K and V may have H_kv heads with H a
multiple of H_kv; query head h then uses K/V head h // (H // H_kv) in the
definition above.  H_kv = H is ordinary multi-head attention.  A key j is visible to query i iff j <= i (queries and keys have
the same length in every workload here, so top-left and bottom-right causal
alignment coincide).
"""
from __future__ import annotations

import numpy as np


def _heads(x: np.ndarray) -> np.ndarray:
    """BSHD -> (B, H, N, d) float64 view/copy."""
    x = np.asarray(x)
    if x.ndim != 4:
        raise ValueError("expected a BSHD array")
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3)), dtype=np.float64)


def kv_head(h: int, H: int, H_kv: int) -> int:
    """The K/V head that query head h reads when K/V have H_kv heads."""
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"H = {H} must be a positive multiple of H_kv = {H_kv}")
    return h // (H // H_kv)


def _rows_softmax_av(s: np.ndarray, vh: np.ndarray):
    """Row softmax of the score block ``s`` (rows x N) times V; returns (O, LSE)."""
    m = np.max(s, axis=1)
    e = np.exp(s - m[:, None])
    l = np.sum(e, axis=1)
    o = (e @ vh) / l[:, None]
    return o, m + np.log(l)


def naive_attention(q, k, v, scale: float, causal: bool, row_chunk: int = 512):
    """Full-row softmax attention, fp64.  Returns (O [B,N,H,d], LSE [B,H,N]).

    Rows are independent, so queries are processed ``row_chunk`` at a time to
    bound the score matrix held in memory; every row still sees its full set
    of keys at once (no online rescaling).
    """
    qh, kh, vh = _heads(q), _heads(k), _heads(v)
    B, H, N, d = qh.shape
    Nk, Hkv = kh.shape[2], kh.shape[1]
    o = np.empty((B, H, N, vh.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    cols = np.arange(Nk)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            for r0 in range(0, N, row_chunk):
                r1 = min(N, r0 + row_chunk)
                s = scale * (qh[b, h, r0:r1] @ kh[b, g].T)
                if causal:
                    rows = np.arange(r0, r1)
                    s[cols[None, :] > rows[:, None]] = -np.inf
                o[b, h, r0:r1], lse[b, h, r0:r1] = _rows_softmax_av(s, vh[b, g])
    return np.transpose(o, (0, 2, 1, 3)), lse


def naive_attention_rows(q, k, v, scale: float, causal: bool, rows):
    """The definition evaluated for selected query rows only.

    ``rows`` is an int array [R, 3] of (b, h, i).  Returns (O_rows [R, d],
    LSE_rows [R]).  Each row costs O(N d), so large workloads can be checked
    on a sample of rows.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    rows = np.asarray(rows, dtype=np.int64)
    out_o = np.empty((rows.shape[0], v.shape[3]), dtype=np.float64)
    out_l = np.empty(rows.shape[0], dtype=np.float64)
    # group by (b, h) so each K/V head slice is converted once
    keys = rows[:, 0] * q.shape[2] + rows[:, 1]
    for key in np.unique(keys):
        sel = np.nonzero(keys == key)[0]
        b, h = int(rows[sel[0], 0]), int(rows[sel[0], 1])
        g = kv_head(h, q.shape[2], k.shape[2])
        kh = np.asarray(k[b, :, g, :], dtype=np.float64)
        vh = np.asarray(v[b, :, g, :], dtype=np.float64)
        qi = np.asarray(q[b, rows[sel, 2], h, :], dtype=np.float64)
        s = scale * (qi @ kh.T)
        if causal:
            s[np.arange(kh.shape[0])[None, :] > rows[sel, 2][:, None]] = -np.inf
        out_o[sel], out_l[sel] = _rows_softmax_av(s, vh)
    return out_o, out_l


def tiled_attention(q, k, v, scale: float, causal: bool, Br: int = 64, Bc: int = 64):
    """The tiled online-softmax recurrence in fp64 ([FA3-report] section 3;
    [FA-explain], FA2's single final normalisation per query block).

    For each query block the keys are visited Bc at a time; the running row
    max m and row sum l are updated as

        m'  = max(m, rowmax S_j)
        P_j = exp(S_j - m')
        l   = exp(m - m') * l + rowsum P_j
        O   = exp(m - m') * O + P_j V_j

    and O / l, m + ln l are produced once at the end.  Causal key blocks that
    lie entirely above the diagonal are skipped.  Returns (O, LSE) like
    ``naive_attention``.
    """
    qh, kh, vh = _heads(q), _heads(k), _heads(v)
    B, H, N, d = qh.shape
    Nk, Hkv = kh.shape[2], kh.shape[1]
    o = np.empty((B, H, N, vh.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            for r0 in range(0, N, Br):
                r1 = min(N, r0 + Br)
                qi = qh[b, h, r0:r1]
                rows = np.arange(r0, r1)
                m = np.full(r1 - r0, -np.inf)
                l = np.zeros(r1 - r0)
                acc = np.zeros((r1 - r0, vh.shape[3]))
                for c0 in range(0, Nk, Bc):
                    if causal and c0 > r1 - 1:
                        break
                    c1 = min(Nk, c0 + Bc)
                    s = scale * (qi @ kh[b, g, c0:c1].T)
                    if causal:
                        s[np.arange(c0, c1)[None, :] > rows[:, None]] = -np.inf
                    m_new = np.maximum(m, np.max(s, axis=1))
                    p = np.exp(s - m_new[:, None])
                    alpha = np.exp(m - m_new)
                    l = alpha * l + np.sum(p, axis=1)
                    acc = alpha[:, None] * acc + p @ vh[b, g, c0:c1]
                    m = m_new
                o[b, h, r0:r1] = acc / l[:, None]
                lse[b, h, r0:r1] = m + np.log(l)
    return np.transpose(o, (0, 2, 1, 3)), lse
