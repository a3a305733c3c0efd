"""Pins for the fp64 attention oracle (CPU only).

Every check compares the oracle with something other than itself: closed forms,
special cases, or an independent library routine (torch's CPU
scaled_dot_product_attention and logsumexp in float64).
"""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import naive_attention, naive_attention_rows, tiled_attention


def _rand(shape, seed):
    return workloads.gen_random(shape, seed).astype(np.float64)


def _sdpa(q, k, v, scale, causal):
    """torch CPU fp64 SDPA on BSHD numpy arrays -> (O BSHD, LSE [B,H,N])."""
    qt = torch.from_numpy(np.transpose(q, (0, 2, 1, 3)).copy())
    kt = torch.from_numpy(np.transpose(k, (0, 2, 1, 3)).copy())
    vt = torch.from_numpy(np.transpose(v, (0, 2, 1, 3)).copy())
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    s = scale * (qt @ kt.transpose(-1, -2))
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return np.transpose(o.numpy(), (0, 2, 1, 3)), lse.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_naive_matches_torch_sdpa_tiny(causal):
    w = workloads.TINY
    q, k, v = (x.astype(np.float64) for x in workloads.gen_qkv(w))
    o, lse = naive_attention(q, k, v, w.softmax_scale, causal)
    o_ref, lse_ref = _sdpa(q, k, v, w.softmax_scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,Br,Bc", [(256, 64, 64), (200, 64, 64), (131, 32, 48)])
def test_tiled_equals_naive(causal, N, Br, Bc):
    q, k, v = (_rand((2, N, 3, 64), s) for s in (1, 2, 3))
    o1, l1 = naive_attention(q, k, v, 0.125, causal, row_chunk=37)
    o2, l2 = tiled_attention(q, k, v, 0.125, causal, Br=Br, Bc=Bc)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-13)


def test_rows_variant_equals_full():
    q, k, v = (_rand((2, 150, 2, 32), s) for s in (4, 5, 6))
    rows = workloads.sample_rows(2, 2, 150, 40, seed=7)
    for causal in (False, True):
        o, lse = naive_attention(q, k, v, 0.3, causal)
        oo, ll = naive_attention_rows(q, k, v, 0.3, causal, rows)
        b, h, i = rows.T
        np.testing.assert_allclose(oo, o[b, i, h], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(ll, lse[b, h, i], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("fn", [naive_attention, tiled_attention])
@pytest.mark.parametrize("causal", [False, True])
def test_identical_value_rows_give_that_row(fn, causal):
    q, k = _rand((1, 130, 2, 64), 8), _rand((1, 130, 2, 64), 9)
    row = _rand((64,), 10)
    v = np.broadcast_to(row, (1, 130, 2, 64)).copy()
    o, _ = fn(q, k, v, 1 / 8, causal)
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("fn", [naive_attention, tiled_attention])
def test_causal_row0_is_v0_exactly(fn):
    q, k, v = (_rand((2, 70, 3, 32), s) for s in (11, 12, 13))
    o, lse = fn(q, k, v, 0.2, True)
    assert np.array_equal(o[:, 0], v[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.2 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]),
                               rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("fn", [naive_attention, tiled_attention])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_is_uniform_attention(fn, causal):
    N = 97
    q = np.zeros((1, N, 2, 16))
    k, v = _rand((1, N, 2, 16), 14), _rand((1, N, 2, 16), 15)
    o, lse = fn(q, k, v, 0.25, causal)
    if causal:
        expect = np.cumsum(v, axis=1) / np.arange(1, N + 1)[None, :, None, None]
        lse_expect = np.log(np.arange(1, N + 1))[None, None, :].repeat(2, axis=1)
    else:
        expect = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
        lse_expect = np.full((1, 2, N), math.log(N))
    np.testing.assert_allclose(o, expect, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_expect, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("fn", [naive_attention, tiled_attention])
def test_single_spike_closed_form(fn):
    """q_i = t_i e0, k_0 = e0, other keys orthogonal to e0: only key 0 scores.

    O_i = (e^{c t_i} v_0 + sum_{j>0} v_j) / (e^{c t_i} + N - 1),
    LSE_i = ln(e^{c t_i} + N - 1).  A dropped or misplaced scale fails this.
    """
    N, d, c = 40, 8, 0.37
    t = np.linspace(-3, 5, N)
    q = np.zeros((1, N, 1, d))
    q[0, :, 0, 0] = t
    k = np.zeros((1, N, 1, d))
    k[0, 0, 0, 0] = 1.0
    k[0, 1:, 0, 1:] = _rand((N - 1, d - 1), 16)
    v = _rand((1, N, 1, d), 17)
    o, lse = fn(q, k, v, c, False)
    w0 = np.exp(c * t)
    expect = (w0[:, None] * v[0, 0, 0][None, :] + v[0, 1:, 0].sum(axis=0)[None, :]) / (w0 + N - 1)[:, None]
    np.testing.assert_allclose(o[0, :, 0], expect, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], np.log(w0 + N - 1), rtol=1e-14)


def test_two_keys_logistic_closed_form():
    """Two keys: the weight of key 0 is the logistic function of the score gap."""
    q, k, v = (_rand((1, 2, 1, 4), s) for s in (18, 19, 20))
    o, _ = naive_attention(q, k, v, 0.5, False)
    for i in range(2):
        gap = 0.5 * (q[0, i, 0] @ (k[0, 0, 0] - k[0, 1, 0]))
        w = 1.0 / (1.0 + math.exp(-gap))
        np.testing.assert_allclose(o[0, i, 0], w * v[0, 0, 0] + (1 - w) * v[0, 1, 0], rtol=1e-14)


def test_causal_prefix_independence():
    """Rows i < r do not change when keys/values of rows > r change."""
    q, k, v = (_rand((1, 64, 2, 16), s) for s in (21, 22, 23))
    o1, l1 = naive_attention(q, k, v, 0.3, True)
    k2, v2 = k.copy(), v.copy()
    k2[:, 40:] += 5.0
    v2[:, 40:] -= 3.0
    o2, l2 = tiled_attention(q, k2, v2, 0.3, True, Br=16, Bc=16)
    assert np.allclose(o2[:, :40], o1[:, :40], rtol=1e-13, atol=1e-14)
    assert np.allclose(l2[:, :, :40], l1[:, :, :40], rtol=1e-13, atol=1e-14)
    assert not np.allclose(o2[:, 40:], o1[:, 40:])


# --- grouped-query / multi-query attention ([FA3-report] section 3.4) -------

def _sdpa_gqa(q, k, v, scale, causal):
    """torch CPU fp64 SDPA with its own grouped-query head mapping (enable_gqa)."""
    qt = torch.from_numpy(np.transpose(q, (0, 2, 1, 3)).copy())
    kt = torch.from_numpy(np.transpose(k, (0, 2, 1, 3)).copy())
    vt = torch.from_numpy(np.transpose(v, (0, 2, 1, 3)).copy())
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale,
                                                         enable_gqa=True)
    return np.transpose(o.numpy(), (0, 2, 1, 3))


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 3), (4, 1), (3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_torch_sdpa(H, Hkv, causal):
    q = _rand((2, 70, H, 16), 40)
    k = _rand((2, 70, Hkv, 16), 41)
    v = _rand((2, 70, Hkv, 16), 42)
    o, _ = naive_attention(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, _sdpa_gqa(q, k, v, 0.3, causal), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("H,Hkv", [(4, 2), (4, 1)])
def test_gqa_is_mha_on_replicated_heads(H, Hkv):
    """Each group of H // Hkv query heads sees the same K/V head: the result is
    multi-head attention on K/V with every head written out H // Hkv times."""
    q = _rand((1, 90, H, 32), 43)
    k = _rand((1, 90, Hkv, 32), 44)
    v = _rand((1, 90, Hkv, 32), 45)
    kr = np.concatenate([k[:, :, [g], :] for g in range(Hkv) for _ in range(H // Hkv)], axis=2)
    vr = np.concatenate([v[:, :, [g], :] for g in range(Hkv) for _ in range(H // Hkv)], axis=2)
    for causal in (False, True):
        o, lse = naive_attention(q, k, v, 0.2, causal)
        o_r, lse_r = naive_attention(q, kr, vr, 0.2, causal)
        np.testing.assert_array_equal(o, o_r)
        np.testing.assert_array_equal(lse, lse_r)
        ot, lset = tiled_attention(q, k, v, 0.2, causal, Br=32, Bc=48)
        np.testing.assert_allclose(ot, o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lset, lse, rtol=1e-12, atol=1e-13)


def test_mqa_heads_share_one_kv():
    """H_kv = 1: query head h alone against the single K/V head gives head h."""
    q = _rand((1, 50, 3, 16), 46)
    k = _rand((1, 50, 1, 16), 47)
    v = _rand((1, 50, 1, 16), 48)
    o, lse = naive_attention(q, k, v, 0.25, True)
    for h in range(3):
        oh, lh = naive_attention(q[:, :, [h], :], k, v, 0.25, True)
        np.testing.assert_array_equal(o[:, :, [h], :], oh)
        np.testing.assert_array_equal(lse[:, [h], :], lh)


def test_gqa_rows_variant_equals_full():
    q = _rand((2, 64, 6, 16), 49)
    k = _rand((2, 64, 2, 16), 50)
    v = _rand((2, 64, 2, 16), 51)
    o, lse = naive_attention(q, k, v, 0.5, True)
    rows = np.array([[0, 0, 0], [1, 5, 63], [0, 3, 17], [1, 2, 40]])
    oo, ll = naive_attention_rows(q, k, v, 0.5, True, rows)
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(oo[r], o[b, i, h], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(ll[r], lse[b, h, i], rtol=1e-13, atol=1e-14)


def test_kv_head_rejects_bad_counts():
    from oracle import kv_head
    assert [kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    for H, Hkv in ((4, 3), (2, 4), (4, 0)):
        with pytest.raises(ValueError):
            kv_head(0, H, Hkv)
