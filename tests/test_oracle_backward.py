"""Pins for the fp64 attention-gradient oracle (CPU only).

Each check compares ``oracle.attention_backward`` with something other than its
own formula: torch's fp64 autograd through softmax attention, central finite
differences of the forward oracle (itself pinned in test_oracle_attention.py),
invariants that follow from the softmax (shift invariance in K, rows of P
summing to one) and a one-token closed form.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import attention_backward, attention_backward_heads, naive_attention


def _rand(shape, seed):
    return workloads.gen_random(shape, seed).astype(np.float64)


def _torch_grads(q, k, v, do, scale, causal):
    t = [torch.from_numpy(np.transpose(x, (0, 2, 1, 3)).copy()).requires_grad_(True)
         for x in (q, k, v)]
    s = scale * (t[0] @ t[1].transpose(-1, -2))
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ t[2]
    o.backward(torch.from_numpy(np.transpose(do, (0, 2, 1, 3)).copy()))
    return [np.transpose(x.grad.numpy(), (0, 2, 1, 3)) for x in t]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 8), (37, 16), (130, 32)])
def test_matches_torch_autograd(causal, N, d):
    q, k, v, do = (_rand((2, N, 3, d), s) for s in (1, 2, 3, 4))
    got = attention_backward(q, k, v, do, 0.3, causal)
    ref = _torch_grads(q, k, v, do, 0.3, causal)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_central_finite_differences(causal):
    """dL/dx for L = sum(dO * O(q, k, v)), O from the forward oracle."""
    N, d, scale = 5, 3, 0.7
    q, k, v, do = (_rand((1, N, 1, d), s) for s in (5, 6, 7, 8))
    grads = attention_backward(q, k, v, do, scale, causal)
    eps = 1e-6
    for which, g in enumerate(grads):
        for idx in np.ndindex(q.shape):
            xs = [q.copy(), k.copy(), v.copy()]
            xs[which][idx] += eps
            lp = np.sum(do * naive_attention(*xs, scale, causal)[0])
            xs[which][idx] -= 2 * eps
            lm = np.sum(do * naive_attention(*xs, scale, causal)[0])
            assert abs((lp - lm) / (2 * eps) - g[idx]) <= 1e-7, (which, idx)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_invariants(causal):
    """Adding one vector to every key leaves each row's softmax unchanged, so
    the key gradients sum to zero; the rows of P sum to one, so the value
    gradients sum to the sum of the output gradients."""
    q, k, v, do = (_rand((2, 90, 2, 16), s) for s in (9, 10, 11, 12))
    dq, dk, dv = attention_backward(q, k, v, do, 0.25, causal)
    scale_k = np.abs(dk).max()
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12 * scale_k * 90)
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), rtol=1e-12, atol=1e-11)


def test_single_token_closed_form():
    """N = 1: P = 1, so dS = 0 (dQ = dK = 0) and dV = dO."""
    q, k, v, do = (_rand((3, 1, 2, 8), s) for s in (13, 14, 15, 16))
    for causal in (False, True):
        dq, dk, dv = attention_backward(q, k, v, do, 0.5, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-15)
        np.testing.assert_allclose(dk, 0.0, atol=1e-15)
        np.testing.assert_array_equal(dv, do)


def test_heads_variant_equals_full():
    q, k, v, do = (_rand((2, 40, 3, 8), s) for s in (17, 18, 19, 20))
    full = attention_backward(q, k, v, do, 0.4, True)
    heads = np.array([[0, 2], [1, 0]])
    part = attention_backward_heads(q, k, v, do, 0.4, True, heads)
    for f, p_ in zip(full, part):
        for r, (b, h) in enumerate(heads):
            np.testing.assert_array_equal(p_[r], f[b, :, h, :])


def _torch_grads_gqa(q, k, v, do, scale, causal):
    t = [torch.from_numpy(np.transpose(x, (0, 2, 1, 3)).copy()).requires_grad_(True)
         for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(t[0], t[1], t[2], is_causal=causal,
                                                         scale=scale, enable_gqa=True)
    o.backward(torch.from_numpy(np.transpose(do, (0, 2, 1, 3)).copy()))
    return [np.transpose(x.grad.numpy(), (0, 2, 1, 3)) for x in t]


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_torch_autograd(H, Hkv, causal):
    """K/V gradients of a grouped-query head are the sums over its group
    (torch's enable_gqa attention differentiated by autograd)."""
    q, do = _rand((2, 45, H, 16), 21), _rand((2, 45, H, 16), 22)
    k, v = _rand((2, 45, Hkv, 16), 23), _rand((2, 45, Hkv, 16), 24)
    got = attention_backward(q, k, v, do, 0.3, causal)
    ref = _torch_grads_gqa(q, k, v, do, 0.3, causal)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (8, 4)])
def test_heads_variant_grouped_query(H, Hkv):
    """For grouped-query inputs the per-head helper returns dQ of the query
    head and dK, dV of the K/V head it reads (the group sums), equal to the
    full oracle's; torch autograd pins the full oracle for these shapes."""
    q, do = _rand((2, 33, H, 8), 25), _rand((2, 33, H, 8), 26)
    k, v = _rand((2, 33, Hkv, 8), 27), _rand((2, 33, Hkv, 8), 28)
    full = attention_backward(q, k, v, do, 0.45, True)
    heads = np.array([[0, H - 1], [1, 0], [1, H // 2]])
    part = attention_backward_heads(q, k, v, do, 0.45, True, heads)
    r = H // Hkv
    for i, (b, h) in enumerate(heads):
        np.testing.assert_allclose(part[0][i], full[0][b, :, h, :], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(part[1][i], full[1][b, :, h // r, :], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(part[2][i], full[2][b, :, h // r, :], rtol=1e-13, atol=1e-14)
    ref = _torch_grads_gqa(q, k, v, do, 0.45, True)
    np.testing.assert_allclose(part[1][0], ref[1][0, :, (H - 1) // r, :], rtol=1e-10, atol=1e-12)
