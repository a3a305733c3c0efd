"""Parity over a seeded spread of odd shapes (GPU).

The other GPU tests pick their shapes by the code path each one exercises;
this file draws a fixed list from a seeded generator instead: sequence
lengths on and around every tile size the kernels use (32-row waves, 64-key
bf16 tiles, 128-key FP8 tiles and quantisation blocks, 256-row workgroups),
batch 1-3, 1-3 K/V heads with 1, 2 or 4 query heads each, both masks and every
head dim.  Each case goes through the public entry points against the oracle
with the bars of the dedicated tests:
  * attn_fwd_bf16_gqa: the exact attention of oracle.naive_attention;
  * attn_fwd_fp8_gqa: the oracle's FP8 emulation, per element within the
    bound of tests/fp8_bound.py;
  * attn_bwd_bf16 (head dims 64 and 128): oracle.attention_backward, per
    element within the bf16 bound of tests/test_gpu_bwd.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_bound import check_fp8, emulation_with_bound
from gpu_helpers import DEV, say, to_np
from test_gpu_bwd import _bounds, _check, _gpu
from test_gpu_gqa import _gate

import exact_attention_74_amd as ea

pytestmark = pytest.mark.gpu

_NS = [1, 2, 31, 33, 63, 65, 127, 129, 191, 255, 257, 383, 385, 511, 513, 767, 1023, 1025, 1279]


def _draw(n, dims, seed, gqa=True):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        N = int(rng.choice(_NS))
        d = int(rng.choice(dims))
        hkv = int(rng.integers(1, 4))
        H = hkv * int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 4))
        causal = bool(rng.integers(0, 2))
        out.append((B, N, H, hkv if gqa else H, d, causal))
    return out


def _ids(shapes):
    return [f"b{B}n{N}h{H}kv{K}d{d}" + ("c" if c else "") for B, N, H, K, d, c in shapes]


FWD = _draw(14, [64, 128, 256], 2026)
FP8 = _draw(10, [64, 128, 256], 2027)
BWD = _draw(8, [64, 128], 2028, gqa=False)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("B,N,H,Hkv,d,causal", FWD, ids=_ids(FWD))
def test_bf16_forward_seeded_shapes(B, N, H, Hkv, d, causal):
    tag = "seeded_bf16_" + _ids([(B, N, H, Hkv, d, causal)])[0]
    say(tag)
    q, k, v = (workloads.to_bf16_f32(x) for x in workloads.gen_qkv_gqa(B, N, H, Hkv, d, 700 + N + d))
    scale = d ** -0.5
    o, lse = ea.attn_fwd_bf16_gqa(_dev(q), _dev(k), _dev(v), causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.naive_attention(q, k, v, scale, causal)
    _gate(to_np(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, tag)


@pytest.mark.parametrize("B,N,H,Hkv,d,causal", FP8, ids=_ids(FP8))
def test_fp8_forward_seeded_shapes(B, N, H, Hkv, d, causal):
    tag = "seeded_fp8_" + _ids([(B, N, H, Hkv, d, causal)])[0]
    say(tag)
    q, k, v = (workloads.to_bf16_f32(x)
               for x in workloads.gen_qkv_gqa(B, N, H, Hkv, d, 800 + N + d, "outlier_sd10"))
    signs = workloads.gen_signs(d)
    q8, sq = oracle.blockquant_hadamard(q, signs, 128)
    k8, sk = oracle.blockquant_hadamard(k, signs, 128)
    v8, sv = oracle.blockquant_hadamard(v, None, 128)
    scale = d ** -0.5
    t = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (q8, k8, v8, sq, sk, sv)]
    o, lse = ea.attn_fwd_fp8_gqa(*t, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    o_em, l_em, bound = emulation_with_bound(q8, k8, v8, sq, sk, sv, scale, causal)
    o = to_np(o)
    check_fp8(o, o_em, bound, tag)
    assert np.isfinite(o).all()
    assert float(np.abs(lse.cpu().numpy().astype(np.float64) - l_em).max()) <= 1e-3


@pytest.mark.parametrize("B,N,H,Hkv,d,causal", BWD, ids=_ids(BWD))
def test_bf16_backward_seeded_shapes(B, N, H, Hkv, d, causal):
    tag = "seeded_bwd_" + _ids([(B, N, H, Hkv, d, causal)])[0]
    say(tag)
    w = workloads.Workload("bwds", B, H, N, d, False, seed=900 + N + d)
    q, k, v = (workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w))
    do = workloads.to_bf16_f32(workloads.gen_random((B, N, H, d), 950 + N))
    scale = d ** -0.5
    dq, dk, dv, o = _gpu(q, k, v, do, causal, scale)
    ref = oracle.attention_backward(q, k, v, do, scale, causal)
    _check((dq, dk, dv), ref, _bounds(q, k, v, do, o, scale, causal), tag)
