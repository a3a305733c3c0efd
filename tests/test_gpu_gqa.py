"""Grouped-query / multi-query attention on the GPU ([FA3-report] section 3.4:
query head h reads K/V head h // (H // H_kv), K/V stored once).

bf16: the gates of the bf16 tests against the fp64 oracle with the GQA head
mapping, and bit-identity with the multi-head kernel run on K/V whose heads are
written out once per query head (the same arithmetic on the same values).
fp8: the tight gate against the FP8 emulation with the head mapping.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_bound import check_fp8, emulation_with_bound
from gpu_helpers import DEV, err_stats, lse_rows, rows_of, say, to_np

import exact_attention_74_amd as ea

pytestmark = pytest.mark.gpu

GATE_MAX, GATE_RMSE, GATE_LSE = 1e-2, 2e-3, 2e-5


def _host(B, N, H, Hkv, d, seed, dist="normal"):
    return [workloads.to_bf16_f32(x) for x in workloads.gen_qkv_gqa(B, N, H, Hkv, d, seed, dist)]


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(DEV)


def _bf16_gqa(q, k, v, causal, scale):
    o, lse = ea.attn_fwd_bf16_gqa(_dev(q), _dev(k), _dev(v), causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return to_np(o), lse.cpu().numpy().astype(np.float64)


def _replicate(x, H):
    Hkv = x.shape[2]
    return np.ascontiguousarray(np.repeat(x, H // Hkv, axis=2))


def _gate(o, lse, o_ref, lse_ref, tag):
    mx, rmse = err_stats(o, o_ref)
    lerr = float(np.abs(lse - lse_ref).max())
    print(f"{tag}: max_abs={mx:.3e} rmse={rmse:.3e} lse_max={lerr:.3e}", flush=True)
    assert mx <= GATE_MAX and rmse <= GATE_RMSE, (mx, rmse)
    assert lerr <= GATE_LSE, lerr


@pytest.mark.parametrize("N,d,H,Hkv,causal", [
    (200, 128, 6, 3, False), (200, 128, 6, 3, True),
    (1000, 64, 8, 1, False), (1000, 128, 4, 2, True),
    (1500, 128, 8, 2, False), (1500, 64, 4, 1, True), (500, 256, 4, 2, True),
    (700, 256, 4, 1, False)])
def test_bf16_gqa_full_parity(N, d, H, Hkv, causal):
    """Full oracle parity; N = 1500 takes the 8-wave workgroups, d = 256 the
    pipelined loop with O in the AGPRs (both masks), ragged tails."""
    tag = f"gqa_bf16_n{N}_d{d}_h{H}kv{Hkv}" + ("_causal" if causal else "")
    say(tag)
    q, k, v = _host(2, N, H, Hkv, d, seed=90 + N + H)
    scale = d ** -0.5
    o, lse = _bf16_gqa(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.naive_attention(q, k, v, scale, causal)
    _gate(o, lse, o_ref, lse_ref, tag)


@pytest.mark.parametrize("H,Hkv,causal", [(8, 2, False), (8, 1, True), (4, 4, False)])
def test_bf16_gqa_bitwise_equals_replicated_mha(H, Hkv, causal):
    N, d = 700, 128
    say(f"gqa_bf16_bitwise_h{H}kv{Hkv}")
    q, k, v = _host(1, N, H, Hkv, d, seed=120 + H + Hkv)
    o, lse = _bf16_gqa(q, k, v, causal, 0.1)
    o2, lse2 = ea.attn_fwd_bf16(_dev(q), _dev(_replicate(k, H)), _dev(_replicate(v, H)),
                                causal=causal, softmax_scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(torch.from_numpy(o), torch.from_numpy(to_np(o2)))
    assert np.array_equal(lse, lse2.cpu().numpy().astype(np.float64))


def test_bf16_gqa_full_size_sampled_rows():
    """A grouped-query shape at full size: B2 H32 H_kv8 N4096 d128, causal and
    not; 256 sampled rows each against the oracle."""
    B, N, H, Hkv, d = 2, 4096, 32, 8, 128
    q, k, v = _host(B, N, H, Hkv, d, seed=7)
    for causal in (False, True):
        tag = f"gqa_bf16_b{B}h{H}kv{Hkv}n{N}d{d}" + ("_causal" if causal else "")
        say(tag)
        o, lse = _bf16_gqa(q, k, v, causal, d ** -0.5)
        rows = workloads.sample_rows(B, H, N, 256, seed=8 + causal)
        o_ref, l_ref = oracle.naive_attention_rows(q, k, v, d ** -0.5, causal, rows)
        _gate(rows_of(o, rows), lse_rows(lse, rows), o_ref, l_ref, tag)


def test_bf16_gqa_rejects_bad_head_counts():
    q = torch.zeros((1, 64, 6, 64), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 64, 4, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        ea.attn_fwd_bf16_gqa(q, kv, kv)
    with pytest.raises(ValueError):
        ea.attn_fwd_bf16(q, kv, kv)


def _rmse(a, b):
    return float(np.sqrt(np.mean((np.asarray(a, np.float64) - b) ** 2)))


@pytest.mark.parametrize("N,d,H,Hkv,causal", [(300, 128, 6, 2, False), (1000, 64, 4, 1, True),
                                               (1000, 128, 8, 2, True), (600, 256, 4, 2, True),
                                               (700, 256, 4, 2, False)])
def test_fp8_gqa_vs_emulation(N, d, H, Hkv, causal):
    tag = f"gqa_fp8_n{N}_d{d}_h{H}kv{Hkv}" + ("_causal" if causal else "")
    say(tag)
    q, k, v = _host(2, N, H, Hkv, d, seed=150 + N + H, dist="outlier_sd10")
    signs = workloads.gen_signs(d)
    q8, sq = oracle.blockquant_hadamard(q, signs, 128)
    k8, sk = oracle.blockquant_hadamard(k, signs, 128)
    v8, sv = oracle.blockquant_hadamard(v, None, 128)
    scale = d ** -0.5
    t = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (q8, k8, v8, sq, sk, sv)]
    o, lse = ea.attn_fwd_fp8_gqa(*t, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    o, lse = to_np(o), lse.cpu().numpy().astype(np.float64)
    o_em, l_em, bound = emulation_with_bound(q8, k8, v8, sq, sk, sv, scale, causal)
    o_ex, _ = oracle.naive_attention(q, k, v, scale, causal)
    check_fp8(o, o_em, bound, tag)
    e_kernel, e_scheme = _rmse(o, o_em), _rmse(o_em, o_ex)
    lerr = float(np.abs(lse - l_em).max())
    print(f"{tag}: rmse(gpu-emul)={e_kernel:.3e} rmse(emul-exact)={e_scheme:.3e} "
          f"lse(gpu-emul)={lerr:.3e}", flush=True)
    assert e_kernel <= 0.1 * e_scheme
    assert lerr <= 1e-3
    assert np.isfinite(o).all()
