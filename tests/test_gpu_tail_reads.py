"""Rows past the end of the sequence must read as zeros in every kernel.

The kernels copy whole 64- or 128-row K/V (and, for the gradients, Q/dO and
LSE/D) tiles into LDS, so the last tile of a ragged sequence reaches past row
N - 1.  Those rows must come back as zeros from the buffer range check, not
from whatever memory follows: a masked key has P = 0, but 0 x NaN is NaN in
the P.V product, so a NaN (or, in e4m3, a 0x7F code) behind the tensor would
leak into real output rows.

Here every input is the leading part of a larger allocation whose remainder
is NaN (0x7F for e4m3 codes), with ragged N and B >= 2, so the rows after the
last batch entry's row N - 1 hold NaN.  The fill stays inside the allocation:
no access leaves it.  Outputs must be finite and agree with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_bound import check_fp8, emulation_with_bound
from gpu_helpers import DEV, err_stats, say, to_np

import exact_attention_74_amd as ea

pytestmark = pytest.mark.gpu

PAD_ROWS = 256  # rows of NaN behind each tensor (more than a tile of 128)


def _padded(x: np.ndarray, dtype, fill) -> torch.Tensor:
    """x (BSHD) on the device as the leading part of a larger buffer whose
    remaining PAD_ROWS * H * d elements hold ``fill``."""
    B, N, H, d = x.shape
    n = x.size
    buf = torch.full((n + PAD_ROWS * H * d,), fill, dtype=dtype, device=DEV)
    src = torch.from_numpy(np.ascontiguousarray(x))
    buf[:n] = (src.to(dtype) if dtype != torch.uint8 else src).reshape(-1).to(DEV)
    return buf[:n].view(B, N, H, d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [129, 1000])
def test_bf16_forward_nan_behind_inputs(N, d, causal):
    w = workloads.Workload(f"tail_bf16_n{N}_d{d}", 2, 3, N, d, causal, seed=900 + N + d)
    say(w.name + ("_causal" if causal else ""))
    q, k, v = (workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w))
    tq, tk, tv = (_padded(x, torch.bfloat16, float("nan")) for x in (q, k, v))
    o, lse = ea.attn_fwd_bf16(tq, tk, tv, causal=causal, softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    o, lse = to_np(o), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    o_ref, l_ref = oracle.naive_attention(q, k, v, w.softmax_scale, causal)
    mx, rmse = err_stats(o, o_ref)
    assert mx <= 1e-2 and rmse <= 2e-3, (mx, rmse)
    assert np.abs(lse - l_ref).max() <= 2e-5


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [129, 1000])
def test_fp8_forward_nan_codes_behind_inputs(N, d, causal):
    w = workloads.Workload(f"tail_fp8_n{N}_d{d}", 2, 3, N, d, causal, seed=950 + N + d,
                           dist="outlier_sd10")
    say(w.name + ("_causal" if causal else ""))
    q, k, v = (workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w))
    signs = workloads.gen_signs(d)
    q8, sq = oracle.blockquant_hadamard(q, signs, 128)
    k8, sk = oracle.blockquant_hadamard(k, signs, 128)
    v8, sv = oracle.blockquant_hadamard(v, None, 128)
    t8 = [_padded(c, torch.uint8, 0x7F) for c in (q8, k8, v8)]
    ts = [torch.from_numpy(s).to(DEV) for s in (sq, sk, sv)]
    o, lse = ea.attn_fwd_fp8(*t8, *ts, causal=causal, softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    o, lse = to_np(o), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    o_em, l_em, bound = emulation_with_bound(q8, k8, v8, sq, sk, sv, w.softmax_scale, causal)
    check_fp8(o, o_em, bound, w.name)
    o_ex, _ = oracle.naive_attention(q, k, v, w.softmax_scale, causal)
    e_kernel = float(np.sqrt(np.mean((o - o_em) ** 2)))
    e_scheme = float(np.sqrt(np.mean((o_em - o_ex) ** 2)))
    assert e_kernel <= 0.1 * e_scheme, (e_kernel, e_scheme)
    assert np.abs(lse - l_em).max() <= 1e-3


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [129, 1000])
def test_backward_nan_behind_inputs_and_workspace(N, d, causal):
    """Q, K, V, O, dO, LSE and the workspace all sit at the front of larger
    NaN-filled buffers."""
    B, H = 2, 3
    w = workloads.Workload(f"tail_bwd_n{N}_d{d}", B, H, N, d, causal, seed=980 + N + d)
    say(w.name + ("_causal" if causal else ""))
    q, k, v = (workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w))
    do = workloads.to_bf16_f32(workloads.gen_random((B, N, H, d), 990 + N))
    tq, tk, tv, tdo = (_padded(x, torch.bfloat16, float("nan")) for x in (q, k, v, do))
    o, lse = ea.attn_fwd_bf16(tq, tk, tv, causal=causal, softmax_scale=w.softmax_scale)
    to = _padded(to_np(o).astype(np.float32), torch.bfloat16, float("nan"))
    lbuf = torch.full((B * H * N + 1024,), float("nan"), dtype=torch.float32, device=DEV)
    lbuf[:B * H * N] = lse.reshape(-1)
    tlse = lbuf[:B * H * N].view(B, H, N)
    nws = ea.lib().attn_bwd_bf16_workspace_bytes(B, H, N) // 4
    wbuf = torch.full((nws + 1024,), float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = ea.attn_bwd_bf16(tq, tk, tv, to, tlse, tdo, causal=causal,
                                  softmax_scale=w.softmax_scale, workspace=wbuf[:nws])
    torch.cuda.synchronize()
    refs = oracle.attention_backward(q, k, v, do, w.softmax_scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        g = to_np(g)
        assert np.isfinite(g).all(), name
        nrm = float(np.sqrt(np.mean(r ** 2)))
        if nrm > 1e-6:
            assert float(np.sqrt(np.mean((g - r) ** 2))) / nrm <= 1e-2, name
