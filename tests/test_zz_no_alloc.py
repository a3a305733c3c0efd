"""attn_bwd_bf16_noalloc, the gradient entry point that allocates nothing
(for callers under graph capture or that may not call hipMalloc): through the
C ABI it must return exactly what attn_bwd_bf16_gqa returns with a caller
workspace, on two calls in a row, the second with a smaller problem (the
shared scratch still holds the first call's rows)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import DEV, say, to_np

import exact_attention_74_amd as ea

pytestmark = pytest.mark.gpu


def _problem(B, N, H, Hkv, d, causal, seed):
    q, k, v = workloads.gen_qkv_gqa(B, N, H, Hkv, d, seed)
    do = workloads.gen_random((B, N, H, d), seed + 7)
    host = [workloads.to_bf16_f32(x) for x in (q, k, v, do)]
    tq, tk, tv, tdo = (torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in host)
    scale = d ** -0.5
    o, lse = ea.attn_fwd_bf16_gqa(tq, tk, tv, causal=causal, softmax_scale=scale)
    return host, (tq, tk, tv, o, tdo, lse), scale


def _with_workspace(t, B, H, Hkv, N, d, causal, scale):
    q, k, v, o, do, lse = t
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.lib().attn_bwd_bf16_workspace_bytes(B, H, N) // 4, dtype=torch.float32,
                     device=DEV)
    rc = ea.lib().attn_bwd_bf16_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                    dv.data_ptr(), ws.data_ptr(), B, H, Hkv, N, d, int(causal),
                                    scale, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    return dq, dk, dv


def _no_alloc(t, B, H, Hkv, N, d, causal, scale):
    q, k, v, o, do, lse = t
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    torch.cuda.synchronize()
    rc = ea.lib().attn_bwd_bf16_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d,
                                        int(causal), scale, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, ea.strerror(rc)
    return dq, dk, dv


def test_no_alloc_matches_workspace_entry_point_twice():
    # first a larger grouped-query causal problem, then a smaller MHA one
    for (B, N, H, Hkv, d, causal, seed) in ((2, 1000, 8, 2, 128, True, 700),
                                            (1, 300, 2, 2, 64, False, 710)):
        say(f"noalloc B{B} N{N} H{H} Hkv{Hkv} d{d} causal={causal}")
        host, t, scale = _problem(B, N, H, Hkv, d, causal, seed)
        ref = _with_workspace(t, B, H, Hkv, N, d, causal, scale)
        got = _no_alloc(t, B, H, Hkv, N, d, causal, scale)
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g, r), name
        # and within the gradient gate against the fp64 oracle
        refs = oracle.attention_backward(*host, scale, causal)
        for name, g, r in zip(("dq", "dk", "dv"), got, refs):
            e = to_np(g) - r
            assert np.sqrt(np.mean(e ** 2)) <= 1e-2 * np.sqrt(np.mean(r ** 2)), name



def test_no_alloc_at_the_scratch_limit():
    """B H N = 2^21 rows: the per-row workspace (8 bytes a row) fills the
    scratch array exactly.  Bit for bit against the workspace entry point;
    inputs drawn on the device (no oracle is involved in this comparison)."""
    B, H, N, d = 8, 16, 16384, 128
    assert 8 * B * H * N == ea.NOALLOC_SCRATCH_BYTES
    say(f"noalloc at the scratch limit b{B}h{H}n{N}d{d}")
    g = torch.Generator(device=DEV).manual_seed(11)
    q, k, v, do = (torch.randn((B, N, H, d), generator=g, device=DEV).to(torch.bfloat16)
                   for _ in range(4))
    scale = d ** -0.5
    o, lse = ea.attn_fwd_bf16(q, k, v, causal=True, softmax_scale=scale)
    t = (q, k, v, o, do, lse)
    want = _with_workspace(t, B, H, H, N, d, True, scale)
    got = _no_alloc(t, B, H, H, N, d, True, scale)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv"), got, want):
        assert torch.isfinite(x.float()).all(), name
        assert torch.equal(x, y), name
