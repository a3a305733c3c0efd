"""The FP8 pre-pass fused with a rotary embedding, on the GPU
([FA3-report] sections 2.2 and 3.3: quantisation riding on the RoPE pass).

Codes and scales must equal, bit for bit, the oracle's pre-pass applied to
the oracle's fp32 RoPE of the same bf16 rows (both take every decision in
fp32 with the same rounding steps).  End to end, Q and K through the fused
pre-pass and V through the plain one must give FP8 attention that meets the
FP8 gates against exact attention on the fp64-rotated inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_bound import check_fp8, emulation_with_bound
from gpu_helpers import DEV, say, to_np

import exact_attention_74_amd as ea

pytestmark = pytest.mark.gpu


def _host(B, N, H, d, seed, dist="outlier30"):
    w = workloads.Workload("rope", B, H, N, d, False, seed=seed, dist=dist)
    return [workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w)]


def _dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(DEV)


def _gpu_rope_quant(x, cos, sin, interleaved, signs, block_rows):
    s = None if signs is None else torch.from_numpy(signs).to(DEV)
    c, sc = ea.rope_blockquant_hadamard(_dev(x), _dev(cos, torch.float32), _dev(sin, torch.float32),
                                        interleaved, s, block_rows)
    torch.cuda.synchronize()
    return c.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 130, 1024])
@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("rotate,block_rows", [(True, 128), (False, 128), (True, 0)])
def test_rope_blockquant_bit_exact(d, N, interleaved, rotate, block_rows):
    say(f"rope blockquant d{d} N{N} inter{interleaved} rot{rotate} br{block_rows}")
    x = _host(2, N, 3, d, seed=80 + N)[0]
    cos, sin = workloads.rope_tables(N, d, offset=5)
    signs = workloads.gen_signs(d) if rotate else None
    c_gpu, s_gpu = _gpu_rope_quant(x, cos, sin, interleaved, signs, block_rows)
    c_ref, s_ref = oracle.blockquant_hadamard(oracle.rope_fp32(x, cos, sin, interleaved), signs,
                                              block_rows)
    assert np.array_equal(s_gpu, s_ref), np.abs(s_gpu - s_ref).max()
    assert np.array_equal(c_gpu, c_ref), f"{np.count_nonzero(c_gpu != c_ref)} codes differ"


def test_rope_blockquant_angle_zero_equals_plain_prepass():
    """cos = 1, sin = 0: the fused kernel gives exactly the plain pre-pass."""
    say("rope blockquant angle zero")
    x = _host(1, 300, 2, 128, seed=90)[0]
    cos, sin = np.ones((300, 64), np.float32), np.zeros((300, 64), np.float32)
    signs = workloads.gen_signs(128)
    c1, s1 = _gpu_rope_quant(x, cos, sin, True, signs, 128)
    c2, s2 = ea.blockquant_hadamard(_dev(x), torch.from_numpy(signs).to(DEV), 128)
    torch.cuda.synchronize()
    assert np.array_equal(c1, c2.cpu().numpy()) and np.array_equal(s1, s2.cpu().numpy())


@pytest.mark.parametrize("causal", [False, True])
def test_rope_fp8_attention_end_to_end(causal):
    B, N, H, d = 2, 1024, 4, 128
    say(f"rope fp8 end to end causal={causal}")
    q, k, v = _host(B, N, H, d, seed=91, dist="outlier_sd10")
    cos, sin = workloads.rope_tables(N, d)
    signs = workloads.gen_signs(d)
    ts = torch.from_numpy(signs).to(DEV)
    tc, tsn = _dev(cos, torch.float32), _dev(sin, torch.float32)
    q8, sq = ea.rope_blockquant_hadamard(_dev(q), tc, tsn, False, ts)
    k8, sk = ea.rope_blockquant_hadamard(_dev(k), tc, tsn, False, ts)
    v8, sv = ea.blockquant_hadamard(_dev(v), None)
    scale = d ** -0.5
    o, _ = ea.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    o = to_np(o)
    # exact attention on the fp64-rotated bf16 inputs
    qr, kr = (oracle.rope_fp64(x, cos, sin, False) for x in (q, k))
    o_ex, _ = oracle.naive_attention(qr, kr, v, scale, causal)
    # the FP8 emulation from the oracle's own fused pre-pass
    qc, qs = oracle.blockquant_hadamard(oracle.rope_fp32(q, cos, sin, False), signs, 128)
    kc, ks = oracle.blockquant_hadamard(oracle.rope_fp32(k, cos, sin, False), signs, 128)
    vc, vs = oracle.blockquant_hadamard(v, None, 128)
    o_em, _, bound = emulation_with_bound(qc, kc, vc, qs, ks, vs, scale, causal)
    check_fp8(o, o_em, bound, f"rope fp8 causal={causal}")
    rmse = float(np.sqrt(np.mean((o - o_ex) ** 2)))
    e_kernel = float(np.sqrt(np.mean((o - o_em) ** 2)))
    e_scheme = float(np.sqrt(np.mean((o_em - o_ex) ** 2)))
    print(f"rope fp8 causal={causal}: rmse vs exact {rmse:.3e}, gpu-emul {e_kernel:.3e}, "
          f"emul-exact {e_scheme:.3e}", flush=True)
    assert rmse <= 3e-2
    assert e_kernel <= 0.1 * e_scheme
