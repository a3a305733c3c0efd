"""The Python binding's argument checks, on the CPU.

The C ABI receives bare pointers, so the binding is what stops an undersized,
mistyped, strided or host-resident output (or scale) tensor from reaching a
kernel that would write or read past it.  Every case here must raise before
the library is called.  Tensors live on torch's "meta" device (shapes and
dtypes without storage), with the binding's device type switched to it.
"""
import pytest
import torch

import exact_attention_74_amd as ea


@pytest.fixture(autouse=True)
def meta_device(monkeypatch):
    monkeypatch.setattr(ea, "_DEVICE_TYPE", "meta")
    monkeypatch.setattr(ea, "_call", lambda *a: pytest.fail("the library must not be called"))


M = torch.device("meta")
B, N, H, d = 2, 300, 4, 64
NSB = (N + 127) // 128


def t(shape, dtype=torch.bfloat16, device=M):
    return torch.empty(shape, dtype=dtype, device=device)


def qkv():
    return t((B, N, H, d)), t((B, N, H, d)), t((B, N, H, d))


BAD_O = [t((B, N, H, d - 8)), t((B, N - 1, H, d)), t((B, N, H, d), torch.float32),
         t((B, N, H, 2 * d))[..., :d], t((B, N, H, d), device=torch.device("cpu"))]
BAD_LSE = [t((B, H, N - 1), torch.float32), t((B, H, N), torch.bfloat16),
           t((B, N, H), torch.float32).transpose(1, 2), t((B, H, N), torch.float32, torch.device("cpu"))]


@pytest.mark.parametrize("i", range(len(BAD_O)))
def test_bf16_forward_rejects_bad_out(i):
    with pytest.raises(ValueError):
        ea.attn_fwd_bf16(*qkv(), out=BAD_O[i])


@pytest.mark.parametrize("i", range(len(BAD_LSE)))
def test_bf16_forward_rejects_bad_lse(i):
    with pytest.raises(ValueError):
        ea.attn_fwd_bf16(*qkv(), lse=BAD_LSE[i])


def fp8_args(**kw):
    a = dict(q8=t((B, N, H, d), torch.uint8), k8=t((B, N, H, d), torch.uint8),
             v8=t((B, N, H, d), torch.uint8), q_scale=t((B, H, NSB), torch.float32),
             k_scale=t((B, H, NSB), torch.float32), v_scale=t((B, H, NSB), torch.float32))
    a.update(kw)
    return a


@pytest.mark.parametrize("name", ["q_scale", "k_scale", "v_scale"])
@pytest.mark.parametrize("bad", [t((B, H, NSB - 1), torch.float32),
                                 t((B, H, NSB), torch.float16),
                                 t((B, H, NSB), torch.float32, torch.device("cpu")),
                                 t((B, H, 2 * NSB), torch.float32)[..., ::2]])
def test_fp8_forward_rejects_bad_scales(name, bad):
    with pytest.raises(ValueError):
        ea.attn_fwd_fp8(**fp8_args(**{name: bad}))


@pytest.mark.parametrize("i", range(len(BAD_O)))
def test_fp8_forward_rejects_bad_out(i):
    with pytest.raises(ValueError):
        ea.attn_fwd_fp8(**fp8_args(), out=BAD_O[i])


@pytest.mark.parametrize("i", range(len(BAD_LSE)))
def test_fp8_forward_rejects_bad_lse(i):
    with pytest.raises(ValueError):
        ea.attn_fwd_fp8(**fp8_args(), lse=BAD_LSE[i])


def test_fp8_gqa_scale_heads():
    k8 = t((B, N, 2, d), torch.uint8)
    ok = t((B, 2, NSB), torch.float32)
    with pytest.raises(ValueError):  # K/V scales must have H_kv heads
        ea.attn_fwd_fp8_gqa(**fp8_args(k8=k8, v8=k8, k_scale=t((B, H, NSB), torch.float32),
                                       v_scale=ok))


@pytest.mark.parametrize("bad_out,bad_scale", [
    (t((B, N, H, d - 1), torch.uint8), None),
    (t((B, N, H, d), torch.bfloat16), None),
    (t((B, N, H, d), torch.uint8, torch.device("cpu")), None),
    (None, t((B, H, NSB - 1), torch.float32)),
    (None, t((B, H, NSB), torch.float64)),
    (None, t((B, H, NSB), torch.float32, torch.device("cpu"))),
])
def test_prepasses_reject_bad_outputs(bad_out, bad_scale):
    x = t((B, N, H, d))
    with pytest.raises(ValueError):
        ea.blockquant_hadamard(x, None, 128, out=bad_out, scale=bad_scale)
    cs = t((N, d // 2), torch.float32)
    with pytest.raises(ValueError):
        ea.rope_blockquant_hadamard(x, cs, cs, True, None, 128, out=bad_out, scale=bad_scale)


def test_prepass_rejects_host_signs():
    with pytest.raises(ValueError):
        ea.blockquant_hadamard(t((B, N, H, d)), t((d,), torch.float32, torch.device("cpu")))


@pytest.mark.parametrize("name", ["dq", "dk", "dv"])
@pytest.mark.parametrize("bad", [t((B, N, H, d - 8)), t((B, N, H, d), torch.float16),
                                 t((B, N, H, d), device=torch.device("cpu")),
                                 t((B, N, H, 2 * d))[..., ::2]])
def test_backward_rejects_bad_gradients(name, bad):
    q, k, v = qkv()
    lse = t((B, H, N), torch.float32)
    with pytest.raises(ValueError):
        ea.attn_bwd_bf16(q, k, v, t((B, N, H, d)), lse, t((B, N, H, d)), **{name: bad})


def test_backward_rejects_bad_lse_and_gqa_gradient_heads():
    q, k, v = qkv()
    with pytest.raises(ValueError):
        ea.attn_bwd_bf16(q, k, v, t((B, N, H, d)), t((B, H, N - 1), torch.float32),
                         t((B, N, H, d)))
    k2, v2 = t((B, N, 2, d)), t((B, N, 2, d))
    with pytest.raises(ValueError):  # dk for a grouped-query call must have H_kv heads
        ea.attn_bwd_bf16(q, k2, v2, t((B, N, H, d)), t((B, H, N), torch.float32),
                         t((B, N, H, d)), dk=t((B, N, H, d)))


def test_inputs_on_other_devices_rejected():
    q, k, v = qkv()
    with pytest.raises(ValueError):
        ea.attn_fwd_bf16(q, k, t((B, N, H, d), device=torch.device("cpu")))


def test_valid_arguments_reach_the_library(monkeypatch):
    """The checks accept exactly-shaped outputs: each entry point reaches the
    library call once (recorded here instead of made)."""
    calls = []
    monkeypatch.setattr(ea, "_call", lambda fn, *a: calls.append(fn))
    monkeypatch.setattr(ea, "_stream_ptr", lambda x: 0)
    q, k, v = qkv()
    ea.attn_fwd_bf16(q, k, v, out=t((B, N, H, d)), lse=t((B, H, N), torch.float32))
    ea.attn_fwd_fp8(**fp8_args(), out=t((B, N, H, d)), lse=t((B, H, N), torch.float32))
    ea.blockquant_hadamard(q, t((d,), torch.float32), 128, out=t((B, N, H, d), torch.uint8),
                           scale=t((B, H, NSB), torch.float32))
    cs = t((N, d // 2), torch.float32)
    ea.rope_blockquant_hadamard(q, cs, cs, False, None, 0, out=t((B, N, H, d), torch.uint8),
                                scale=t((B, H, NSB), torch.float32))
    k2, v2 = t((B, N, 2, d)), t((B, N, 2, d))
    ea.attn_bwd_bf16(q, k2, v2, t((B, N, H, d)), t((B, H, N), torch.float32), t((B, N, H, d)),
                     dq=t((B, N, H, d)), dk=t((B, N, 2, d)), dv=t((B, N, 2, d)))
    assert calls == ["attn_fwd_bf16", "attn_fwd_fp8", "blockquant_hadamard",
                     "rope_blockquant_hadamard", "attn_bwd_bf16_gqa"]
