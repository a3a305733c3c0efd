"""exact_attention_74_amd: fused exact attention forward (bf16 and FP8) for MI355X.

Thin ctypes binding over ``libexattn.so`` (C ABI declared in include/exattn.h).
The functions here only check and marshal torch tensors (device pointers,
shapes, the current HIP stream); every step of the computation runs in the
library's gfx950 kernels.  There is no CPU or eager fallback: if the library is
missing or fails to load, every call raises.

Entry points (same names as the C ABI):
  attn_fwd_bf16(q, k, v, causal=False, softmax_scale=None) -> (o, lse)
  blockquant_hadamard(x, signs=None, block_rows=128) -> (x8, scale)
  attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal=False, softmax_scale=None) -> (o, lse)
  attn_fwd_bf16_same_phase(q, k, v, causal=False, softmax_scale=None) -> (o, lse): the same
    results from the same-phase schedule (attn_fwd_bf16 pipelines the interior key tiles)
  attn_fwd_bf16_gqa / attn_fwd_fp8_gqa: the same with K/V (and their scales) on
    H_kv heads, H a multiple of H_kv (grouped-query / multi-query attention).
  attn_bwd_bf16(q, k, v, o, lse, do, causal=False, softmax_scale=None) -> (dq, dk, dv)
  rope_blockquant_hadamard(x, cos, sin, interleaved, signs=None, block_rows=128) -> (x8, scale)
Tensors are BSHD (batch, seqlen, heads, head_dim), contiguous, on a HIP device.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libexattn.so")

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_float = ctypes.c_float

# (name, argtypes) for every symbol of include/exattn.h
SIGNATURES = {
    "attn_fwd_bf16": [_c_void_p] * 5 + [_c_int] * 5 + [_c_float, _c_void_p],
    "attn_fwd_bf16_same_phase": [_c_void_p] * 5 + [_c_int] * 5 + [_c_float, _c_void_p],
    "attn_fwd_fp8": [_c_void_p] * 8 + [_c_int] * 5 + [_c_float, _c_void_p],
    "attn_fwd_bf16_gqa": [_c_void_p] * 5 + [_c_int] * 6 + [_c_float, _c_void_p],
    "attn_fwd_fp8_gqa": [_c_void_p] * 8 + [_c_int] * 6 + [_c_float, _c_void_p],
    "attn_bwd_bf16": [_c_void_p] * 10 + [_c_int] * 5 + [_c_float, _c_void_p],
    "attn_bwd_bf16_gqa": [_c_void_p] * 10 + [_c_int] * 6 + [_c_float, _c_void_p],
    "attn_bwd_bf16_workspace_bytes": [_c_int] * 3,
    "attn_bwd_bf16_noalloc": [_c_void_p] * 9 + [_c_int] * 6 + [_c_float, _c_void_p],
    "rope_blockquant_hadamard": [_c_void_p] * 6 + [_c_int] * 6 + [_c_void_p],
    "blockquant_hadamard": [_c_void_p] * 4 + [_c_int] * 5 + [_c_void_p],
    "exattn_strerror": [_c_int],
    "exattn_abi_version": [],
}
RESTYPES = {"exattn_strerror": ctypes.c_char_p, "attn_bwd_bf16_workspace_bytes": ctypes.c_longlong}

ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_VALUE, ERR_HIP, ERR_SCRATCH = -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 16 << 20  # EXATTN_NOALLOC_SCRATCH_BYTES

# torch device type that every tensor argument must have (HIP devices appear
# as "cuda" in PyTorch-ROCm)
_DEVICE_TYPE = "cuda"

_lib = None


class ExattnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed with code {code}: {strerror(code)}")


def lib() -> ctypes.CDLL:
    """The loaded libexattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m exact_attention_74_amd.build` (no fallback exists)")
        h = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = RESTYPES.get(name, _c_int)
        _lib = h
    return _lib


def strerror(code: int) -> str:
    return lib().exattn_strerror(int(code)).decode()


def _stream_ptr(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_bshd(name: str, t: torch.Tensor, dtype) -> tuple[int, int, int, int]:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != _DEVICE_TYPE:
        raise ValueError(f"{name} must be on a HIP device (got {t.device})")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must have dtype {dtype} (got {t.dtype})")
    if t.dim() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 4-D BSHD tensor")
    return tuple(t.shape)


def _check_out(name: str, t, shape, dtype, device) -> None:
    """A caller-supplied output (or a scale input) must match exactly: the C
    ABI sees only a pointer, so a short buffer would be overrun on the GPU."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    dtypes = dtype if isinstance(dtype, tuple) else (dtype,)
    if (t.dtype not in dtypes or tuple(t.shape) != tuple(shape) or not t.is_contiguous()
            or t.device != device):
        raise ValueError(f"{name} must be a contiguous {dtypes[0]} tensor of shape "
                         f"{tuple(shape)} on {device} (got {t.dtype} {tuple(t.shape)} on "
                         f"{t.device}{'' if t.is_contiguous() else ', not contiguous'})")


def _call(fn: str, *args) -> None:
    rc = getattr(lib(), fn)(*args)
    if rc != 0:
        raise ExattnError(fn, rc)


def _kv_heads(name: str, q_shape, k_shape, v_shape, grouped: bool) -> int:
    """K/V head count after checking the K/V shapes against Q's [B, N, H, d]."""
    B, N, H, d = q_shape
    if k_shape != v_shape:
        raise ValueError(f"{name}: k and v must have the same shape")
    if (k_shape[0], k_shape[1], k_shape[3]) != (B, N, d):
        raise ValueError(f"{name}: k, v must be [B, N, H_kv, d] with q's B, N, d")
    Hkv = k_shape[2]
    if not grouped and Hkv != H:
        raise ValueError(f"{name}: q, k, v must have the same shape (use {name}_gqa for H_kv < H)")
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"{name}: H = {H} must be a multiple of H_kv = {Hkv}")
    return Hkv


def _bf16(fn, q, k, v, causal, softmax_scale, out, lse):
    shape = _check_bshd("q", q, torch.bfloat16)
    Hkv = _kv_heads("attn_fwd_bf16", shape, _check_bshd("k", k, torch.bfloat16),
                    _check_bshd("v", v, torch.bfloat16), fn.endswith("_gqa"))
    B, N, H, d = shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    for name, t in (("k", k), ("v", v)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out("out", out, (B, N, H, d), torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    heads = (H, Hkv) if fn.endswith("_gqa") else (H,)
    _call(fn, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
          B, *heads, N, d, int(bool(causal)), scale, _stream_ptr(q))
    return out, lse


def attn_fwd_bf16(q, k, v, causal: bool = False, softmax_scale: float | None = None,
                  out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """O = softmax(scale Q K^T [causal]) V in bf16; returns (O bf16 BSHD, LSE fp32 [B,H,N])."""
    return _bf16("attn_fwd_bf16", q, k, v, causal, softmax_scale, out, lse)


def attn_fwd_bf16_same_phase(q, k, v, causal: bool = False, softmax_scale: float | None = None,
                             out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """attn_fwd_bf16 with the same-phase schedule everywhere (attn_fwd_bf16
    pipelines the interior key tiles: non-causal everywhere, causal from N = 1024);
    results bit-identical to it."""
    return _bf16("attn_fwd_bf16_same_phase", q, k, v, causal, softmax_scale, out, lse)


def attn_fwd_bf16_gqa(q, k, v, causal: bool = False, softmax_scale: float | None = None,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """attn_fwd_bf16 with K/V on H_kv heads ([B, N, H_kv, d]); query head h uses
    K/V head h // (H // H_kv)."""
    return _bf16("attn_fwd_bf16_gqa", q, k, v, causal, softmax_scale, out, lse)


def _quant_outputs(x, out, scale):
    """The pre-pass outputs: allocated here, or checked when the caller passes them."""
    B, N, H, d = x.shape
    nsb = (N + 127) // 128
    if out is None:
        out = torch.empty((B, N, H, d), dtype=torch.uint8, device=x.device)
    else:
        _check_out("out", out, (B, N, H, d), (torch.uint8, torch.float8_e4m3fn), x.device)
    if scale is None:
        scale = torch.empty((B, H, nsb), dtype=torch.float32, device=x.device)
    else:
        _check_out("scale", scale, (B, H, nsb), torch.float32, x.device)
    return out, scale


def blockquant_hadamard(x, signs: torch.Tensor | None = None, block_rows: int = 128,
                        out: torch.Tensor | None = None, scale: torch.Tensor | None = None):
    """Rotate (if ``signs``) and block-quantise a bf16 BSHD tensor to e4m3.

    Returns (codes uint8 BSHD, scale fp32 [B, H, ceil(N/128)]).
    """
    B, N, H, d = _check_bshd("x", x, torch.bfloat16)
    if signs is not None:
        if signs.device != x.device or signs.dtype != torch.float32 or signs.numel() != d:
            raise ValueError("signs must be d float32 values on the same device")
        signs = signs.contiguous()
    out, scale = _quant_outputs(x, out, scale)
    _call("blockquant_hadamard", x.data_ptr(), out.data_ptr(), scale.data_ptr(),
          signs.data_ptr() if signs is not None else None, B, H, N, d, int(block_rows),
          _stream_ptr(x))
    return out, scale


def _fp8(fn, q8, k8, v8, q_scale, k_scale, v_scale, causal, softmax_scale, out, lse):
    codes = (torch.uint8, torch.float8_e4m3fn)
    shape = _check_bshd("q8", q8, codes)
    Hkv = _kv_heads("attn_fwd_fp8", shape, _check_bshd("k8", k8, codes),
                    _check_bshd("v8", v8, codes), fn.endswith("_gqa"))
    B, N, H, d = shape
    nsb = (N + 127) // 128
    for name, t in (("k8", k8), ("v8", v8)):
        if t.device != q8.device:
            raise ValueError(f"{name} must be on q8's device")
    for name, s, h in (("q_scale", q_scale, H), ("k_scale", k_scale, Hkv), ("v_scale", v_scale, Hkv)):
        _check_out(name, s, (B, h, nsb), torch.float32, q8.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=q8.device)
    else:
        _check_out("out", out, (B, N, H, d), torch.bfloat16, q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    else:
        _check_out("lse", lse, (B, H, N), torch.float32, q8.device)
    heads = (H, Hkv) if fn.endswith("_gqa") else (H,)
    _call(fn, q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_scale.data_ptr(),
          k_scale.data_ptr(), v_scale.data_ptr(), out.data_ptr(), lse.data_ptr(), B, *heads, N, d,
          int(bool(causal)), scale, _stream_ptr(q8))
    return out, lse


def rope_blockquant_hadamard(x, cos, sin, interleaved: bool, signs: torch.Tensor | None = None,
                             block_rows: int = 128, out: torch.Tensor | None = None,
                             scale: torch.Tensor | None = None):
    """blockquant_hadamard of x after a rotary embedding with the float32
    cos/sin tables [N, d/2] (pairs (2i, 2i+1) if ``interleaved`` else (i, i+d/2))."""
    B, N, H, d = _check_bshd("x", x, torch.bfloat16)
    for name, t in (("cos", cos), ("sin", sin)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != x.device
                or tuple(t.shape) != (N, d // 2) or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [N, d/2] tensor on x's device")
    if signs is not None:
        if signs.device != x.device or signs.dtype != torch.float32 or signs.numel() != d:
            raise ValueError("signs must be d float32 values on the same device")
        signs = signs.contiguous()
    out, scale = _quant_outputs(x, out, scale)
    _call("rope_blockquant_hadamard", x.data_ptr(), out.data_ptr(), scale.data_ptr(),
          signs.data_ptr() if signs is not None else None, cos.data_ptr(), sin.data_ptr(),
          int(bool(interleaved)), B, H, N, d, int(block_rows), _stream_ptr(x))
    return out, scale


def attn_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False,
                 softmax_scale: float | None = None, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None):
    """FP8 attention on e4m3 codes (uint8 or float8_e4m3fn) with block scales."""
    return _fp8("attn_fwd_fp8", q8, k8, v8, q_scale, k_scale, v_scale, causal, softmax_scale,
                out, lse)


def attn_fwd_fp8_gqa(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False,
                     softmax_scale: float | None = None, out: torch.Tensor | None = None,
                     lse: torch.Tensor | None = None):
    """attn_fwd_fp8 with K/V codes [B, N, H_kv, d] and K/V scales [B, H_kv, ceil(N/128)]."""
    return _fp8("attn_fwd_fp8_gqa", q8, k8, v8, q_scale, k_scale, v_scale, causal, softmax_scale,
                out, lse)


def attn_bwd_bf16(q, k, v, o, lse, do, causal: bool = False, softmax_scale: float | None = None,
                  dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                  dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Gradients (dQ, dK, dV) of attn_fwd_bf16 given its output ``o``, its LSE and
    the output gradient ``do`` (all bf16 BSHD except the fp32 [B, H, N] LSE).
    k and v may have H_kv heads (grouped-query); dk, dv then have H_kv heads.

    ``workspace``: optional float32 device tensor of at least
    attn_bwd_bf16_workspace_bytes(B, H, N) bytes; allocated here if omitted.
    """
    shape = _check_bshd("q", q, torch.bfloat16)
    for name, t in (("o", o), ("do", do)):
        if _check_bshd(name, t, torch.bfloat16) != shape:
            raise ValueError(f"{name} must have q's shape")
    Hkv = _kv_heads("attn_bwd_bf16", shape, _check_bshd("k", k, torch.bfloat16),
                    _check_bshd("v", v, torch.bfloat16), grouped=True)
    B, N, H, d = shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device")
    _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_out("dq", dq, (B, N, H, d), torch.bfloat16, q.device)
    _check_out("dk", dk, tuple(k.shape), torch.bfloat16, q.device)
    _check_out("dv", dv, tuple(v.shape), torch.bfloat16, q.device)
    nbytes = lib().attn_bwd_bf16_workspace_bytes(B, H, N)
    if nbytes < 0:
        raise ExattnError("attn_bwd_bf16_workspace_bytes", nbytes)
    if workspace is None:
        workspace = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device=q.device)
    elif (workspace.dtype != torch.float32 or workspace.device != q.device
          or workspace.numel() * 4 < nbytes or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous float32 tensor of >= {nbytes} bytes")
    _call("attn_bwd_bf16_gqa", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
          do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
          workspace.data_ptr(), B, H, Hkv, N, d, int(bool(causal)), scale, _stream_ptr(q))
    return dq, dk, dv


def attn_bwd_bf16_noalloc(q, k, v, o, lse, do, dq, dk, dv, causal: bool = False,
                          softmax_scale: float | None = None):
    """attn_bwd_bf16 into caller-supplied dq, dk, dv with no device allocation
    at all (the per-row workspace lives in the library's fixed per-GPU
    scratch; 8 B H N must be <= NOALLOC_SCRATCH_BYTES).  Calls overlapping on
    one GPU race on that scratch.  Returns (dq, dk, dv)."""
    shape = _check_bshd("q", q, torch.bfloat16)
    for name, t in (("o", o), ("do", do)):
        if _check_bshd(name, t, torch.bfloat16) != shape:
            raise ValueError(f"{name} must have q's shape")
    Hkv = _kv_heads("attn_bwd_bf16", shape, _check_bshd("k", k, torch.bfloat16),
                    _check_bshd("v", v, torch.bfloat16), grouped=True)
    B, N, H, d = shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        if t.device != q.device:
            raise ValueError(f"{name} must be on q's device")
    _check_out("lse", lse, (B, H, N), torch.float32, q.device)
    _check_out("dq", dq, (B, N, H, d), torch.bfloat16, q.device)
    _check_out("dk", dk, tuple(k.shape), torch.bfloat16, q.device)
    _check_out("dv", dv, tuple(v.shape), torch.bfloat16, q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    _call("attn_bwd_bf16_noalloc", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
          do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv,
          N, d, int(bool(causal)), scale, _stream_ptr(q))
    return dq, dk, dv


__all__ = ["attn_fwd_bf16", "attn_fwd_fp8", "attn_fwd_bf16_gqa", "attn_fwd_fp8_gqa", "attn_bwd_bf16",
           "attn_bwd_bf16_noalloc",
           "blockquant_hadamard", "rope_blockquant_hadamard", "lib", "strerror",
           "ExattnError", "LIB_PATH", "SIGNATURES"]
