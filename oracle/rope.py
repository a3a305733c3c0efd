"""Rotary position embedding (RoPE) ahead of the FP8 pre-pass.

Test infrastructure only (see the package docstring).

[FA3-report] sections 2.2 and 3.3: the block quantisation of Q and K can be
fused into the rotary-embedding pass, which is memory-bound and reads and
writes Q and K anyway, so quantising costs no extra memory pass.  The pages do
not restate RoPE itself; this is the standard definition: for sequence
position n and pair i, with angle n theta_i,

    (x_a, x_b)  ->  (x_a cos - x_b sin,  x_a sin + x_b cos)

where the pair (a, b) is (2i, 2i + 1) ("interleaved") or (i, i + d/2)
("half-split").  cos and sin arrive as tables [N, d/2] (fp32), so the
frequency schedule (base, scaling, position offset) is the caller's choice.
"""
from __future__ import annotations

import numpy as np


def _pairs(d: int, interleaved: bool):
    i = np.arange(d // 2)
    return (2 * i, 2 * i + 1) if interleaved else (i, i + d // 2)


def rope_fp64(x, cos, sin, interleaved: bool) -> np.ndarray:
    """The rotation in fp64: x BSHD, cos/sin [N, d/2]; returns fp64 BSHD."""
    x = np.asarray(x, np.float64)
    c = np.asarray(cos, np.float64)[None, :, None, :]
    s = np.asarray(sin, np.float64)[None, :, None, :]
    a, b = _pairs(x.shape[-1], interleaved)
    y = x.copy()
    y[..., a] = x[..., a] * c - x[..., b] * s
    y[..., b] = x[..., a] * s + x[..., b] * c
    return y


def rope_fp32(x, cos, sin, interleaved: bool) -> np.ndarray:
    """The same rotation in float32 as the fused kernel computes it: each of
    the four products and the difference / sum rounded to fp32 on its own (no
    fused multiply-add).  Returns float32 BSHD."""
    x = np.asarray(x, np.float32)
    c = np.asarray(cos, np.float32)[None, :, None, :]
    s = np.asarray(sin, np.float32)[None, :, None, :]
    a, b = _pairs(x.shape[-1], interleaved)
    xa, xb = x[..., a], x[..., b]
    y = x.copy()
    y[..., a] = (xa * c).astype(np.float32) - (xb * s).astype(np.float32)
    y[..., b] = (xa * s).astype(np.float32) + (xb * c).astype(np.float32)
    return y
