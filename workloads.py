"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random numbers and names shapes. It holds none of the
attention, softmax, rotation or quantisation arithmetic: both the CPU oracle
(``oracle/``) and the HIP library are fed from here, and neither imports the
other.

Every tensor is generated in float32 on the host with ``numpy.random.default_rng``
and, for the bf16 path, cast to bfloat16 by torch (round to nearest even).  The
layout is BSHD, ``(batch, seqlen, nheads, head_dim)``, the layout of the
FlashAttention-3 Python interface described in the 0539edu blog on FlashAttention
V3, section 4.2.

Workload shapes follow the sizes the FlashAttention-3 report (zako-mio knowledge
base, section 4.1 and 4.2) measures on: sequence lengths 512..16k, head dims 64
and 128, and the ablation shape {batch 4, heads 16, head dim 128, seqlen ~8k}.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    dist: str = "normal"          # "normal" | "outlier30" | "outlier_sd10"
    d_logical: int | None = None  # head dim before zero padding (d=96 -> 128)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(self.d_logical or self.d) ** 0.5

    def flops(self) -> float:
        """4*B*H*N^2*d (two N x N x d matmuls), halved for causal.

        Uses the logical head dim, so a zero-padded d=96 run is credited with
        d=96 work only.
        """
        f = 4.0 * self.B * self.H * self.N * self.N * float(self.d_logical or self.d)
        return f / 2 if self.causal else f


# The tiny case, the mid-size bf16 case, the sequence sweep, the fp8 case and the
# long single-request case.
TINY = Workload("tiny_b1h2n256d64", 1, 2, 256, 64, False, seed=0)
TINY_CAUSAL = dataclasses.replace(TINY, name="tiny_b1h2n256d64_causal", causal=True)
MID = Workload("bf16_b2h32n4096d128", 2, 32, 4096, 128, False, seed=1)
MID_CAUSAL = dataclasses.replace(MID, name="bf16_b2h32n4096d128_causal", causal=True)
FP8 = Workload("fp8_b4h16n8192d128", 4, 16, 8192, 128, False, seed=3, dist="outlier30")
FP8_PAGE = dataclasses.replace(FP8, name="fp8_b4h16n8192d128_pagedist", dist="outlier_sd10")
BF16_HEADLINE = Workload("bf16_b4h16n8192d128", 4, 16, 8192, 128, False, seed=3)
LONG = Workload("long_b1h8n32768d128_causal", 1, 8, 32768, 128, True, seed=5)

SIGNS_SEED = 4


def sweep(causal: bool) -> list[Workload]:
    """16384 tokens per batch: N in 512..16k, B = 16384/N.

    H=16 at d=128, H=32 at d=64, and d=96 (H=16) zero-padded to 128.
    """
    out = []
    for n in (512, 1024, 2048, 4096, 8192, 16384):
        b = 16384 // n
        tag = "c" if causal else "nc"
        out.append(Workload(f"sweep_n{n}_d128_{tag}", b, 16, n, 128, causal, seed=2))
        out.append(Workload(f"sweep_n{n}_d64_{tag}", b, 32, n, 64, causal, seed=2))
        out.append(Workload(f"sweep_n{n}_d96_{tag}", b, 16, n, 128, causal, seed=2, d_logical=96))
    return out


def gen_qkv(w: Workload) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V as float32 BSHD arrays drawn from ``w.seed``.

    dist:
      normal        N(0, 1)
      outlier30     N(0, 1), and an iid Bernoulli(1e-3) subset of entries x30
      outlier_sd10  N(0, 1) + N(0, 100) * Bernoulli(1e-3)  (variance 100)
    d_logical < d: columns d_logical.. are zero (caller-side head-dim padding).
    """
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.N, w.H, w.d)
    out = []
    for _ in range(3):
        x = rng.standard_normal(shape, dtype=np.float32)
        if w.dist == "outlier30":
            m = rng.random(shape, dtype=np.float32) < 1e-3
            x = np.where(m, x * np.float32(30.0), x)
        elif w.dist == "outlier_sd10":
            m = rng.random(shape, dtype=np.float32) < 1e-3
            x = x + np.where(m, np.float32(10.0) * rng.standard_normal(shape, dtype=np.float32),
                             np.float32(0.0))
        elif w.dist != "normal":
            raise ValueError(w.dist)
        if w.d_logical is not None and w.d_logical < w.d:
            x[..., w.d_logical:] = 0.0
        out.append(np.ascontiguousarray(x, dtype=np.float32))
    return out[0], out[1], out[2]


def gen_qkv_gqa(B: int, N: int, H: int, Hkv: int, d: int, seed: int, dist: str = "normal"):
    """Q on H heads and K, V on Hkv heads (BSHD float32) for grouped-query
    attention, drawn like ``gen_qkv``: Q from ``seed``, K and V from the next
    draws of the same stream."""
    q = gen_qkv(Workload("q", B, H, N, d, False, seed=seed, dist=dist))[0]
    _, k, v = gen_qkv(Workload("kv", B, Hkv, N, d, False, seed=seed + 1, dist=dist))
    return q, k, v


def rope_tables(N: int, d: int, base: float = 10000.0, offset: int = 0):
    """cos, sin tables [N, d/2] (float32) of the usual RoPE frequency schedule,
    angle (offset + n) * base^(-2 i / d), evaluated in fp64 and rounded once."""
    n = np.arange(N, dtype=np.float64)[:, None] + offset
    inv = base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    ang = n * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def gen_signs(d: int, seed: int = SIGNS_SEED) -> np.ndarray:
    """d random signs (+1/-1, float32) for the incoherent-processing diagonal."""
    rng = np.random.default_rng(seed)
    return np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)


def gen_random(shape, seed: int) -> np.ndarray:
    """Plain N(0,1) float32 array (small ad-hoc test shapes)."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def sample_rows(B: int, H: int, N: int, count: int, seed: int) -> np.ndarray:
    """``count`` distinct (b, h, i) query coordinates, int64 [count, 3].

    Always includes row 0 and row N-1 of (0, 0) so the first and last query
    tiles are covered.
    """
    rng = np.random.default_rng(seed)
    total = B * H * N
    count = min(count, total)
    flat = rng.choice(total, size=count, replace=False)
    flat[0] = 0
    if count > 1:
        flat[1] = N - 1
    flat = np.unique(flat)
    b = flat // (H * N)
    h = (flat // N) % H
    i = flat % N
    return np.stack([b, h, i], axis=1).astype(np.int64)


# (b, h) heads of the FP8 workload whose sampled query rows the FP8 accuracy
# figures are taken on (128 rows each, seed 77 + h)
FP8_ACCURACY_HEADS = ((0, 0), (1, 5), (2, 10), (3, 15))


def fp8_accuracy_rows(N: int):
    """[(b, h, rows)] for the FP8 accuracy figures: 128 sampled query rows in
    each head of FP8_ACCURACY_HEADS (rows as int64 indices into the sequence)."""
    return [(b, h, sample_rows(1, 1, N, 128, seed=77 + h)[:, 2]) for b, h in FP8_ACCURACY_HEADS]


def to_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (RNE, via torch) and return the values as float32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float32).numpy()
