"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
call the library through its binding, and compute error metrics."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads

DEV = torch.device("cuda:0")


def say(msg: str) -> None:
    """Name the case before any GPU work, so a failing run says which it was."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_inputs(w: workloads.Workload):
    """(q, k, v) as bf16-rounded float32 numpy (oracle side) and bf16 device tensors."""
    host = [workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w)]
    dev = [torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in host]
    return host, dev


def to_dev_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def err_stats(got: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    d = np.abs(np.asarray(got, np.float64) - ref)
    return float(d.max()), float(np.sqrt(np.mean(d ** 2)))


def rows_of(o_bshd: np.ndarray, rows: np.ndarray) -> np.ndarray:
    b, h, i = rows.T
    return o_bshd[b, i, h]


def lse_rows(lse: np.ndarray, rows: np.ndarray) -> np.ndarray:
    b, h, i = rows.T
    return lse[b, h, i]
