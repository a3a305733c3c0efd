"""The e4m3 MFMA's deviation from the exact dot product, on the device.

tests/fp8_bound.py bounds |O_gpu - O_emulation| assuming that the FP8
kernel's MFMA (e4m3 x e4m3 -> fp32, 64-wide k-steps chained in the
accumulator) returns each dot product within EPS_MFMA * sum |a_k b_k| of its
exact value.  That is not fp32 rounding of the exact sum: on gfx950 the
measured deviation reaches about 2^-15 of sum |a_k b_k|.  This test measures
it with a probe kernel (tests/probes/mfma_fp8_probe.hip, built with the
library) on e4m3 codes of the FP8 workloads' distributions and checks the
assumption.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from fp8_bound import EPS_MFMA
from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libmfma_fp8_probe.so")


@pytest.mark.parametrize("dist", ["outlier_sd10", "outlier30", "normal"])
@pytest.mark.parametrize("ks", [1, 2, 4])
def test_mfma_fp8_dot_product_deviation(dist, ks):
    say(f"mfma fp8 probe {dist} ks={ks}")
    assert os.path.exists(PROBE), f"{PROBE} missing: run __graft_entry__.build()"
    lib = ctypes.CDLL(PROBE)
    nprob, K = 128, 64 * ks
    w = workloads.Workload("mfma", 1, 1, 64 * nprob, K, False, seed=600 + ks, dist=dist)
    x = workloads.gen_qkv(w)
    a8, _ = oracle.blockquant_hadamard(x[0], workloads.gen_signs(K), 128)
    b8, _ = oracle.blockquant_hadamard(x[1], workloads.gen_signs(K), 128)
    A = np.ascontiguousarray(a8.reshape(-1, K)[: 32 * nprob].reshape(nprob, 32, K))
    BT = np.ascontiguousarray(b8.reshape(-1, K)[: 32 * nprob].reshape(nprob, 32, K))
    tA, tB = torch.from_numpy(A).to(DEV), torch.from_numpy(BT).to(DEV)
    tD = torch.empty((nprob, 32, 32), dtype=torch.float32, device=DEV)
    rc = lib.mfma_fp8_probe(ctypes.c_void_p(tA.data_ptr()), ctypes.c_void_p(tB.data_ptr()),
                            ctypes.c_void_p(tD.data_ptr()), nprob, ks)
    assert rc == 0
    D = tD.cpu().numpy().astype(np.float64)
    av, bv = oracle.e4m3_decode(A), oracle.e4m3_decode(BT)
    exact = np.einsum("prk,pck->prc", av, bv)
    mag = np.einsum("prk,pck->prc", np.abs(av), np.abs(bv))
    rel = np.abs(D - exact) / mag
    print(f"{dist} K={K}: max |D - exact| / sum|ab| = {rel.max():.3e} "
          f"(2^{np.log2(rel.max()):.1f}), median {np.median(rel):.3e}", flush=True)
    assert rel.max() <= EPS_MFMA
