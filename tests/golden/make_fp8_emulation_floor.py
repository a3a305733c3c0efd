"""Writes fp8_emulation_floor.json: the RMSE against exact attention of the
oracle's FP8 emulation on the FP8 workload (B4 H16 N8192 d128) and on the
report's outlier distribution, for the four combinations of block vs
per-tensor scales and Hadamard rotation vs none, on the sampled rows of
workloads.fp8_accuracy_rows.  Calls only the oracle and the seeded generators.

Usage: python tests/golden/make_fp8_emulation_floor.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def floors(w):
    q, k, v = (workloads.to_bf16_f32(x) for x in workloads.gen_qkv(w))
    signs = workloads.gen_signs(w.d)
    out = {}
    for br, rot in ((128, True), (128, False), (0, True), (0, False)):
        sg = signs if rot else None
        if br == 0:  # one scale over the whole tensor, as the pre-pass in per-tensor mode
            full = [oracle.blockquant_hadamard(x, s, 0) for x, s in ((q, sg), (k, sg), (v, None))]
        em, ex = [], []
        for b, h, rows in workloads.fp8_accuracy_rows(w.N):
            sl = [x[b:b + 1, :, h:h + 1] for x in (q, k, v)]
            r3 = np.stack([np.zeros_like(rows), np.zeros_like(rows), rows], axis=1)
            if br == 0:
                codes = [c[b:b + 1, :, h:h + 1] for c, _ in full]
                scales = [sc[b:b + 1, h:h + 1] for _, sc in full]
            else:
                qz = [oracle.blockquant_hadamard(x, s, 128)
                      for x, s in ((sl[0], sg), (sl[1], sg), (sl[2], None))]
                codes = [c for c, _ in qz]
                scales = [sc for _, sc in qz]
            o, _ = oracle.fp8_attention_emulation(*codes, *scales, w.softmax_scale, False, rows=r3)
            o_ex, _ = oracle.naive_attention_rows(*sl, w.softmax_scale, False, r3)
            em.append(o)
            ex.append(o_ex)
        em, ex = np.concatenate(em), np.concatenate(ex)
        key = f"{'block' if br else 'per_tensor'}_{'rotation' if rot else 'no_rotation'}"
        out[key] = float(np.sqrt(np.mean((em - ex) ** 2)))
        print(w.name, key, out[key], flush=True)
    out["rms_exact"] = float(np.sqrt(np.mean(ex ** 2)))
    return out


if __name__ == "__main__":
    res = {"workload": "B4 H16 N8192 d128 non-causal; 128 sampled query rows in each of the "
                       "(b, h) heads of workloads.FP8_ACCURACY_HEADS (seed 77 + h)",
           "metric": "RMSE of the FP8 emulation's O against fp64 exact attention",
           "fp8_outlier30": floors(workloads.FP8),
           "fp8_page_outlier_sd10": floors(workloads.FP8_PAGE)}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_emulation_floor.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))
