#!/usr/bin/env python3
"""Benchmark of the attention forward hot path on one MI355X.

One step = the whole path over one batch of synthetic input (d=128, N=8192,
non-causal, inputs resident in HBM):
  fp8 leg, B=4 H=16 (N(0,1) with 0.1% of entries x30, seed 3):
    blockquant_hadamard(Q), (K) with the seeded sign vector, (V) without,
    then attn_fwd_fp8 on the codes;
  bf16 leg, B=2 H=16 (the N=8192 point of the 16384-token sweep, N(0,1),
    seed 2): attn_fwd_bf16.
Each launch is bracketed by HIP events on the stream it runs on; the printed
``value`` is the bf16 attention TFLOP/s (4*B*H*N^2*d per launch over its
median event time), with the fp8 figure and the pre-pass GB/s beside it.

After the timed steps, further legs are timed the same way, each on its own
launches: the bf16 gradients, the RoPE-fused pre-pass, the causal forwards,
the head-dim-256 forwards, the bf16 forward on B2 H32 N4096, the GFX clock
during the two headline forwards, the 16384-token sweep (36 configurations),
the long single request B1 H8 N32768 causal, the FP8 accuracy figures with the
2 x 2 ablation of block scales and rotation, and (unless --no-cpu-baseline)
the fp64 CPU oracle on a bounded sample of the bf16 workload.  Prints ONE
JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CALIB_COPY_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--causal", action="store_true", help="time the causal variant instead")
    p.add_argument("--N", type=int, default=8192)
    p.add_argument("--B", type=int, default=2, help="batch of the bf16 leg")
    p.add_argument("--B8", type=int, default=4, help="batch of the fp8 leg")
    p.add_argument("--H", type=int, default=16)
    p.add_argument("--d", type=int, default=128)
    p.add_argument("--bwd-reps", type=int, default=20,
                   help="timed launches of the bf16 gradients (attn_bwd_bf16) on the bf16 "
                        "workload, after the timed steps; 0 skips them")
    p.add_argument("--rope-reps", type=int, default=20,
                   help="timed launches of the RoPE-fused pre-pass on the fp8 workload's Q; 0 "
                        "skips them")
    p.add_argument("--causal-reps", type=int, default=20,
                   help="launches of the causal forwards on the same workloads (0: skip)")
    p.add_argument("--pipe-reps", type=int, default=20,
                   help="launches of attn_fwd_bf16 (pipelined) and attn_fwd_bf16_same_phase, "
                        "alternated, at the bf16 workload and B4 H16 N4096 (0: skip)")
    p.add_argument("--d256-reps", type=int, default=20,
                   help="launches of the head-dim-256 forwards, B2 H8 N8192 (0: skip)")
    p.add_argument("--c2-reps", type=int, default=20,
                   help="launches of the bf16 forward on B2 H32 N4096 d128, non-causal and causal "
                        "(0: skip)")
    p.add_argument("--sweep-reps", type=int, default=10,
                   help="launches per configuration of the 16384-token bf16 sweep (N 512..16k x "
                        "d 64/96/128 x both masks; 0: skip)")
    p.add_argument("--long-reps", type=int, default=10,
                   help="launches of the long single-request forward B1 H8 N32768 d128 causal "
                        "(0: skip)")
    p.add_argument("--sclk-seconds", type=float, default=1.0,
                   help="seconds of back-to-back launches per kernel while the GFX clock is "
                        "sampled (0: skip)")
    p.add_argument("--no-fp8-accuracy", action="store_true",
                   help="skip the FP8 accuracy / ablation figures")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one plain 256 MiB device copy (untimed), the reference that "
                        "scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    return p.parse_args()


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch (read + write) from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when that summary is for another
    workload or the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    h = hashlib.sha256()
    for src in k["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != k["sha256"]:
        return None
    return k["read_bytes"] + k["write_bytes"]


def cpu_baseline(w, target_s: float):
    """Time the fp64 CPU oracle on whole (b, h) heads of the workload until
    ``target_s`` seconds have passed; report TFLOP/s with the same flop count."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    rng = np.random.default_rng(w.seed)
    heads = 0
    el = 0.0  # oracle time only; each head's inputs are drawn before its timer starts
    while el < target_s and heads < w.B * w.H:
        q, k, v = (workloads.to_bf16_f32(rng.standard_normal((1, w.N, 1, w.d), dtype=np.float32))
                   for _ in range(3))
        t1 = time.perf_counter()
        oracle.naive_attention(q, k, v, w.softmax_scale, w.causal, row_chunk=1024)
        dt = time.perf_counter() - t1
        el += dt
        heads += 1
        if heads == 1:
            first = dt
    flops = 4.0 * heads * w.N * w.N * w.d / (2 if w.causal else 1)
    return {
        "value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{heads} of {w.B * w.H} (b,h) heads of N={w.N} d={w.d}"
                  f"{' causal' if w.causal else ''}, fp64 numpy naive attention, {el:.1f} s of "
                  f"oracle time (first head {first:.1f} s); input generation not timed",
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


WARM_SECONDS = 0.025


def time_reps(fn, reps: int, stream) -> float:
    """Median seconds of ``reps`` launches of ``fn``, each bracketed by HIP
    events on ``stream``, after untimed launches that take about
    WARM_SECONDS (at least three).  The warm-up puts the GPU in its sustained
    state for this shape: with three untimed launches only, the medians moved
    with the number of timed ones (10 vs 40 launches: 1133 vs 1225 TFLOP/s at
    B2 H16 N8192, 862 vs 746 at B32 N512, whose short bursts still ran at the
    boost clock)."""
    import numpy as np
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    per = (time.perf_counter() - t0) / 3
    for _ in range(max(0, math.ceil(WARM_SECONDS / max(per, 1e-6)) - 3)):
        fn()
    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e-3


class ClockSampler:
    """GFX (shader) clock of one GPU, sampled from amd-smi's metrics table by a
    host thread (mean of the per-XCD current clocks, about every 2 ms) while
    the main thread keeps the GPU busy."""

    def __init__(self, dev):
        import amdsmi
        import torch
        self._smi = amdsmi
        amdsmi.amdsmi_init()
        p = torch.cuda.get_device_properties(dev)
        want = (int(p.pci_domain_id), int(p.pci_bus_id), int(p.pci_device_id))
        self.handle = None
        for hnd in amdsmi.amdsmi_get_processor_handles():
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(hnd)  # "dddd:bb:dd.f"
            dom, bus, rest = bdf.split(":")
            if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                self.handle = hnd
        if self.handle is None:
            raise RuntimeError(f"no amd-smi device at PCI {want}")

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self.handle)
        xs = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
        if xs:
            return float(sum(xs)) / len(xs)
        c = m.get("current_gfxclk")
        return float(c) if isinstance(c, (int, float)) else None

    def measure(self, fn, seconds: float, stream):
        """Mean MHz and sample count while ``fn`` is launched back to back for
        about ``seconds`` (the first 20% of the samples, while the clock
        settles, are dropped)."""
        import threading
        import torch
        samples, stop = [], threading.Event()

        def poll():
            while not stop.is_set():
                v = self._read()
                if v is not None:
                    samples.append(v)
                time.sleep(0.002)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        th = threading.Thread(target=poll, daemon=True)
        th.start()
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                fn()
            n += 10
            stream.synchronize()
        stop.set()
        th.join()
        kept = samples[len(samples) // 5:]
        return (float(np.mean(kept)) if kept else None), len(kept), n


def fp64_rows_reference(q, k, v, b, h, rows, scale):
    """Exact softmax attention (fp64, on the device) of the query rows ``rows``
    of head (b, h); q, k, v bf16 BSHD device tensors.  Used for the accuracy
    figures of the bench, which do not load the CPU oracle."""
    import torch
    idx = torch.as_tensor(rows, device=q.device)
    qr = q[b, idx, h].double()
    kh, vh = k[b, :, h].double().contiguous(), v[b, :, h].double().contiguous()
    s = (qr @ kh.T) * scale
    p = torch.softmax(s, dim=1)
    return p @ vh


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (attention "
              "heads are independent, so several GPUs would each take a share of the heads, "
              "with no communication).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_74_amd as ea
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sfx = "_causal" if a.causal else ""
    w16 = workloads.Workload(f"attn_fwd_b{a.B}h{a.H}n{a.N}d{a.d}{sfx}", a.B, a.H, a.N, a.d,
                             a.causal, seed=2)
    w8 = workloads.Workload(f"attn_fwd_b{a.B8}h{a.H}n{a.N}d{a.d}{sfx}_fp8_outlier30", a.B8, a.H,
                            a.N, a.d, a.causal, seed=3, dist="outlier30")

    def dev_bf16(x):
        return torch.from_numpy(x).to(torch.bfloat16).to(dev)

    q, k, v = (dev_bf16(x) for x in workloads.gen_qkv(w16))
    q8in, k8in, v8in = (dev_bf16(x) for x in workloads.gen_qkv(w8))
    signs = torch.from_numpy(workloads.gen_signs(a.d)).to(dev)
    B, B8, H, N, d = a.B, a.B8, a.H, a.N, a.d
    nsb = (N + 127) // 128
    o16 = torch.empty_like(q)
    lse16 = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    o8 = torch.empty_like(q8in)
    lse8 = torch.empty((B8, H, N), dtype=torch.float32, device=dev)
    codes = [torch.empty((B8, N, H, d), dtype=torch.uint8, device=dev) for _ in range(3)]
    scales = [torch.empty((B8, H, nsb), dtype=torch.float32, device=dev) for _ in range(3)]
    scale = w16.softmax_scale
    stream = torch.cuda.current_stream(dev)

    names = ["blockquant_q", "blockquant_k", "blockquant_v", "attn_fwd_fp8", "attn_fwd_bf16"]

    def step(evs=None):
        calls = [
            lambda: ea.blockquant_hadamard(q8in, signs, 128, out=codes[0], scale=scales[0]),
            lambda: ea.blockquant_hadamard(k8in, signs, 128, out=codes[1], scale=scales[1]),
            lambda: ea.blockquant_hadamard(v8in, None, 128, out=codes[2], scale=scales[2]),
            lambda: ea.attn_fwd_fp8(codes[0], codes[1], codes[2], *scales, causal=a.causal,
                                    softmax_scale=scale, out=o8, lse=lse8),
            lambda: ea.attn_fwd_bf16(q, k, v, causal=a.causal, softmax_scale=scale, out=o16,
                                     lse=lse16),
        ]
        for i, c in enumerate(calls):
            if evs is not None:
                evs[i][0].record(stream)
            c()
            if evs is not None:
                evs[i][1].record(stream)

    if a.calib_copy:
        src = torch.empty(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    print(f"[bench] workload {w16.name}: warmup {a.warmup}", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in names] for _ in range(a.steps)]
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {n: [events[s][i][0].elapsed_time(events[s][i][1]) for s in range(a.steps)]
           for i, n in enumerate(names)}
    mean = {n: float(np.mean(v)) for n, v in per.items()}
    med = {n: float(np.median(v)) for n, v in per.items()}

    t16 = med["attn_fwd_bf16"] * 1e-3
    t8 = med["attn_fwd_fp8"] * 1e-3
    tf16 = w16.flops() / t16 / 1e12
    tf8 = w8.flops() / t8 / 1e12
    tf16_best = w16.flops() / (min(per["attn_fwd_bf16"]) * 1e-3) / 1e12
    tf8_best = w8.flops() / (min(per["attn_fwd_fp8"]) * 1e-3) / 1e12
    # pre-pass algorithmic bytes per tensor: read bf16, write e4m3, write fp32 scales
    bq_bytes = B8 * N * H * d * (2 + 1) + B8 * H * nsb * 4
    t_bq = np.median([med["blockquant_q"], med["blockquant_k"], med["blockquant_v"]]) * 1e-3
    ok = bool(torch.isfinite(o16).all().item() and torch.isfinite(o8).all().item())

    out = {
        "metric": "attention fwd TFLOP/s (bf16 & fp8, d=128, N=8k) + % of MFMA peak",
        "value": round(tf16, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(wall / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16; fp8 leg: N(0,1) with 0.1% entries x30)",
        "config": {"workload": w16.name, "B": B, "H": H, "N": N, "d": d, "causal": a.causal,
                   "softmax_scale": scale, "global_batch": B, "seq_len": N,
                   "parallelism": "single GPU (heads and query blocks across CUs)"},
        "timing": "median of the per-launch HIP event times over the timed steps",
        "pct_of_peak": round(100 * tf16 / PEAK_BF16_TFLOPS, 2),
        "best": {"attn_fwd_bf16": round(tf16_best, 2), "attn_fwd_fp8": round(tf8_best, 2)},
        "fp8": {"value": round(tf8, 2), "unit": "TFLOP/s", "dtype": "fp8 e4m3",
                "pct_of_peak": round(100 * tf8 / PEAK_FP8_TFLOPS, 2),
                "workload": w8.name, "B": B8, "ms": round(med["attn_fwd_fp8"], 4)},
        "blockquant_hadamard": {"gbps": round(bq_bytes / t_bq / 1e9, 1),
                                "pct_of_hbm_peak": round(100 * bq_bytes / t_bq / 1e9 / PEAK_HBM_GBS, 2),
                                "bytes_per_launch": bq_bytes, "us": round(t_bq * 1e6, 2)},
        "kernel_ms_mean": {n: round(v, 4) for n, v in mean.items()},
        "kernel_ms_median": {n: round(v, 4) for n, v in med.items()},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_bf16", "achieved": round(tf16, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf16 / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic("attn_fwd_bf16", f"attn_fwd_b{B}h{H}n{N}d{d}"
                                                 if not a.causal else "none"),
                     "algorithmic_flops_per_launch": w16.flops()},
        "outputs_finite": ok,
    }
    if a.bwd_reps > 0:
        # Gradients of the bf16 forward (not part of the forward step above):
        # dO seeded N(0,1), O and LSE from the last timed step.
        print(f"[bench] backward: {a.bwd_reps} launches", file=sys.stderr, flush=True)
        do = dev_bf16(workloads.gen_random((B, N, H, d), 1002))
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = torch.empty(max(1, ea.lib().attn_bwd_bf16_workspace_bytes(B, H, N) // 4),
                         dtype=torch.float32, device=dev)

        def bwd():
            ea.attn_bwd_bf16(q, k, v, o16, lse16, do, causal=a.causal, softmax_scale=scale,
                             dq=dq, dk=dk, dv=dv, workspace=ws)
        t_bwd = time_reps(bwd, a.bwd_reps, stream)
        bname = w16.name.replace("attn_fwd", "attn_bwd")
        bflops = 2.5 * w16.flops()  # five N^2 d products against the forward's two
        out["backward"] = {
            "kernel": "attn_bwd_bf16 (prep + dK/dV + dQ kernels)", "workload": bname,
            "value": round(bflops / t_bwd / 1e12, 2), "unit": "TFLOP/s",
            "flops_counted": "2.5 x forward (10 B H N^2 d, halved for causal)",
            "pct_of_peak": round(100 * bflops / t_bwd / 1e12 / PEAK_BF16_TFLOPS, 2),
            "ms": round(t_bwd * 1e3, 4), "reps": a.bwd_reps,
            "timing": "median of per-call HIP event times",
            "finite": bool(all(torch.isfinite(x).all().item() for x in (dq, dk, dv)))}
        # The other mask on the same inputs, and head dim 64 (H doubled, the
        # 16384-token sweep's d = 64 shape): the kernels' other instances.
        variants = {}
        print("[bench] backward variants: other mask, d = 64", file=sys.stderr, flush=True)
        o_c, lse_c = ea.attn_fwd_bf16(q, k, v, causal=not a.causal, softmax_scale=scale)

        def bwd_c():
            ea.attn_bwd_bf16(q, k, v, o_c, lse_c, do, causal=not a.causal, softmax_scale=scale,
                             dq=dq, dk=dk, dv=dv, workspace=ws)
        t_c = time_reps(bwd_c, a.bwd_reps, stream)
        fl_c = 2.5 * dataclasses.replace(w16, causal=not a.causal).flops()
        variants["causal" if not a.causal else "non_causal"] = {
            "workload": bname + ("_causal" if not a.causal else "_noncausal"),
            "value": round(fl_c / t_c / 1e12, 2), "ms": round(t_c * 1e3, 4)}
        del o_c, lse_c
        if d == 128:
            w64 = workloads.Workload(f"attn_bwd_b{B}h{2 * H}n{N}d64{sfx}", B, 2 * H, N, 64, a.causal,
                                     seed=2)
            q6, k6, v6 = (dev_bf16(x) for x in workloads.gen_qkv(w64))
            do6 = dev_bf16(workloads.gen_random((B, N, 2 * H, 64), 1003))
            o6, lse6 = ea.attn_fwd_bf16(q6, k6, v6, causal=a.causal, softmax_scale=w64.softmax_scale)
            g6 = [torch.empty_like(q6) for _ in range(3)]

            def bwd_64():
                ea.attn_bwd_bf16(q6, k6, v6, o6, lse6, do6, causal=a.causal,
                                 softmax_scale=w64.softmax_scale, dq=g6[0], dk=g6[1], dv=g6[2])
            t_64 = time_reps(bwd_64, a.bwd_reps, stream)
            variants["d64"] = {"workload": w64.name, "value": round(2.5 * w64.flops() / t_64 / 1e12, 2),
                               "ms": round(t_64 * 1e3, 4),
                               "finite": bool(all(torch.isfinite(x).all().item() for x in g6))}
            del q6, k6, v6, do6, o6, lse6, g6
        out["backward"]["variants"] = variants
    if a.rope_reps > 0:
        # The pre-pass fused with a rotary embedding (half-split pairs), on the
        # fp8 workload's Q; algorithmic bytes add the cos/sin tables, read once.
        print(f"[bench] rope pre-pass: {a.rope_reps} launches", file=sys.stderr, flush=True)
        rc, rsn = (torch.from_numpy(x).to(dev) for x in workloads.rope_tables(N, d))

        def rq():
            ea.rope_blockquant_hadamard(q8in, rc, rsn, False, signs, 128, out=codes[0],
                                        scale=scales[0])
        t_rq = time_reps(rq, a.rope_reps, stream)
        rq_bytes = bq_bytes + 2 * N * (d // 2) * 4
        out["rope_blockquant_hadamard"] = {
            "workload": f"{w8.name} (Q), half-split RoPE", "gbps": round(rq_bytes / t_rq / 1e9, 1),
            "pct_of_hbm_peak": round(100 * rq_bytes / t_rq / 1e9 / PEAK_HBM_GBS, 2),
            "bytes_per_launch": rq_bytes, "us": round(t_rq * 1e6, 2),
            "vs_plain_prepass_us": round(t_bq * 1e6, 2)}
    if a.causal_reps > 0 and not a.causal:
        # The same two workloads with the causal mask (visible key pairs only:
        # 2 B H N^2 d flop); causal work at d <= 128 runs on persistent slots
        # over equal-cost pairs of query blocks.
        print(f"[bench] causal forwards: {a.causal_reps} launches each", file=sys.stderr,
              flush=True)
        t_c16 = time_reps(lambda: ea.attn_fwd_bf16(q, k, v, causal=True, softmax_scale=scale,
                                                   out=o16, lse=lse16), a.causal_reps, stream)
        t_c8 = time_reps(lambda: ea.attn_fwd_fp8(codes[0], codes[1], codes[2], *scales,
                                                 causal=True, softmax_scale=scale, out=o8,
                                                 lse=lse8), a.causal_reps, stream)
        f16, f8 = w16.flops() / 2, w8.flops() / 2
        out["causal"] = {
            "flops_counted": "2 B H N^2 d (visible pairs)", "timing": "median of per-call HIP event times",
            "attn_fwd_bf16": {"workload": w16.name + "_causal", "value": round(f16 / t_c16 / 1e12, 2),
                              "pct_of_peak": round(100 * f16 / t_c16 / 1e12 / PEAK_BF16_TFLOPS, 2),
                              "ms": round(t_c16 * 1e3, 4)},
            "attn_fwd_fp8": {"workload": w8.name + "_causal", "value": round(f8 / t_c8 / 1e12, 2),
                             "pct_of_peak": round(100 * f8 / t_c8 / 1e12 / PEAK_FP8_TFLOPS, 2),
                             "ms": round(t_c8 * 1e3, 4)},
            "finite": bool(torch.isfinite(o16).all().item() and torch.isfinite(o8).all().item())}
    if a.pipe_reps > 0 and not a.causal and a.d == 128:
        # The two schedules of the bf16 forward on the same inputs, alternated
        # twice: attn_fwd_bf16 (the intra-wave pipelined loop at d = 128
        # non-causal) against attn_fwd_bf16_same_phase.  They must agree bit
        # for bit.
        print(f"[bench] schedules: {a.pipe_reps} launches x 2 rounds", file=sys.stderr,
              flush=True)
        legs = {}
        for name, (Bp, Np) in (("headline", (B, N)), ("b4n4096", (4, 4096))):
            if (Bp, Np) == (B, N):
                qp, kp, vp, wp = q, k, v, w16
            else:
                wp = workloads.Workload(f"attn_fwd_b{Bp}h{H}n{Np}d{d}", Bp, H, Np, d, False, seed=2)
                qp, kp, vp = (dev_bf16(x) for x in workloads.gen_qkv(wp))
            op, lp = torch.empty_like(qp), torch.empty((Bp, H, Np), dtype=torch.float32, device=dev)
            op2, lp2 = torch.empty_like(op), torch.empty_like(lp)
            piped = lambda: ea.attn_fwd_bf16(qp, kp, vp, softmax_scale=scale, out=op, lse=lp)
            same = lambda: ea.attn_fwd_bf16_same_phase(qp, kp, vp, softmax_scale=scale, out=op2,
                                                       lse=lp2)
            tp, ts = [], []
            for _ in range(2):
                tp.append(time_reps(piped, a.pipe_reps, stream))
                ts.append(time_reps(same, a.pipe_reps, stream))
            f = wp.flops()
            legs[name] = {"workload": wp.name,
                          "pipelined": round(f / min(tp) / 1e12, 2),
                          "same_phase": round(f / min(ts) / 1e12, 2),
                          "bit_identical": bool(torch.equal(op, op2) and torch.equal(lp, lp2))}
        out["schedules"] = {"kernels": "attn_fwd_bf16 (pipelined) vs attn_fwd_bf16_same_phase",
                            "unit": "TFLOP/s",
                            "timing": "best of two medians of per-call HIP event times, alternated",
                            **legs}
    if a.d256_reps > 0:
        # Head dim 256 (the report's best FP8 case), B2 H8 N8192: the 2048-wide
        # model at d = 256.  FP8 codes from the pre-pass (untimed here).
        print(f"[bench] d=256 forwards: {a.d256_reps} launches each", file=sys.stderr, flush=True)
        w256 = workloads.Workload("attn_fwd_b2h8n8192d256_outlier30", 2, 8, 8192, 256, False,
                                  seed=4, dist="outlier30")
        x256 = [dev_bf16(x) for x in workloads.gen_qkv(w256)]
        s256 = torch.from_numpy(workloads.gen_signs(256)).to(dev)
        q2, sq2 = ea.blockquant_hadamard(x256[0], s256, 128)
        k2, sk2 = ea.blockquant_hadamard(x256[1], s256, 128)
        v2, sv2 = ea.blockquant_hadamard(x256[2], None, 128)
        o2 = torch.empty_like(x256[0])
        l2 = torch.empty((2, 8, 8192), dtype=torch.float32, device=dev)
        sc2 = w256.softmax_scale
        t_a16 = time_reps(lambda: ea.attn_fwd_bf16(*x256, softmax_scale=sc2, out=o2, lse=l2),
                          a.d256_reps, stream)
        t_a8 = time_reps(lambda: ea.attn_fwd_fp8(q2, k2, v2, sq2, sk2, sv2, softmax_scale=sc2,
                                                 out=o2, lse=l2), a.d256_reps, stream)
        f = w256.flops()
        out["d256"] = {
            "workload": w256.name, "timing": "median of per-call HIP event times",
            "attn_fwd_fp8": {"value": round(f / t_a8 / 1e12, 2),
                             "pct_of_peak": round(100 * f / t_a8 / 1e12 / PEAK_FP8_TFLOPS, 2),
                             "ms": round(t_a8 * 1e3, 4)},
            "attn_fwd_bf16": {"value": round(f / t_a16 / 1e12, 2),
                              "pct_of_peak": round(100 * f / t_a16 / 1e12 / PEAK_BF16_TFLOPS, 2),
                              "ms": round(t_a16 * 1e3, 4)},
            "finite": bool(torch.isfinite(o2).all().item())}
        del x256, q2, k2, v2, o2, l2
    if a.c2_reps > 0 and a.d == 128:
        # The bf16 workload B2 H32 N4096 d128 (N(0,1), seed 1), both masks.
        print(f"[bench] B2 H32 N4096 forwards: {a.c2_reps} launches each", file=sys.stderr,
              flush=True)
        wc2 = workloads.Workload("attn_fwd_b2h32n4096d128", 2, 32, 4096, 128, False, seed=1)
        xc2 = [dev_bf16(x) for x in workloads.gen_qkv(wc2)]
        oc2 = torch.empty_like(xc2[0])
        lc2 = torch.empty((2, 32, 4096), dtype=torch.float32, device=dev)
        res = {"workload": wc2.name, "timing": "median of per-call HIP event times"}
        for causal in (False, True):
            t = time_reps(lambda: ea.attn_fwd_bf16(*xc2, causal=causal,
                                                   softmax_scale=wc2.softmax_scale, out=oc2,
                                                   lse=lc2), a.c2_reps, stream)
            f = wc2.flops() / (2 if causal else 1)
            res["causal" if causal else "non_causal"] = {
                "value": round(f / t / 1e12, 2),
                "pct_of_peak": round(100 * f / t / 1e12 / PEAK_BF16_TFLOPS, 2),
                "ms": round(t * 1e3, 4)}
        res["finite"] = bool(torch.isfinite(oc2).all().item())
        out["b2h32n4096"] = res
        del xc2, oc2, lc2
    if a.sclk_seconds > 0:
        # GFX clock while each headline kernel runs back to back: the fraction
        # of the published peak (quoted at 2.4 GHz) that the achieved rate
        # reaches at the clock the chip actually ran at.
        print("[bench] gfx clock during the bf16 and fp8 forwards", file=sys.stderr, flush=True)
        try:
            cs = ClockSampler(dev)
            res = {"source": "amd-smi gpu_metrics current_gfxclks (mean over the XCDs), sampled "
                             "every ~2 ms by a host thread during back-to-back launches",
                   "peak_clock_mhz": 2400.0}
            for name, fn, tf, peak in (
                    ("attn_fwd_bf16", lambda: ea.attn_fwd_bf16(q, k, v, causal=a.causal,
                                                               softmax_scale=scale, out=o16,
                                                               lse=lse16), tf16, PEAK_BF16_TFLOPS),
                    ("attn_fwd_fp8", lambda: ea.attn_fwd_fp8(codes[0], codes[1], codes[2],
                                                             *scales, causal=a.causal,
                                                             softmax_scale=scale, out=o8,
                                                             lse=lse8), tf8, PEAK_FP8_TFLOPS)):
                mhz, n, launches = cs.measure(fn, a.sclk_seconds, stream)
                res[name] = {"mhz": None if mhz is None else round(mhz, 1), "samples": n,
                             "launches": launches,
                             "frac_of_peak_at_this_clock": None if not mhz else
                             round(tf / (peak * mhz / 2400.0), 4)}
            out["sclk"] = res
        except Exception as e:  # the clock is context; the bench goes on without it
            out["sclk"] = {"error": f"{type(e).__name__}: {e}"}
    if a.sweep_reps > 0 and a.d == 128:
        # The 16384-token sweep: N 512..16k, B = 16384 / N; d 128 (H16), d 64
        # (H32) and d 96 zero-padded to 128 (H16, credited with d = 96 work);
        # both masks; seeded N(0,1) inputs.
        print(f"[bench] 16384-token sweep: {a.sweep_reps} launches per configuration",
              file=sys.stderr, flush=True)
        rows = []
        for wnc in workloads.sweep(False):
            x = [dev_bf16(t) for t in workloads.gen_qkv(wnc)]
            ox = torch.empty_like(x[0])
            lx = torch.empty((wnc.B, wnc.H, wnc.N), dtype=torch.float32, device=dev)
            for causal in (False, True):
                wc = workloads.Workload(wnc.name.replace("_nc", "_c") if causal else wnc.name,
                                        wnc.B, wnc.H, wnc.N, wnc.d, causal, wnc.seed,
                                        d_logical=wnc.d_logical)
                t = time_reps(lambda: ea.attn_fwd_bf16(*x, causal=causal,
                                                       softmax_scale=wc.softmax_scale, out=ox,
                                                       lse=lx), a.sweep_reps, stream)
                tf = wc.flops() / t / 1e12
                rows.append({"workload": wc.name, "B": wc.B, "H": wc.H, "N": wc.N, "d": wc.d,
                             "d_counted": wc.d_logical or wc.d, "causal": causal,
                             "value": round(tf, 2),
                             "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                             "ms": round(t * 1e3, 4),
                             "finite": bool(torch.isfinite(ox).all().item())})
            del x, ox, lx
        out["sweep"] = {"kernel": "attn_fwd_bf16", "unit": "TFLOP/s",
                        "flops_counted": "4 B H N^2 d (d = 96 for the padded runs), halved for "
                                         "causal", "timing": "median of per-call HIP event times",
                        "configs": rows}
    if a.long_reps > 0:
        # Long single request: B1 H8 N32768 d128 causal (seed 5), bf16, and the
        # same inputs through the FP8 path (pre-pass untimed).
        print(f"[bench] long request B1 H8 N32768 causal: {a.long_reps} launches",
              file=sys.stderr, flush=True)
        wl = workloads.LONG
        xl = [dev_bf16(t) for t in workloads.gen_qkv(wl)]
        ol = torch.empty_like(xl[0])
        ll = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device=dev)
        t = time_reps(lambda: ea.attn_fwd_bf16(*xl, causal=True, softmax_scale=wl.softmax_scale,
                                               out=ol, lse=ll), a.long_reps, stream)
        c8 = [ea.blockquant_hadamard(xl[0], signs, 128), ea.blockquant_hadamard(xl[1], signs, 128),
              ea.blockquant_hadamard(xl[2], None, 128)]
        t8l = time_reps(lambda: ea.attn_fwd_fp8(c8[0][0], c8[1][0], c8[2][0], c8[0][1], c8[1][1],
                                                c8[2][1], causal=True,
                                                softmax_scale=wl.softmax_scale, out=ol, lse=ll),
                        a.long_reps, stream)
        f = wl.flops()
        out["long_c5"] = {
            "workload": wl.name, "flops_counted": "2 B H N^2 d (visible pairs)",
            "timing": "median of per-call HIP event times",
            "attn_fwd_bf16": {"value": round(f / t / 1e12, 2),
                              "pct_of_peak": round(100 * f / t / 1e12 / PEAK_BF16_TFLOPS, 2),
                              "ms": round(t * 1e3, 4)},
            "attn_fwd_fp8": {"value": round(f / t8l / 1e12, 2),
                             "pct_of_peak": round(100 * f / t8l / 1e12 / PEAK_FP8_TFLOPS, 2),
                             "ms": round(t8l * 1e3, 4)},
            "finite": bool(torch.isfinite(ol).all().item())}
        del xl, ol, ll, c8
    if not a.no_fp8_accuracy and a.d == 128 and a.N == 8192 and a.B8 == 4 and a.H == 16:
        # FP8 accuracy on both outlier distributions: the GPU path (pre-pass +
        # forward) against an fp64 evaluation of exact attention on 512 sampled
        # rows, for block vs per-tensor scales x rotation vs none; beside it the
        # oracle's emulation floor of each case (stored by
        # tests/golden/make_fp8_emulation_floor.py on the same rows).
        print("[bench] fp8 accuracy and ablation", file=sys.stderr, flush=True)
        floor_path = os.path.join(ROOT, "tests", "golden", "fp8_emulation_floor.json")
        floors = json.load(open(floor_path)) if os.path.exists(floor_path) else {}
        acc = {"reference": "fp64 exact attention of the bf16 inputs on the device, 4 heads x "
                            "128 sampled rows", "workload": "B4 H16 N8192 d128 non-causal"}
        for key, wa in (("fp8_outlier30", w8),
                        ("fp8_page_outlier_sd10", workloads.Workload(
                            "fp8_page", B8, H, N, d, False, seed=3, dist="outlier_sd10"))):
            xa = [q8in, k8in, v8in] if wa is w8 else [dev_bf16(t) for t in workloads.gen_qkv(wa)]
            sel = workloads.fp8_accuracy_rows(N)
            ref = torch.cat([fp64_rows_reference(*xa, b, h, r, scale) for b, h, r in sel])
            res = {"rms_exact": round(float(ref.pow(2).mean().sqrt()), 6)}
            for br, rot in ((128, True), (128, False), (0, True), (0, False)):
                sg = signs if rot else None
                cq = [ea.blockquant_hadamard(xa[0], sg, br), ea.blockquant_hadamard(xa[1], sg, br),
                      ea.blockquant_hadamard(xa[2], None, br)]
                oa, _ = ea.attn_fwd_fp8(cq[0][0], cq[1][0], cq[2][0], cq[0][1], cq[1][1], cq[2][1],
                                        softmax_scale=scale)
                got = torch.cat([oa[b, torch.as_tensor(r, device=dev), h].double()
                                 for b, h, r in sel])
                name = f"{'block' if br else 'per_tensor'}_{'rotation' if rot else 'no_rotation'}"
                res[name] = {"rmse": round(float((got - ref).pow(2).mean().sqrt()), 6),
                             "emulation_floor": floors.get(key, {}).get(name)}
            res["ratio_per_tensor_no_rotation_to_block_rotation"] = round(
                res["per_tensor_no_rotation"]["rmse"] / res["block_rotation"]["rmse"], 3)
            acc[key] = res
            del xa
        out["fp8_accuracy"] = acc
    if not a.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w16, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
