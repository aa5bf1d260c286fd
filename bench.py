#!/usr/bin/env python3
"""Benchmark of the quantized mul_mat hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--no-prefill]

A step is one pass of the hot path over one batch: quantize the fp32
activations to int8 blocks (quantize_row_q8) and multiply them with the packed
4-bit weights (mul_mat), for every projection of the workload.  The weights are
encoded and repacked once before timing (load time).  Steps rotate over copies
of the weights whose total exceeds twice the 256 MB Infinity Cache, so the
weight stream really comes from HBM.  The K timed steps are captured once in a
HIP graph and replayed, so host-side launch cost is not part of the time.

Printed: one JSON line with the headline metric (Q4_K GEMV weight GB/s of the
chosen workload), the roofline of its dominant kernel, the CPU oracle baseline
and the prefill GEMM (int8 MFMA) throughput.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
MALL_BYTES = 256 << 20
METRIC = "Q4_K GEMV weight GB/s (% HBM peak); prefill GEMM int8 TOPS (% MFMA peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--layout", default="repacked", choices=["repacked", "canonical"])
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--all", action="store_true", help="report every workload")
    ap.add_argument("--prefill-only", action="store_true", help="measure only the prefill GEMM")
    return ap.parse_args()


class Prepared:
    """One workload on the GPU: weight copies, activations, outputs."""

    def __init__(self, key: str, layout: str, min_bytes: int):
        import torch
        import bit_quantized_mat_quantize_amd as qmm
        from bit_quantized_mat_quantize_amd.inputs import workload

        self.wl = workload(key)
        self.layout = layout
        dev = torch.device("cuda:0")
        self.projs = []
        acts = {}
        wbytes = self.wl.weight_bytes
        self.copies = max(1, -(-min_bytes // wbytes))
        for p in self.wl.projections:
            afmt = "q8_K" if p.wfmt == "q4_K" else "q8_0"
            wf = torch.from_numpy(p.weights()).to(dev)
            canon = qmm.quantize_weights(wf, p.wfmt)
            del wf
            w0 = qmm.repack_weights(canon, p.wfmt, p.N, p.K) if layout == "repacked" else canon
            ws = [w0] + [w0.clone() for _ in range(self.copies - 1)]
            key_a = p.act_key or p.name
            if key_a not in acts:
                x = torch.from_numpy(p.acts()).to(dev)
                y = torch.empty(qmm.act_bytes(afmt, p.M, p.K), dtype=torch.uint8, device=dev)
                acts[key_a] = (x, y, afmt, True)
            else:
                x, y, afmt, _ = acts[key_a]
                acts[key_a] = (x, y, afmt, True)
            out = torch.empty((p.M, p.N), dtype=torch.float32, device=dev)
            self.projs.append(dict(p=p, ws=ws, x=x, y=y, afmt=afmt, out=out, act=key_a))
        self.acts = acts
        torch.cuda.synchronize()

    def step(self, i: int, only: str | None = None):
        """Enqueue one step on the current stream (copy i mod copies)."""
        import bit_quantized_mat_quantize_amd as qmm
        done = set()
        for d in self.projs:
            p = d["p"]
            if only in (None, "quantize") and d["act"] not in done:
                qmm.quantize_row_q8(d["x"], d["afmt"], out=d["y"])
                done.add(d["act"])
            if only in (None, "mul_mat"):
                w = d["ws"][i % self.copies]
                if p.wfmt == "q4_K":
                    qmm.mul_mat_q4_K(w, d["y"], p.M, p.N, p.K, layout=self.layout, out=d["out"])
                else:
                    qmm.mul_mat_q4_0(w, d["y"], p.M, p.N, p.K, layout=self.layout, out=d["out"])


def time_graph(prep: Prepared, steps: int, only=None, reps: int = 1):
    """Capture `steps` steps in one HIP graph, replay it, return ms per step."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):                  # warm the kernels on the capture stream
            prep.step(i, only)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(steps):
            prep.step(i, only)
    g.replay()                               # untimed replay
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        best = ms if best is None else min(best, ms)
    del g
    return best


def cpu_baseline(key: str, seconds: float):
    """The oracle's integer path on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    from bit_quantized_mat_quantize_amd.inputs import workload

    wl = workload(key)
    p = max(wl.projections, key=lambda q: q.N * q.K)
    M_s = min(p.M, 2)
    w = oracle.quantize(p.wfmt, p.weights())
    afmt = "q8_K" if p.wfmt == "q4_K" else "q8_0"
    y = oracle.quantize(afmt, p.acts()[:M_s])
    threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.mul_mat(p.wfmt, w, y, M_s, p.N, p.K, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / reps
    wbytes = p.N * p.K * (144 / 256 if p.wfmt == "q4_K" else 18 / 32)
    if p.M <= 8:
        val, unit = wbytes / per / 1e9, "GB/s"
        sample = (f"{p.name} projection of {key} (M={M_s}, N={p.N}, K={p.K}), integer path, "
                  f"{reps} repetitions in {el:.1f} s")
    else:
        val, unit = 2 * M_s * p.N * p.K / per / 1e12, "TOPS"
        sample = (f"{M_s} of the {p.M} activation rows of {key} (N={p.N}, K={p.K}), "
                  f"integer path, {reps} repetitions in {el:.1f} s")
    return {"value": round(val, 4), "unit": unit, "cores": min(threads, oracle.max_threads()),
            "kind": "oracle", "sample": sample}


def measure_decode(key: str, layout: str, steps: int, warmup: int):
    import torch
    prep = Prepared(key, layout, min_bytes=2 * MALL_BYTES)
    for i in range(warmup):
        prep.step(i)
    torch.cuda.synchronize()
    ms_step = time_graph(prep, steps)
    ms_mm = time_graph(prep, steps, only="mul_mat")
    ms_q = time_graph(prep, steps, only="quantize")
    wbytes = prep.wl.weight_bytes
    nlaunch = len(prep.projs)
    per_launch_bytes = wbytes / nlaunch
    per_launch_ms = ms_mm / nlaunch
    achieved = per_launch_bytes / (per_launch_ms * 1e-3) / 1e9
    res = dict(
        key=key, description=prep.wl.description, weight_bytes=wbytes, copies=prep.copies,
        ms_per_step=ms_step, value=wbytes / (ms_step * 1e-3) / 1e9,
        mul_mat_us=ms_mm * 1e3, quantize_us=ms_q * 1e3,
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    )
    del prep
    torch.cuda.empty_cache()
    return res


def measure_prefill(key: str, layout: str, steps: int):
    import torch
    prep = Prepared(key, layout, min_bytes=0)
    p = prep.projs[0]["p"]
    ms_mm = time_graph(prep, steps, only="mul_mat", reps=3)
    ms_q = time_graph(prep, steps, only="quantize", reps=3)
    ops = 2 * p.M * p.N * p.K
    tops = ops / (ms_mm * 1e-3) / 1e12
    res = dict(key=key, description=prep.wl.description, gemm_us=ms_mm * 1e3,
               quantize_us=ms_q * 1e3, tops=round(tops, 1),
               frac_int8_peak=round(tops / INT8_PEAK_TOPS, 4))
    del prep
    torch.cuda.empty_cache()
    return res


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {a.gpus} is not supported "
              "(the multi-GPU sharding is described in the design notes only)", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_quantized_mat_quantize_amd as qmm
    qmm.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if a.prefill_only:
        res = {k: measure_prefill(k, a.layout, a.prefill_steps) for k in ("c5_m512", "c5_m2048")}
        print(json.dumps({"prefill": res}), flush=True)
        return
    head = measure_decode(a.workload, a.layout, a.steps, a.warmup)
    extra = {}
    if a.all:
        for k in ("c1", "c2", "c3", "c4_m4", "c4_m8", "c4_m32"):
            if k != a.workload:
                r = measure_decode(k, a.layout, a.steps, a.warmup)
                extra[k] = {x: (round(v, 3) if isinstance(v, float) else v) for x, v in r.items()}
    prefill = {}
    if not a.no_prefill:
        for k in ("c5_m512", "c5_m2048"):
            prefill[k] = measure_prefill(k, a.layout, a.prefill_steps)
    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(a.workload, a.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(head["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{head['key']}: {head['description']}",
                   "weight_layout": a.layout, "weight_bytes": head["weight_bytes"],
                   "weight_copies_rotated": head["copies"],
                   "step": "quantize_row_q8 + mul_mat per projection, HIP graph replay",
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "kernels_us": {"mul_mat": round(head["mul_mat_us"], 3),
                       "quantize_row_q8": round(head["quantize_us"], 3)},
        "prefill": prefill,
    }
    if extra:
        line["other_workloads"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
