#!/usr/bin/env python3
"""Benchmark of the quantized mul_mat hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--no-prefill]

A step is one pass of the hot path over one batch: quantize the fp32
activations to int8 blocks and multiply them with the packed 4-bit weights, for
every projection of the workload.  Two forms are timed: the two-call form
(quantize_row_q8, then mul_mat per projection) and the fused form
(quantize_mul_mat per input; for Q4_K at M = 1 the quantization runs inside the
GEMV launch, and gate||up is one concatenated matrix).  The faster one is the
headline; the other is reported beside it.  The weights are
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
PREFILL = ("c5_m512", "c5_m2048", "q6K_c5_m512", "q6K_c5_m2048", "q2K_c5_m512", "q2K_c5_m2048",
           "q40_c5_m512", "q40_c5_m2048")


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
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps eagerly instead of replaying a HIP graph "
                         "(for profilers that count per dispatch)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run plain device copies of 256 MiB (a known byte count for "
                         "scaling the HBM read/write counters)")
    return ap.parse_args()


GRAPH = True


class Prepared:
    """One workload on the GPU: weight copies, activations, outputs.

    fused=False: per projection, quantize_row_q8 (once per distinct input)
    then mul_mat.  fused=True: projections that share an input are one matrix
    (canonical rows concatenated along N, then repacked: gate||up), and each
    input takes one quantize_mul_mat call (one launch for Q4_K at M = 1)."""

    def __init__(self, key: str, layout: str, min_bytes: int, fused: bool = False):
        import torch
        import bit_quantized_mat_quantize_amd as qmm
        from bit_quantized_mat_quantize_amd.inputs import workload

        self.wl = workload(key)
        self.layout = layout
        self.fused = fused
        dev = torch.device("cuda:0")
        wbytes = self.wl.weight_bytes
        self.copies = max(1, -(-min_bytes // wbytes))
        groups = {}
        for p in self.wl.projections:
            groups.setdefault(p.act_key or p.name, []).append(p)
        self.items = []
        for key_a, ps in groups.items():
            p0 = ps[0]
            afmt = qmm.ACT_FOR[p0.wfmt]
            x = torch.from_numpy(p0.acts()).to(dev)
            y = torch.empty(qmm.act_bytes(afmt, p0.M, p0.K), dtype=torch.uint8, device=dev)
            canons = []
            for p in ps:
                wf = torch.from_numpy(p.weights()).to(dev)
                canons.append(qmm.quantize_weights(wf, p.wfmt))
                del wf
            parts = [torch.cat(canons)] if fused else canons
            Ns = [sum(p.N for p in ps)] if fused else [p.N for p in ps]
            mats = []
            for c, N in zip(parts, Ns):
                w0 = qmm.repack_weights(c, p0.wfmt, N, p0.K) if layout == "repacked" else c
                ws = [w0] + [w0.clone() for _ in range(self.copies - 1)]
                out = torch.empty((p0.M, N), dtype=torch.float32, device=dev)
                mats.append(dict(ws=ws, N=N, out=out))
            del canons, parts
            self.items.append(dict(p=p0, x=x, y=y, afmt=afmt, mats=mats))
        torch.cuda.synchronize()

    def step(self, i: int, only: str | None = None):
        """Enqueue one step on the current stream (weight copy i mod copies)."""
        import bit_quantized_mat_quantize_amd as qmm
        for it in self.items:
            p = it["p"]
            if self.fused and only is None:
                for m in it["mats"]:
                    qmm.quantize_mul_mat(p.wfmt, m["ws"][i % self.copies], it["x"], m["N"],
                                         layout=self.layout, y=it["y"], out=m["out"])
                continue
            if only in (None, "quantize"):
                qmm.quantize_row_q8(it["x"], it["afmt"], out=it["y"])
            if only in (None, "mul_mat"):
                for m in it["mats"]:
                    qmm.mul_mat(p.wfmt, m["ws"][i % self.copies], it["y"], p.M, m["N"], p.K,
                                layout=self.layout, out=m["out"])

    @property
    def calls_per_step(self) -> int:
        """mul_mat (or quantize_mul_mat) calls per step."""
        return sum(len(it["mats"]) for it in self.items)


def time_graph(prep: Prepared, steps: int, only=None, reps: int = 1):
    """Capture `steps` steps in one HIP graph, replay it, return ms per step
    (with GRAPH off: launch the steps eagerly and time them with events)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):                  # warm the kernels on the timing stream
            prep.step(i, only)
    torch.cuda.synchronize()
    g = None
    if GRAPH:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                prep.step(i, only)
        g.replay()                           # untimed replay
        torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):           # events on the stream the kernels run on
            e0.record()
            if g is not None:
                g.replay()
            else:
                for i in range(steps):
                    prep.step(i, only)
            e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        best = ms if best is None else min(best, ms)
    del g
    return best


MOE = dict(E=8, U=2, N=14336, K=4096)   # eight experts of an FFN gate/up projection, two per token


class MoePrepared:
    """mul_mat_id on Q4_K experts: E matrices [N, K] repacked back to back,
    seeded top-U routing, a step = quantize_row_q8 + mul_mat_id."""

    def __init__(self, T: int, copies: int):
        import numpy as np
        import torch
        import bit_quantized_mat_quantize_amd as qmm
        from bit_quantized_mat_quantize_amd.inputs import activations, weights_t4_skewed
        E, U, N, K = MOE["E"], MOE["U"], MOE["N"], MOE["K"]
        dev = torch.device("cuda:0")
        mats = []
        for e in range(E):
            wf = torch.from_numpy(weights_t4_skewed([6, e], N, K)).to(dev)
            mats.append(qmm.repack_weights(qmm.quantize_weights(wf, "q4_K"), "q4_K", N, K))
            del wf
        w0 = torch.cat(mats)
        del mats
        self.ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        self.copies = copies
        rng = np.random.default_rng(106)
        ids = np.stack([rng.choice(E, U, replace=False) for _ in range(T)]).astype(np.int32)
        self.ids = torch.from_numpy(ids).to(dev)
        self.x = torch.from_numpy(activations([106, T], T, K)).to(dev)
        self.y = torch.empty(qmm.act_bytes("q8_K", T, K), dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, U, N), dtype=torch.float32, device=dev)
        self.wsb = torch.empty(max(qmm.mul_mat_id_workspace_bytes(T, U, E), 16), dtype=torch.uint8,
                               device=dev)
        self.T, self.E, self.U, self.N, self.K = T, E, U, N, K
        self.experts_used = int(len(np.unique(ids)))
        self.expert_bytes = qmm.weight_bytes("q4_K", "repacked", N, K)
        torch.cuda.synchronize()

    def step(self, i: int, only: str | None = None):
        import bit_quantized_mat_quantize_amd as qmm
        if only in (None, "quantize"):
            qmm.quantize_row_q8(self.x, "q8_K", out=self.y)
        if only in (None, "mul_mat"):
            qmm.mul_mat_id_q4_K(self.ws[i % self.copies], self.E, self.y, self.ids, self.N, self.K,
                                layout="repacked", out=self.out, workspace=self.wsb)


def measure_moe(steps: int):
    """Decode (one token) and prefill (512 tokens) through mul_mat_id."""
    import torch
    res = {"experts": MOE["E"], "slots_per_token": MOE["U"], "N": MOE["N"], "K": MOE["K"]}
    for name, T, copies, st in (("decode_T1", 1, 2, steps), ("prefill_T512", 512, 1, max(5, steps // 10))):
        prep = MoePrepared(T, copies)
        ms = time_graph(prep, st, reps=3)
        ms_mm = time_graph(prep, st, only="mul_mat", reps=3)
        r = dict(tokens=T, ms_per_step=round(ms, 6), mul_mat_id_us=round(ms_mm * 1e3, 3),
                 experts_used=prep.experts_used)
        if T == 1:
            wb = prep.experts_used * prep.expert_bytes
            r.update(weight_bytes=wb, weight_GBps=round(wb / (ms_mm * 1e-3) / 1e9, 1),
                     frac_hbm_peak=round(wb / (ms_mm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        else:
            ops = 2 * T * MOE["U"] * MOE["N"] * MOE["K"]
            r.update(tops=round(ops / (ms_mm * 1e-3) / 1e12, 1),
                     frac_int8_peak=round(ops / (ms_mm * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4))
        res[name] = r
        del prep
        torch.cuda.empty_cache()
    return res


def calibrate_copy():
    """Plain device copies of a known size (read 256 MiB, write 256 MiB)."""
    import torch
    n = (256 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return {"bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4, "copies": 3}


def cpu_baseline(key: str, seconds: float):
    """The oracle's integer path on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    from bit_quantized_mat_quantize_amd.inputs import workload

    wl = workload(key)
    p = max(wl.projections, key=lambda q: q.N * q.K)
    M_s = min(p.M, 2)
    w = oracle.quantize(p.wfmt, p.weights())
    afmt = "q8_0" if p.wfmt == "q4_0" else "q8_K"
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
    # the same sample on one thread (half the time budget)
    t0 = time.perf_counter()
    reps1 = 0
    while True:
        oracle.mul_mat(p.wfmt, w, y, M_s, p.N, p.K, nthreads=1)
        reps1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= seconds / 2:
            break
    per1 = el1 / reps1
    wbytes = p.N * p.K * {"q4_0": 18 / 32, "q4_K": 144 / 256, "q6_K": 210 / 256, "q2_K": 84 / 256}[p.wfmt]
    if p.M <= 8:
        val, val1, unit = wbytes / per / 1e9, wbytes / per1 / 1e9, "GB/s"
        sample = (f"{p.name} projection of {key} (M={M_s}, N={p.N}, K={p.K}), integer path, "
                  f"{reps} repetitions in {el:.1f} s")
    else:
        ops = 2 * M_s * p.N * p.K
        val, val1, unit = ops / per / 1e12, ops / per1 / 1e12, "TOPS"
        sample = (f"{M_s} of the {p.M} activation rows of {key} (N={p.N}, K={p.K}), "
                  f"integer path, {reps} repetitions in {el:.1f} s")
    return {"value": round(val, 4), "unit": unit, "cores": min(threads, oracle.max_threads()),
            "kind": "oracle", "sample": sample, "value_1_thread": round(val1, 4),
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def system_info() -> dict:
    """GPU name and the HIP / ROCm versions of this run."""
    import torch
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as fh:
            rocm = fh.read().strip()
    except OSError:
        pass
    return {"gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip, "rocm": rocm}


def measure_decode(key: str, layout: str, steps: int, warmup: int):
    """Step time of the two-call path and of the fused path, plus the
    per-kernel times that give the roofline of the dominant kernel."""
    import torch
    res = dict(key=key)
    for fused in (False, True):
        prep = Prepared(key, layout, min_bytes=2 * MALL_BYTES, fused=fused)
        for i in range(warmup):
            prep.step(i)
        torch.cuda.synchronize()
        wbytes = prep.wl.weight_bytes
        ms_step = time_graph(prep, steps, reps=3)
        tag = "fused" if fused else "unfused"
        res[tag] = dict(ms_per_step=ms_step, value=wbytes / (ms_step * 1e-3) / 1e9,
                        calls_per_step=prep.calls_per_step)
        if not fused:
            res[tag]["mul_mat_us"] = time_graph(prep, steps, only="mul_mat", reps=3) * 1e3
            res[tag]["quantize_us"] = time_graph(prep, steps, only="quantize", reps=3) * 1e3
            ops = sum(2 * q.M * q.N * q.K for q in prep.wl.projections)
            if max(q.M for q in prep.wl.projections) > 1:  # small batch: also int8 TOPS
                res[tag]["mul_mat_tops"] = ops / (res[tag]["mul_mat_us"] * 1e-6) / 1e12
        res.update(description=prep.wl.description, weight_bytes=wbytes, copies=prep.copies)
        del prep
        torch.cuda.empty_cache()
    return res


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gemv1_q4_K_c2.md")
TRAFFIC_SOURCES = ("bit_quantized_mat_quantize_amd/csrc/gemv.hip",
                   "bit_quantized_mat_quantize_amd/csrc/qmm_device.h")


def profiled_traffic(kernel: str, key: str):
    """HBM bytes per launch measured with the FETCH_SIZE / WRITE_SIZE counters
    (scaled by a plain copy of known size), or None when no measurement exists
    for this kernel and workload or the kernel sources changed since."""
    import hashlib
    import re
    if not os.path.exists(TRAFFIC_FILE):
        return None
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    sha = h.hexdigest()[:16]
    pat = re.compile(r"traffic kernel=(\S+) workload=(\S+) bytes_per_launch=(\d+) sources_sha256_16=(\w+)")
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            m = pat.search(line)
            if m and m.group(1) == kernel and m.group(2) == key and m.group(4) == sha:
                return int(m.group(3))
    return None


def roofline_of(res: dict, path: str) -> dict:
    """Roofline of the dominant kernel: weight bytes per launch / launch time."""
    r = res[path]
    n = r["calls_per_step"]
    ms = r["ms_per_step"] if path == "fused" else r["mul_mat_us"] * 1e-3
    achieved = res["weight_bytes"] / n / (ms / n * 1e-3) / 1e9
    kernel = "k_gemv1_fused_q4_K" if path == "fused" else "k_gemv1_q4_K"
    traffic = profiled_traffic(kernel, res["key"]) if n == 1 and res["key"] == "c2" else None
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}


def measure_prefill(key: str, layout: str, steps: int):
    import torch
    prep = Prepared(key, layout, min_bytes=0)
    p = prep.items[0]["p"]
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
    global GRAPH
    GRAPH = not a.no_graph
    qmm.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if a.prefill_only:
        res = {k: measure_prefill(k, a.layout, a.prefill_steps) for k in PREFILL}
        print(json.dumps({"prefill": res}), flush=True)
        return
    head = measure_decode(a.workload, a.layout, a.steps, a.warmup)
    extra = {}
    if a.all:
        for k in ("c1", "c2", "c3", "c4_m4", "c4_m8", "c4_m32", "q6K_down", "q2K_c2"):
            if k != a.workload:
                r = measure_decode(k, a.layout, a.steps, a.warmup)
                print(f"bench.py: {k} done", file=sys.stderr, flush=True)
                extra[k] = _rounded(r)
    q6 = measure_decode("q6K_c2", a.layout, a.steps, a.warmup)
    moe = measure_moe(a.steps)
    print("bench.py: mul_mat_id done", file=sys.stderr, flush=True)
    prefill = {}
    if not a.no_prefill:
        for k in PREFILL:
            prefill[k] = measure_prefill(k, a.layout, a.prefill_steps)
            print(f"bench.py: {k} done", file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(a.workload, a.cpu_seconds)

    best = "fused" if head["fused"]["ms_per_step"] <= head["unfused"]["ms_per_step"] else "unfused"
    hb = head[best]
    line = {
        "metric": METRIC,
        "value": round(hb["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(hb["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{head['key']}: {head['description']}",
                   "weight_layout": a.layout, "weight_bytes": head["weight_bytes"],
                   "weight_copies_rotated": head["copies"],
                   "step": ("quantize_mul_mat (Q8_K quantization inside the GEMV launch)"
                            if best == "fused" else "quantize_row_q8 + mul_mat")
                           + ", HIP graph replay",
                   "parallelism": "single GPU"},
        "roofline": roofline_of(head, best),
        "cpu_baseline": cpu,
        "two_call_step": {"ms_per_step": round(head["unfused"]["ms_per_step"], 6),
                          "value": round(head["unfused"]["value"], 2),
                          "mul_mat_us": round(head["unfused"]["mul_mat_us"], 3),
                          "quantize_row_q8_us": round(head["unfused"]["quantize_us"], 3),
                          "roofline_mul_mat": roofline_of(head, "unfused")},
        "prefill": prefill,
        "q6_K_gemv": {"workload": f"q6K_c2: {q6['description']}",
                      "value": round(q6["unfused"]["value"], 2), "unit": "GB/s",
                      "ms_per_step": round(q6["unfused"]["ms_per_step"], 6),
                      "mul_mat_us": round(q6["unfused"]["mul_mat_us"], 3),
                      "roofline_mul_mat": roofline_of(q6, "unfused")},
        "mul_mat_id_q4_K": moe,
        "system": system_info(),
    }
    if extra:
        line["other_workloads"] = extra
    if not GRAPH:
        line["timing"] = "eager launches (--no-graph)"
    if a.calibrate_copy:
        line["copy_calibration"] = calibrate_copy()
    print(json.dumps(line), flush=True)


def _rounded(obj):
    if isinstance(obj, dict):
        return {k: _rounded(v) for k, v in obj.items()}
    if isinstance(obj, float):
        return round(obj, 4)
    return obj


if __name__ == "__main__":
    main()
