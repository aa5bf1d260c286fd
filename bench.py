#!/usr/bin/env python3
"""Benchmark of the quantized mul_mat hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only KEY ...] [--all]

A step is one pass of the hot path over one batch: quantize the fp32
activations to int8 blocks and multiply them with the packed weights, for every
projection of the workload.  Two forms are timed for the M = 1 workloads: the
two-call form (quantize_row_q8, then mul_mat per projection) and the fused form
(quantize_mul_mat per input; for Q4_K at M = 1 and K <= 16384 the quantization
runs inside the GEMV launch, and gate||up is one concatenated matrix).  The
faster form is the workload's figure; the other is reported beside it.

Weights are encoded and repacked once before timing (load time).  Every timed
region is exactly K steps replayed from a HIP graph, with the events recorded on
the stream the kernels run on.  The steps rotate over copies of the weights, and
the rotation continues from one replay to the next: a copy is read again only
after every other copy has been read, and the copies together exceed twice the
256 MB Infinity Cache, so every weight byte comes from HBM.  When K steps do not
cover all copies, several graphs of K steps each cover the rotation and are
replayed in turn.

Printed: one JSON line.  Its headline is the Q4_K GEMV weight GB/s of the FFN
workload (c3, the largest single-GPU GEMV configuration) with the roofline of
its dominant kernel and the oracle baseline; beside it every configuration
(c1..c5) with its own roofline and oracle baseline, the prefill GEMM's int8
TOP/s (c5, M = 2048) as the second half of the metric, the calibration probes
(single-kernel HBM read floor and sustained int8 MFMA rate on this machine), and the
NEXT rows (Q6_K, Q2_K, Q4_0 prefill, mul_mat_id).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
MALL_BYTES = 256 << 20
ROTATION_BYTES = 2 * MALL_BYTES
METRIC = "Q4_K GEMV weight GB/s (% HBM peak); prefill GEMM int8 TOPS (% MFMA peak)"
HEADLINE = "c3"
HEADLINE_PREFILL = "c5_m2048"
GEMV_CONFIGS = ("c1", "c2", "c3", "c4_m4", "c4_m8", "c4_m32")
PREFILL_CONFIGS = ("c5_m512", "c5_m2048")
NEXT_DECODE = ("q6K_c2", "q2K_c2")
NEXT_PREFILL = ("q6K_c5_m512", "q6K_c5_m2048", "q2K_c5_m512", "q2K_c5_m2048", "q40_c5_m512", "q40_c5_m2048")
ALL_EXTRA = ("q6K_down",)
WEIGHT_BYTES_PER_ELEMENT = {"q4_0": 18 / 32, "q4_K": 144 / 256, "q6_K": 210 / 256, "q2_K": 84 / 256}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layout", default="repacked", choices=["repacked", "canonical"])
    ap.add_argument("--only", nargs="*", default=None,
                    help="measure only these workload keys (and skip probes, NEXT rows, mul_mat_id)")
    ap.add_argument("--all", action="store_true", help="also the extra workloads (Q6_K down projection)")
    ap.add_argument("--no-next", action="store_true", help="skip the NEXT rows (Q6_K, Q2_K, Q4_0 GEMM, mul_mat_id)")
    ap.add_argument("--no-probes", action="store_true", help="skip the calibration probes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps eagerly instead of replaying HIP graphs "
                         "(for profilers that count per dispatch)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run plain device copies of 256 MiB (a known byte count for "
                         "scaling the HBM read/write counters)")
    return ap.parse_args()


GRAPH = True


def log(msg: str) -> None:
    print(f"bench.py: {msg}", file=sys.stderr, flush=True)


def rotation_copies(min_copies: int, steps: int) -> int:
    """The fewest copies >= min_copies whose rotation lines up with K-step
    replays (copies divides K, or K divides copies), so that the rotation
    continues across replays without re-reading a copy early."""
    c = max(1, min_copies)
    while not (steps % c == 0 or c % steps == 0):
        c += 1
    return c


# ----------------------------------------------------------------- inputs
_FP32 = {}


def fp32_weights(p):
    """fp32 weights of projection p from the seeded generators, cached by
    recipe (c5_m512 and c5_m2048 share one matrix, and so do the formats)."""
    from bit_quantized_mat_quantize_amd.inputs import weights_normal, weights_t4_skewed
    key = (p.w_kind, json.dumps(p.w_seed), p.N, p.K)
    if key not in _FP32:
        if len(_FP32) >= 4:
            _FP32.pop(next(iter(_FP32)))
        _FP32[key] = (weights_normal if p.w_kind == "normal" else weights_t4_skewed)(p.w_seed, p.N, p.K)
    return _FP32[key]


class Prepared:
    """One workload on the GPU: weight copies (rows of one tensor), the fp32
    activations, the Q8 buffers and the outputs.

    fused=False: per input, quantize_row_q8, then mul_mat per projection.
    fused=True: projections that share an input are one matrix (canonical rows
    concatenated along N before the repack: gate||up), and each input takes one
    quantize_mul_mat call."""

    def __init__(self, key: str, layout: str, steps: int, fused: bool = False):
        import torch
        import bit_quantized_mat_quantize_amd as qmm
        from bit_quantized_mat_quantize_amd.inputs import workload

        self.wl = workload(key)
        self.key, self.layout, self.fused = key, layout, fused
        dev = torch.device("cuda:0")
        self.copies = rotation_copies(math.ceil(ROTATION_BYTES / self.wl.weight_bytes), steps)
        groups = {}
        for p in self.wl.projections:
            groups.setdefault(p.act_key or p.name, []).append(p)
        self.groups = []
        for ps in groups.values():
            p0 = ps[0]
            afmt = qmm.ACT_FOR[p0.wfmt]
            x = torch.from_numpy(p0.acts()).to(dev)
            y = torch.empty(qmm.act_bytes(afmt, p0.M, p0.K), dtype=torch.uint8, device=dev)
            canons = []
            for p in ps:
                wf = torch.from_numpy(fp32_weights(p)).to(dev)
                canons.append(qmm.quantize_weights(wf, p.wfmt))
                del wf
            parts = [torch.cat(canons)] if fused else canons
            names = ["||".join(p.name for p in ps)] if fused else [p.name for p in ps]
            Ns = [sum(p.N for p in ps)] if fused else [p.N for p in ps]
            mats = []
            for c, N, name in zip(parts, Ns, names):
                w0 = qmm.repack_weights(c, p0.wfmt, N, p0.K) if layout == "repacked" else c
                nb = w0.numel()
                stride = (nb + 255) // 256 * 256        # every copy 256-byte aligned
                big = torch.empty((self.copies, stride), dtype=torch.uint8, device=dev)
                big[0, :nb].copy_(w0)
                for i in range(1, self.copies):
                    big[i, :nb].copy_(big[0, :nb])
                del w0
                out = torch.empty((p0.M, N), dtype=torch.float32, device=dev)
                mats.append(dict(name=name, ws=big, nb=nb, N=N, out=out,
                                 bytes=int(N * p0.K * WEIGHT_BYTES_PER_ELEMENT[p0.wfmt])))
            del canons, parts
            self.groups.append(dict(p=p0, x=x, y=y, afmt=afmt, mats=mats))
        torch.cuda.synchronize()

    def calls(self):
        """The calls of one step, in order: ("qmm", g, m) for quantize_mul_mat
        of group g and matrix m, ("quantize", g) and ("mul_mat", g, m)."""
        out = []
        for gi, g in enumerate(self.groups):
            if self.fused:
                out += [("qmm", gi, mi) for mi in range(len(g["mats"]))]
            else:
                out.append(("quantize", gi))
                out += [("mul_mat", gi, mi) for mi in range(len(g["mats"]))]
        return out

    def call_bytes(self, call) -> int:
        return 0 if call[0] == "quantize" else self.groups[call[1]]["mats"][call[2]]["bytes"]

    def call_ops(self, call) -> int:
        if call[0] == "quantize":
            return 0
        g = self.groups[call[1]]
        return 2 * g["p"].M * g["mats"][call[2]]["N"] * g["p"].K

    def call_name(self, call) -> str:
        g = self.groups[call[1]]
        if call[0] == "quantize":
            return f"quantize_row_q8 {g['afmt']} M={g['p'].M} K={g['p'].K}"
        m = g["mats"][call[2]]
        what = "quantize_mul_mat" if call[0] == "qmm" else "mul_mat"
        return f"{what} {m['name']} {g['p'].wfmt} M={g['p'].M} N={m['N']} K={g['p'].K}"

    def run(self, call, i: int):
        import bit_quantized_mat_quantize_amd as qmm
        g = self.groups[call[1]]
        p = g["p"]
        if call[0] == "quantize":
            qmm.quantize_row_q8(g["x"], g["afmt"], out=g["y"])
            return
        m = g["mats"][call[2]]
        w = m["ws"][i % self.copies, :m["nb"]]
        if call[0] == "qmm":
            qmm.quantize_mul_mat(p.wfmt, w, g["x"], m["N"], layout=self.layout, y=g["y"], out=m["out"])
        else:
            qmm.mul_mat(p.wfmt, w, g["y"], p.M, m["N"], p.K, layout=self.layout, out=m["out"])

    def step(self, i: int, only=None):
        """Enqueue one step (weight copy i mod copies) on the current stream."""
        for c in self.calls():
            if only is None or c in only:
                self.run(c, i)


WARMUP = 5


def time_steps(prep, steps: int, only=None, min_replays: int = 3):
    """Median and minimum ms per step over timed replays of exactly `steps`
    steps each, after WARMUP untimed eager steps and one untimed cycle of the
    replays.  The graphs cover the copy rotation; replays cycle through them,
    so the rotation continues across replays."""
    import torch
    c = prep.copies
    G = c // steps if c % steps == 0 else 1
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(max(1, WARMUP)):         # warm the kernels on the timing stream
            prep.step(i, only)
    torch.cuda.synchronize()
    graphs = []
    if GRAPH:
        for g in range(G):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=s):
                for i in range(steps):
                    prep.step(g * steps + i, only)
            graphs.append(gr)

    def replay(r):
        if GRAPH:
            graphs[r % G].replay()
        else:
            for i in range(steps):
                prep.step((r % G) * steps + i, only)

    with torch.cuda.stream(s):                  # one untimed cycle of the rotation
        for r in range(G):
            replay(r)
    torch.cuda.synchronize()
    R = max(min_replays, G)
    evs = []
    with torch.cuda.stream(s):
        for r in range(R):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            replay(r)
            e1.record()
            evs.append((e0, e1))
    torch.cuda.synchronize()
    per = sorted(e0.elapsed_time(e1) / steps for e0, e1 in evs)
    del graphs
    return statistics.median(per), per[0]


# ------------------------------------------------------------- rooflines
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_q4_K.md")
_CSRC = "bit_quantized_mat_quantize_amd/csrc/"
KERNEL_SOURCES = {  # the files that define each kernel the counters were taken for
    "k_gemv1_fused_q4_K": ("gemv.hip", "q8k_row.h", "qmm_device.h"),
    "k_gemv1_q4_K": ("gemv.hip", "qmm_device.h"),
    "k_gemv_q4_0": ("gemv.hip", "qmm_device.h"),
    "k_gemv_fused_q4_0": ("gemv.hip", "qmm_device.h"),
    "k_skinny_q4_K": ("skinny.hip", "mfma_common.h", "qmm_device.h"),
    "k_skinny16_q4_K": ("skinny16.hip", "mfma_common.h", "qmm_device.h"),
    "k_skinny16r_q4_K": ("skinny16r.hip", "mfma_common.h", "qmm_device.h"),
    "k_skinny32r_q4_K": ("skinny32r.hip", "mfma_common.h", "qmm_device.h"),
    "k_gemm_q4_K": ("gemm.hip", "mfma_common.h", "qmm_device.h"),
}


def sources_sha(kernel: str):
    import hashlib
    if kernel not in KERNEL_SOURCES:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, _CSRC + f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the FETCH_SIZE and
    WRITE_SIZE counters (each scaled by what it reads for a plain copy of known
    size), or None when no such measurement exists or the kernel sources have
    changed since it was taken."""
    import re
    sha = sources_sha(kernel)
    if sha is None or not os.path.exists(TRAFFIC_FILE):
        return None
    pat = re.compile(r"traffic kernel=(\S+) workload=(\S+) bytes_per_launch=(\d+) sources_sha256_16=(\w+)")
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            m = pat.search(line)
            if m and m.group(1) == kernel and m.group(2) == workload and m.group(4) == sha:
                return int(m.group(3))
    return None


def kernel_of(key: str, call_name: str, fused: bool, layout: str = "repacked") -> str:
    """The kernel the automatic dispatch runs for a measured call (the AUTO
    rules for these shapes are pinned by tests/test_dispatch_log.py)."""
    wfmt = call_name.split()[2]
    M = int(call_name.split("M=")[1].split()[0])
    K = int(call_name.split("K=")[1].split()[0])
    if wfmt == "q4_0":
        N = int(call_name.split("N=")[1].split()[0])
        if M == 1:
            return "k_gemv_fused_q4_0" if fused and K % 64 == 0 and K <= 4096 and N * K <= 1 << 22 else "k_gemv_q4_0"
        return "k_skinny_q4_0" if M <= 32 else "k_gemm_q4_0"
    if wfmt == "q4_K":
        if M == 1:
            return "k_gemv1_fused_q4_K" if fused and K <= 16384 else "k_gemv1_q4_K"
        if M <= 8 and layout == "repacked":
            return "k_skinny16r_q4_K"
        if M <= 32 and layout == "repacked":
            return "k_skinny32r_q4_K"
        if M <= 16:
            return "k_skinny16_q4_K"
        if M <= 32:
            return "k_skinny_q4_K"
        return "k_gemm_q4_K"
    fam = {"q6_K": "q6_K", "q2_K": "q2_K"}[wfmt]
    N = int(call_name.split("N=")[1].split()[0])
    fused_ok = (K <= 4096 and N <= 8192) or (K <= 8192 and N <= 4096) if wfmt == "q6_K" else (K <= 16384 and N <= 8192)
    if M == 1 and fused and fused_ok:
        return f"k_gemv_fused_{fam}"
    return f"k_gemv_{fam}" if M == 1 else (f"k_skinny_{fam}" if M <= 32 else f"k_gemm_{fam}")


# -------------------------------------------------------------- measures
def measure_config(key: str, layout: str, steps: int, forms=(False, True), probe=None):
    """Step time of each form, the per-call times of the faster form, and the
    roofline of its dominant kernel."""
    import torch
    res = {"key": key}
    best = None
    for fused in forms:
        prep = Prepared(key, layout, steps, fused=fused)
        ms, ms_min = time_steps(prep, steps)
        tag = "fused" if fused else "two_call"
        calls = []
        for c in prep.calls():
            cms, _ = time_steps(prep, steps, only={c})
            calls.append(dict(call=prep.call_name(c), us=round(cms * 1e3, 3), bytes=prep.call_bytes(c),
                              ops=prep.call_ops(c)))
        res[tag] = dict(ms_per_step=round(ms, 6), ms_per_step_min=round(ms_min, 6), calls=calls)
        res.update(description=prep.wl.description, weight_bytes=prep.wl.weight_bytes, ops=prep.wl.ops,
                   M=max(p.M for p in prep.wl.projections), copies=prep.copies,
                   rotation_bytes=prep.copies * prep.wl.weight_bytes)
        if best is None or ms < res[best]["ms_per_step"]:
            best = tag
        del prep
        torch.cuda.empty_cache()
        log(f"{key} {tag}: {ms * 1e3:.2f} us per step")
    res["best"] = best
    r = res[best]
    dom = max(r["calls"], key=lambda c: (c["bytes"], c["ops"]))
    kern = kernel_of(key, dom["call"], best == "fused", layout)
    prefill = res["M"] > 32
    if prefill:
        achieved = dom["ops"] / (dom["us"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": profiled_traffic(kern, key)}
    else:
        achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
        wl_tag = key + ("_gate_up" if "||" in dom["call"] else "")
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(kern, wl_tag)}
    roof.update(kernel=kern, call=dom["call"], launch_us=dom["us"],
                per_launch=dom["ops"] if prefill else dom["bytes"])
    if probe is not None:
        if prefill and probe.get("mfma_i8"):
            roof["frac_of_probe"] = round(achieved / probe["mfma_i8"]["TOPS"], 4)
        elif not prefill and probe.get("read"):
            fl = probe["read"].get(str(dom["bytes"]))
            if fl:
                roof["frac_of_probe"] = round(achieved / fl["GBps"], 4)
                roof["probe_floor_us"] = fl["us"]
    res["roofline"] = roof
    ms = r["ms_per_step"]
    if prefill:
        res["value"], res["unit"] = round(res["ops"] / (ms * 1e-3) / 1e12, 1), "TOP/s"
    else:
        res["value"], res["unit"] = round(res["weight_bytes"] / (ms * 1e-3) / 1e9, 1), "GB/s"
        if res["M"] > 1:
            res["int8_tops"] = round(res["ops"] / (ms * 1e-3) / 1e12, 2)
    return res


MOE = dict(E=8, U=2, N=14336, K=4096)   # eight experts of an FFN gate/up projection, two per token


class MoePrepared:
    """mul_mat_id on Q4_K experts: E matrices [N, K] repacked back to back,
    seeded top-U routing, a step = quantize_row_q8 + mul_mat_id.  Copies of the
    whole expert stack rotate so that the routed bytes of the rotation exceed
    twice the Infinity Cache."""

    def __init__(self, T: int, steps: int):
        import numpy as np
        import torch
        import bit_quantized_mat_quantize_amd as qmm
        from bit_quantized_mat_quantize_amd.inputs import activations, weights_t4_skewed
        E, U, N, K = MOE["E"], MOE["U"], MOE["N"], MOE["K"]
        dev = torch.device("cuda:0")
        rng = np.random.default_rng(106)
        ids = np.stack([rng.choice(E, U, replace=False) for _ in range(T)]).astype(np.int32)
        self.experts_used = int(len(np.unique(ids)))
        self.expert_bytes = qmm.weight_bytes("q4_K", "repacked", N, K)
        routed = self.experts_used * self.expert_bytes
        self.copies = rotation_copies(math.ceil(ROTATION_BYTES / routed), steps)
        big = torch.empty((self.copies, E * self.expert_bytes), dtype=torch.uint8, device=dev)
        for e in range(E):
            wf = torch.from_numpy(weights_t4_skewed([6, e], N, K)).to(dev)
            big[0, e * self.expert_bytes:(e + 1) * self.expert_bytes].copy_(
                qmm.repack_weights(qmm.quantize_weights(wf, "q4_K"), "q4_K", N, K))
            del wf
        for i in range(1, self.copies):
            big[i].copy_(big[0])
        self.ws = big
        self.ids = torch.from_numpy(ids).to(dev)
        self.x = torch.from_numpy(activations([106, T], T, K)).to(dev)
        self.y = torch.empty(qmm.act_bytes("q8_K", T, K), dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, U, N), dtype=torch.float32, device=dev)
        self.wsb = torch.empty(max(qmm.mul_mat_id_workspace_bytes(T, U, E), 16), dtype=torch.uint8,
                               device=dev)
        self.T, self.E, self.U, self.N, self.K = T, E, U, N, K
        self.routed_bytes = routed
        torch.cuda.synchronize()

    def step(self, i: int, only=None):
        import bit_quantized_mat_quantize_amd as qmm
        if only is None or "quantize" in only:
            qmm.quantize_row_q8(self.x, "q8_K", out=self.y)
        if only is None or "mul_mat" in only:
            qmm.mul_mat_id_q4_K(self.ws[i % self.copies], self.E, self.y, self.ids, self.N, self.K,
                                layout="repacked", out=self.out, workspace=self.wsb)


def measure_moe(steps: int):
    """Decode (one token) and prefill (512 tokens) through mul_mat_id."""
    import torch
    res = {"experts": MOE["E"], "slots_per_token": MOE["U"], "N": MOE["N"], "K": MOE["K"]}
    for name, T in (("decode_T1", 1), ("prefill_T512", 512)):
        prep = MoePrepared(T, steps)
        ms, _ = time_steps(prep, steps)
        ms_mm, _ = time_steps(prep, steps, only={"mul_mat"})
        r = dict(tokens=T, ms_per_step=round(ms, 6), mul_mat_id_us=round(ms_mm * 1e3, 3),
                 experts_used=prep.experts_used, copies=prep.copies,
                 rotation_routed_bytes=prep.copies * prep.routed_bytes)
        if T == 1:
            wb = prep.routed_bytes
            r.update(weight_bytes=wb, weight_GBps=round(wb / (ms_mm * 1e-3) / 1e9, 1),
                     frac_hbm_peak=round(wb / (ms_mm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        else:
            ops = 2 * T * MOE["U"] * MOE["N"] * MOE["K"]
            r.update(tops=round(ops / (ms_mm * 1e-3) / 1e12, 1),
                     frac_int8_peak=round(ops / (ms_mm * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4))
        res[name] = r
        del prep
        torch.cuda.empty_cache()
        log(f"mul_mat_id {name} done")
    return res


# ---------------------------------------------------------------- probes
def probe_sizes():
    """Byte counts of the GEMV-family launches measured here (one probe per
    size) and 512 MiB for the sustained rate."""
    from bit_quantized_mat_quantize_amd.inputs import workload
    sizes = set()
    for key in GEMV_CONFIGS:
        wl = workload(key)
        groups = {}
        for p in wl.projections:
            groups.setdefault(p.act_key or p.name, []).append(p)
        for ps in groups.values():
            for p in ps:
                sizes.add(int(p.N * p.K * WEIGHT_BYTES_PER_ELEMENT[p.wfmt]))
            if len(ps) > 1:
                sizes.add(int(sum(p.N * p.K * WEIGHT_BYTES_PER_ELEMENT[p.wfmt] for p in ps)))
    sizes.add(512 << 20)
    return sorted(sizes)


def measure_probes(steps: int):
    """Single-kernel streaming-read floor per byte count (best of 1, 2, 4 and 8
    loads per thread; launches back to back in a HIP graph, reading disjoint
    regions of a 1 GiB buffer so that reads come from HBM for the sizes that
    matter), and the sustained int8 MFMA rate."""
    import torch
    from bit_quantized_mat_quantize_amd import _probe
    dev = torch.device("cuda:0")
    res = {"read": {}, "mfma_i8": None}
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    msink = torch.empty(_probe.mfma_sink_bytes() // 4, dtype=torch.int32, device=dev)
    # MFMA first: it also brings the clocks up before the timed configurations
    iters = 2048
    s = torch.cuda.Stream()
    best = None
    with torch.cuda.stream(s):
        for w in range(3):
            _probe.probe_mfma_i8(msink, iters, w)
        torch.cuda.synchronize()
        for rep in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for w in range(4):
                _probe.probe_mfma_i8(msink, iters, w)
            e1.record()
            e1.synchronize()
            ms = e0.elapsed_time(e1) / 4
            best = ms if best is None else min(best, ms)
    tops = _probe.mfma_ops(iters) / (best * 1e-3) / 1e12
    res["mfma_i8"] = {"TOPS": round(tops, 1), "frac_spec": round(tops / INT8_PEAK_TOPS, 4),
                      "launch_us": round(best * 1e3, 2),
                      "kernel": "k_probe_mfma: 4 independent v_mfma_i32_32x32x32_i8 chains per wavefront, "
                                "8 wavefronts per SIMD"}
    buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for nbytes in probe_sizes():
        stride = (nbytes + 4095) // 4096 * 4096
        slots = max(1, min(256, buf.numel() // stride))
        n_launch = max(steps, slots)
        best = None
        for lpt in (1, 2, 4, 8):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                for i in range(3):
                    _probe.probe_read(buf, (i % slots) * stride, nbytes, sink, lpt)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for i in range(n_launch):
                    _probe.probe_read(buf, (i % slots) * stride, nbytes, sink, lpt)
            with torch.cuda.stream(s):
                g.replay()
                per = []
                for rep in range(3):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    g.replay()
                    e1.record()
                    per.append((e0, e1))
            torch.cuda.synchronize()
            ms = min(a.elapsed_time(b) for a, b in per) / n_launch
            if best is None or ms < best[0]:
                best = (ms, lpt)
            del g
        gbps = nbytes / (best[0] * 1e-3) / 1e9
        res["read"][str(nbytes)] = {"bytes": nbytes, "us": round(best[0] * 1e3, 3), "GBps": round(gbps, 1),
                                    "frac_spec": round(gbps / HBM_PEAK_GBS, 4), "loads_per_thread": best[1],
                                    "distinct_bytes_per_replay": min(slots, n_launch) * nbytes}
    del buf, msink
    torch.cuda.empty_cache()
    log("probes done")
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


# ----------------------------------------------------------- CPU baseline
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_runs(fn, n: int) -> float:
    ts = []
    for _ in range(n):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts)


def cpu_baseline(key: str):
    """The oracle's integer path (plain C, OpenMP over output rows) on the GPU
    box's host cores, on the workload's own bytes (encoded by the oracle from
    the same fp32 arrays).  M <= 32 configurations: the whole step, median of 5
    on all cores; the one-thread figure is the median of 3 (one run, or a row
    sample, where that would take long).  Prefill: one sampled run per M (a
    block of activation rows against a block of weight rows)."""
    import oracle
    from bit_quantized_mat_quantize_amd.inputs import workload
    wl = workload(key)
    threads = min(len(os.sched_getaffinity(0)), oracle.max_threads())
    prefill = max(p.M for p in wl.projections) > 32
    if prefill:
        p = wl.projections[0]
        Ms, Ns = 64, 4096
        w = oracle.quantize(p.wfmt, fp32_weights(p)[:Ns])
        afmt = "q8_0" if p.wfmt == "q4_0" else "q8_K"
        x = p.acts()
        y = oracle.quantize(afmt, x[:Ms])
        run = lambda m, nt: oracle.mul_mat(p.wfmt, w, y[:m], m, Ns, p.K, nthreads=nt)  # noqa: E731
        run(Ms, threads)
        t = _time_runs(lambda: run(Ms, threads), 1)
        M1 = 8
        t1 = _time_runs(lambda: run(M1, 1), 1)
        ops, ops1 = 2 * Ms * Ns * p.K, 2 * M1 * Ns * p.K
        return {"value": round(ops / t / 1e12, 5), "unit": "TOP/s", "cores": threads, "kind": "oracle",
                "sample": f"{Ms} of the {p.M} activation rows x {Ns} of the {p.N} weight rows of {key} "
                          f"(K={p.K}), integer path, one run of {t:.2f} s",
                "value_1_thread": round(ops1 / t1 / 1e12, 5),
                "sample_1_thread": f"{M1} rows x {Ns} weight rows, one run of {t1:.2f} s",
                "cpu_model": cpu_model()}
    items = []
    for p in wl.projections:
        afmt = "q8_0" if p.wfmt == "q4_0" else "q8_K"
        items.append((p, oracle.quantize(p.wfmt, fp32_weights(p)), oracle.quantize(afmt, p.acts())))

    def step(nt, rows=None):
        for p, w, y in items:
            m = p.M if rows is None else min(rows, p.M)
            oracle.mul_mat(p.wfmt, w, y[:m], m, p.N, p.K, nthreads=nt)

    step(threads)
    t = _time_runs(lambda: step(threads), 5)
    M = max(p.M for p in wl.projections)
    wb = wl.weight_bytes
    rows1 = M if M <= 8 else 8
    n1 = 3 if M == 1 else 1
    t1 = _time_runs(lambda: step(1, rows1), n1)
    val1 = wb / t1 / 1e9 * (M / rows1 if rows1 < M else 1)  # the per-row cost is the same for every row
    out = {"value": round(wb / t / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"the whole step of {key} ({wl.description}), integer path, median of 5 runs "
                     f"({t * 1e3:.2f} ms)",
           "value_1_thread": round(val1, 4),
           "sample_1_thread": (f"median of {n1}" if rows1 == M else
                               f"{rows1} of the {M} activation rows, one run, scaled to all rows") +
                              f" ({t1 * 1e3:.1f} ms)",
           "cpu_model": cpu_model()}
    if M > 1:
        out["int8_gops"] = round(wl.ops / t / 1e9, 2)
    return out


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


def summary(res: dict) -> dict:
    """The compact per-configuration object of the JSON line."""
    best = res["best"]
    out = {"workload": f"{res['key']}: {res['description']}", "form": best,
           "ms_per_step": res[best]["ms_per_step"], "value": res["value"], "unit": res["unit"],
           "frac_peak": round(res["value"] / (INT8_PEAK_TOPS if res["unit"] == "TOP/s" else HBM_PEAK_GBS), 4),
           "roofline": res["roofline"], "calls": res[best]["calls"],
           "weight_copies_rotated": res["copies"], "rotation_bytes": res["rotation_bytes"]}
    other = "two_call" if best == "fused" else "fused"
    if other in res:
        out["other_form"] = {"form": other, "ms_per_step": res[other]["ms_per_step"]}
    if "int8_tops" in res:
        out["int8_tops"] = res["int8_tops"]
    if "cpu_baseline" in res:
        out["cpu_baseline"] = res["cpu_baseline"]
    return out


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
    steps = a.steps
    only = set(a.only) if a.only is not None else None

    global WARMUP
    WARMUP = a.warmup
    probe = None if (a.no_probes or only is not None) else measure_probes(steps)
    main_keys = [k for k in GEMV_CONFIGS + PREFILL_CONFIGS + (ALL_EXTRA if a.all else ())
                 if only is None or k in only]
    results = {}
    for k in main_keys:
        # quantize_mul_mat fuses only at M = 1; above it is the same two launches
        forms = (False, True) if k in ("c1", "c2", "c3", "q6K_down") else (False,)
        r = measure_config(k, a.layout, steps, forms=forms, probe=probe)
        if not a.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline(k)
            log(f"{k} oracle baseline done")
        results[k] = r
    nxt = {}
    if not a.no_next and only is None:
        for k in NEXT_DECODE + NEXT_PREFILL:
            # Q6_K and Q2_K fuse the quantization into their M = 1 GEMVs
            r = measure_config(k, a.layout, steps, forms=(False, True) if k in NEXT_DECODE else (False,),
                               probe=probe)
            nxt[k] = summary(r)
        nxt["mul_mat_id_q4_K"] = measure_moe(steps)
    elif only is not None:
        for k in [k for k in NEXT_DECODE + NEXT_PREFILL + ALL_EXTRA if k in only and k not in results]:
            nxt[k] = summary(measure_config(k, a.layout, steps,
                                            forms=(False, True) if k in NEXT_DECODE + ("q6K_down",) else (False,),
                                            probe=probe))

    head = results.get(HEADLINE) or (results[main_keys[0]] if main_keys else None)
    line = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": a.warmup,
            "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "int8", "data": "synthetic"}
    if head is not None:
        best = head["best"]
        line.update(value=head["value"], unit=head["unit"], ms_per_step=head[best]["ms_per_step"])
        line["config"] = {
            "workload": f"{head['key']}: {head['description']}", "weight_layout": a.layout,
            "weight_bytes": head["weight_bytes"], "weight_copies_rotated": head["copies"],
            "rotation_bytes": head["rotation_bytes"],
            "step": ("quantize_mul_mat per input (gate||up concatenated; Q8_K quantization inside the GEMV "
                     "launch where K <= 16384)" if best == "fused" else "quantize_row_q8 + mul_mat per projection")
                    + ", HIP graph replay of exactly `steps` steps",
            "parallelism": "single GPU"}
        line["roofline"] = head["roofline"]
        line["cpu_baseline"] = head.get("cpu_baseline")
    pf = results.get(HEADLINE_PREFILL)
    if pf is not None:
        line["prefill_gemm"] = {"workload": f"{pf['key']}: {pf['description']}", "value": pf["value"],
                                "unit": "TOP/s", "frac_int8_peak": round(pf["value"] / INT8_PEAK_TOPS, 4),
                                "ms_per_step": pf[pf["best"]]["ms_per_step"]}
        line["roofline_prefill"] = pf["roofline"]
        line["cpu_baseline_prefill"] = pf.get("cpu_baseline")
    line["configs"] = {k: summary(r) for k, r in results.items()}
    if probe is not None:
        line["probes"] = probe
    if nxt:
        line["next_rows"] = nxt
    line["system"] = system_info()
    if not GRAPH:
        line["timing"] = "eager launches (--no-graph)"
    if a.calibrate_copy:
        line["copy_calibration"] = calibrate_copy()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
