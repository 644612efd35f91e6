#!/usr/bin/env python3
"""Benchmark of the fused low-bit weight-only GEMV on one MI355X.

Default workload (one JSON line): the M = 1 W2 GEMV of a 14336 x 4096 layer
(Llama-3-8B MLP gate/up shape): Lloyd-Max 2-bit codes with OLS group-32
scale/zero, 143 (3.5%) FP16 outlier columns, x FP16 with 1% of channels x100.
One step = one launch of the whole fused path (stream codes, scales, zeros and
the outlier slab; decode; multiply; reduce; add the outlier columns; store y).

Measurement:
* weights are rotated through >= 512 MB of distinct device copies so neither
  the 256 MB Infinity Cache nor the L2s serve repeats; inputs sit in HBM
  before the timed region;
* the timed launches are captured once into a HIP graph (the kernels are
  launched through the library's C ABI during capture) and replayed; hipEvents
  on the replay stream bracket exactly --steps launches, with device
  synchronization on both sides (--eager times Python-side launches instead,
  which measures the interpreter, not the GPU);
* value = algorithmic bytes per step (codes + FP16 scales + FP16 zeros + FP16
  outlier slab + int32 indices + x + y) / time per step.

Other workloads (--workload): w4_4096 (W4 4096x4096), sweep (Llama-3-8B-shaped
decode in one graph -> tokens/s: 225 separate W4 GEMVs per token, and 129 with
q|k|v and gate|up stacked along N), batched (W4 small-M
matrix-core path vs M repeated GEMVs), w2_70b (W2 + outliers at 28672x8192 and
8192x28672, M = 1 and 8), embed (row gather from a 131072 x 4096 W4 table),
kurtosis (the kurtosis-adaptive outlier policy on the W2 layers),
read / copy (plain streaming kernels: the attainable
HBM rate and the byte-counter calibration).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "M=1 dequant-GEMV effective HBM GB/s (% of MI355X peak); eq. tokens/s"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["wq_gemv.hip", "wq_mma.hip", "wq_mma.h", "wq_common.cuh", "wq_device.h",
                  "wq_select.cuh"]


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="w2_14336",
                   choices=["w2_14336", "w4_4096", "sweep", "batched", "w2_70b", "embed",
                            "kurtosis", "refine", "read", "copy", "probe_sweep"])
    p.add_argument("--bytes", type=int, default=26157628,
                   help="bytes per launch of the read / copy workloads")
    p.add_argument("--probe-sizes", default="",
                   help="probe_sweep workload: comma-separated byte counts")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--m", type=int, default=0,
                   help="batched workload: only this M (default: 2, 4, 8 and 16)")
    p.add_argument("--shape", default="",
                   help="batched workload: only this NxK (default: 14336x4096 and 4096x14336)")
    p.add_argument("--eager", action="store_true", help="time Python-side launches, no graph")
    p.add_argument("--w4-zeros", default="fp16", choices=["fp16", "packed"],
                   help="zero points of the W4 workloads (w4_4096, sweep, batched): FP16, or "
                        "packed two per byte (the W4P format)")
    p.add_argument("--layout", default="best", choices=["best", "tiled", "rowmajor"],
                   help="packed-array layout whose time the M = 1 GEMV workloads report as "
                        "`value` (best: the faster of the two; the other one is timed too and "
                        "reported beside it)")
    return p.parse_args()


def kernel_source_hash() -> str:
    """Hash of the M = 1 kernels' code with comments and layout removed, so
    that counters stay attached to the code they were taken on and survive
    edits of comments only."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_weight_only_gemv_amd", "csrc", f), encoding="utf-8") as fh:
            t = fh.read()
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        h.update(" ".join(t.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def sweep_bytes_per_token(fmt: int, ratio: float) -> int:
    """Algorithmic bytes of one Llama-3-8B-shaped decode step (32 layers x 7
    projections + LM head) in the given format."""
    import synthetic
    tot = 0
    for (_, _, _, N, K) in synthetic.config3_shapes():
        n_out = int(np.floor(ratio * K)) if ratio > 0 else 0
        G = K // 32
        codes = N * K // (4 if fmt == 2 else 2)
        zeros = N * ((G + 1) // 2) if fmt == 5 else 2 * N * G   # W4P: packed, else FP16
        tot += codes + 2 * N * G + zeros + 2 * N * n_out + 4 * n_out + 2 * K + 2 * N
    return tot


class Timer:
    """Times exactly `steps` calls of fn(i) after `warmup` untimed ones.  The
    steps are captured into a HIP graph of `per` launches (the library is
    called through its C ABI during capture), a whole multiple of `period` (the
    number of rotated buffer copies, so that every replay walks all of them),
    replayed R times with an event on the launching stream between replays; a
    second graph holds the steps - R per left over.  One synchronization ends
    the timed region.  Returns a Timing: the time per step (median over the
    replays, their 10th and 90th percentiles, and the mean over all steps)."""

    REPLAYS = 20
    LEAD_CYCLES = 250_000

    def __init__(self, torch, eager=False):
        self.torch, self.eager = torch, eager

    def _capture(self, fn, n):
        torch = self.torch
        graph = torch.cuda.CUDAGraph()
        stream = torch.cuda.current_stream()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(n):
                    fn(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        return graph

    def __call__(self, fn, steps, warmup, period=1):
        torch = self.torch
        steps = max(1, int(steps))
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        period = max(1, int(period))
        per = -(-max(1, steps // self.REPLAYS) // period) * period
        per = min(per, steps)
        reps = steps // per
        rest = steps - reps * per
        stream = torch.cuda.current_stream()
        g_main = g_rest = None
        if not self.eager:
            g_main = self._capture(fn, per)
            if rest:
                g_rest = self._capture(fn, rest)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
        torch.cuda.synchronize()
        # a bounded spin on the stream first (about 0.1 ms), so that the
        # launches below are queued on the GPU before the first event fires:
        # the timed region then holds the kernels, not the host's latency to
        # submit the first of them
        torch.cuda._sleep(self.LEAD_CYCLES)
        ev[0].record(stream)
        for r in range(reps):
            if g_main is not None:
                g_main.replay()
            else:
                for i in range(per):
                    fn(r * per + i)
            ev[r + 1].record(stream)
        if rest:
            if g_rest is not None:
                g_rest.replay()
            else:
                for i in range(rest):
                    fn(reps * per + i)
        ev[reps + 1].record(stream)
        torch.cuda.synchronize()
        t = np.array([ev[r].elapsed_time(ev[r + 1]) / per for r in range(reps)])
        mean = ev[0].elapsed_time(ev[reps + 1]) / steps
        return Timing(float(np.median(t)), float(np.percentile(t, 10)),
                      float(np.percentile(t, 90)), float(mean), steps)


class Timing(float):
    """Milliseconds per step (the median over replays) with the spread."""

    def __new__(cls, median, p10, p90, mean, steps):
        o = super().__new__(cls, median)
        o.p10, o.p90, o.mean, o.steps = p10, p90, mean, steps
        return o

    def us(self):
        return {"median": round(self * 1e3, 3), "p10": round(self.p10 * 1e3, 3),
                "p90": round(self.p90 * 1e3, 3), "mean": round(self.mean * 1e3, 3)}


def clone_layer(DeviceLayer, base):
    c = DeviceLayer.__new__(DeviceLayer)
    c.__dict__.update(base.__dict__)
    c.codes, c.scales, c.zeros = base.codes.clone(), base.scales.clone(), base.zeros.clone()
    if base.n_out:
        c.idx, c.wout = base.idx.clone(), base.wout.clone()
    if base.tiled is not None:
        c.tiled = base.tiled.clone()
    return c


def rotated(DeviceLayer, base, nbytes):
    ncopy = max(1, -(-ROTATE_BYTES // nbytes))
    return [base] + [clone_layer(DeviceLayer, base) for _ in range(ncopy - 1)]


def traffic_for(label):
    """HBM bytes per launch from stored counter runs, if they were taken on the
    current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(label)
    if not e or e.get("kernel_source_hash") != kernel_source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def read_probe_rate(torch, timer, nbytes, steps, warmup):
    """Attainable streaming-read rate at this many bytes per launch: the plain
    read kernel over rotated buffers, timed like the GEMV (GB/s)."""
    import bit_weight_only_gemv_amd as B
    nb = (nbytes + 15) // 16 * 16
    ncopy = max(1, -(-ROTATE_BYTES // nb))
    bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
    sink = torch.empty(B.wq_read_probe_sink_words(nb), dtype=torch.int32, device="cuda")
    ms = timer(lambda i: B.wq_read_probe(bufs[i % ncopy], nb, sink), steps, warmup, ncopy)
    del bufs
    return nb / (ms * 1e-3) / 1e9


def gemv_workload(a, torch, L, label, timer):
    import bit_weight_only_gemv_amd as B
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    t0 = time.time()
    hl = pack_host(L.fmt, L.W, L.profile, L.ratio)
    pack_s = time.time() - t0
    base = DeviceLayer(hl, tiled=True)
    nbytes = base.nbytes(1)
    layers = rotated(DeviceLayer, base, nbytes)
    ncopy = len(layers)
    x = torch.from_numpy(L.x.reshape(-1).view(np.int16)).cuda()
    ys = [torch.empty(base.N, dtype=torch.int16, device="cuda") for _ in range(ncopy)]
    torch.cuda.synchronize()

    def step_rowmajor(i):
        layers[i % ncopy].gemv(x, ys[i % ncopy])

    def step_tiled(i):
        layers[i % ncopy].gemv_tiled(x, ys[i % ncopy])

    steps = {"rowmajor": step_rowmajor, "tiled": step_tiled}
    times = {k: timer(fn, a.steps, a.warmup, ncopy) for k, fn in steps.items()}
    layout = min(times, key=times.get) if a.layout == "best" else a.layout
    other = "rowmajor" if layout == "tiled" else "tiled"
    ms, ms_other = times[layout], times[other]
    gbs = nbytes / (ms * 1e-3) / 1e9
    bpt = sweep_bytes_per_token(L.fmt, L.ratio)
    traffic = traffic_for(f"{label}_{layout}")
    del layers
    probe = read_probe_rate(torch, timer, nbytes, a.steps, a.warmup)
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded Gaussian weights and activations; no checkpoint)",
        "config": {"workload": label, "N": base.N, "K": base.K, "M": 1, "n_out": base.n_out,
                   "format": {4: "W4", 2: "W2", 5: "W4P (packed zero points)"}[L.fmt] + " group-32",
                   "accumulate": "f32",
                   "bytes_per_step": nbytes, "rotated_copies": ncopy, "layout": layout,
                   "timing": "eager launches" if a.eager else "hip graph replay"},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "attainable": {"read_probe_GB/s": round(probe, 1),
                       "pct_of_read_probe": round(100 * gbs / probe, 2),
                       "about": "a plain streaming read of the same bytes per launch, rotated "
                                "and graph-replayed in the same run"},
        "eq_tokens_per_s": round(gbs * 1e9 / bpt, 1),
        "eq_tokens_basis_bytes_per_token": bpt,
        "host_pack_s": round(pack_s, 2),
        f"{other}_layout": {"us": round(ms_other * 1e3, 3),
                            "GB/s": round(nbytes / (ms_other * 1e-3) / 1e9, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(L, nbytes)
    return out


SWEEP_GROUPS = {
    # one GEMV per projection: 7 per layer + the LM head = 225 per token
    "unfused": [("q",), ("k",), ("v",), ("o",), ("gate",), ("up",), ("down",)],
    # projections that read the same activation stacked along N into one GEMV
    # (q|k|v 6144 x 4096, gate|up 28672 x 4096): 4 per layer + the head = 129
    "fused": [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)],
}


def _with_fmt(L, fmt):
    import dataclasses
    return dataclasses.replace(L, fmt=fmt)


def w4_fmt(a) -> int:
    return 5 if a.w4_zeros == "packed" else 4


def sweep_workload(a, torch, timer):
    """One Llama-3-8B-shaped W4 decode step per graph replay, two ways:
    225 separate GEMVs, and 129 GEMVs with q|k|v and gate|up stacked along N
    (same weights, same bytes, fewer launches).  Each group of GEMVs runs on
    the layout (row-major or tiled) measured faster for it over its 32 layers;
    tokens_per_s is the fused step's rate."""
    import synthetic
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    shapes = synthetic.config3_shapes()
    nlayers = shapes[-1][0]
    proj = {}
    for (layer, p, name, N, K) in shapes:
        if layer == 0:
            proj[name] = (p, N, K)
    head = shapes[-1]
    protos = {}
    for groups in SWEEP_GROUPS.values():
        for g in groups:
            if g not in protos:
                Ws = [synthetic.config3_layer(0, proj[n][0], proj[n][1], proj[n][2], n).W for n in g]
                protos[g] = DeviceLayer(pack_host(w4_fmt(a), np.concatenate(Ws, axis=0)), tiled=True)
    hL = synthetic.config3_layer(head[0], head[1], head[3], head[4], head[2])
    head_layer = DeviceLayer(pack_host(w4_fmt(a), hL.W), tiled=True)
    torch.cuda.synchronize()
    steps = max(1, min(a.steps, 50))
    out = {"workload": "w4_llama3_8b_decode_step" + ("_w4p" if w4_fmt(a) == 5 else ""),
           "steps": steps}
    for label, groups in SWEEP_GROUPS.items():
        layers = {g: [protos[g]] + [clone_layer(DeviceLayer, protos[g]) for _ in range(nlayers - 1)]
                  for g in groups}
        xs = {g: torch.from_numpy(synthetic.gaussian_x_fp16(1, protos[g].K, 3, 0, i).reshape(-1)
                                  .view(np.int16)).cuda() for i, g in enumerate(groups)}
        ys = {g: torch.empty(protos[g].N, dtype=torch.int16, device="cuda") for g in groups}
        xh = torch.from_numpy(hL.x.reshape(-1).view(np.int16)).cuda()
        yh = torch.empty(head_layer.N, dtype=torch.int16, device="cuda")
        # layout per group: the faster one over the group's 32 (cold) layers
        pick = {}
        for g in list(groups) + ["head"]:
            ls = [head_layer] if g == "head" else layers[g]
            x, y = (xh, yh) if g == "head" else (xs[g], ys[g])
            t = {}
            for lay in ("rowmajor", "tiled"):
                def run(i, ls=ls, x=x, y=y, lay=lay):
                    for d in ls:
                        (d.gemv_tiled if lay == "tiled" else d.gemv)(x, y)
                t[lay] = timer(run, 5, 2)
            pick[g] = min(t, key=t.get)
        calls = []
        for li in range(nlayers):
            for g in groups:
                d = layers[g][li]
                calls.append((d.gemv_tiled if pick[g] == "tiled" else d.gemv, xs[g], ys[g]))
        calls.append((head_layer.gemv_tiled if pick["head"] == "tiled" else head_layer.gemv, xh, yh))
        total = sum(layers[g][0].nbytes(1) for g in groups) * nlayers + head_layer.nbytes(1)

        def step(i, calls=calls):
            for fn, x, y in calls:
                fn(x, y)

        ms = timer(step, steps, min(a.warmup, 5))
        out[label] = {"gemvs_per_token": len(calls), "ms_per_token": round(ms, 4),
                      "tokens_per_s": round(1e3 / ms, 1), "bytes_per_token": total,
                      "GB/s": round(total / (ms * 1e-3) / 1e9, 1),
                      "layouts": {("|".join(g) if g != "head" else g): pick[g] for g in pick}}
        del layers, calls
        torch.cuda.synchronize()
    best = out["fused"]
    out.update({"ms_per_token": best["ms_per_token"], "tokens_per_s": best["tokens_per_s"],
                "pct_of_hbm_peak": round(100 * best["GB/s"] / HBM_PEAK_GBS, 2),
                "roofline_tokens_per_s": round(HBM_PEAK_GBS * 1e9 / best["bytes_per_token"], 1)})
    return out


def batched_workload(a, torch, timer):
    """Small-M products (SPECTRA section 4.2) on the W4 14336 x 4096 and
    4096 x 14336 layers: the tiled layout's batched kernel (the same buffer as
    the M = 1 kernel), the row-major arrays' batched kernel, M repeated GEMVs,
    and the tiled M = 1 GEMV of the same layer in the same run."""
    import synthetic
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    rows = []
    shapes = [(14336, 4096), (4096, 14336)]
    if a.shape:
        shapes = [tuple(int(v) for v in a.shape.lower().split("x"))]
    for (N, K) in shapes:
        Lb = synthetic.config4(16, N, K)
        base = DeviceLayer(pack_host(w4_fmt(a), Lb.W), tiled=True)
        n1 = base.nbytes(1)
        l1 = rotated(DeviceLayer, base, n1)
        x1 = torch.from_numpy(np.ascontiguousarray(Lb.x[0]).view(np.int16)).cuda()
        y1 = [torch.empty(N, dtype=torch.int16, device="cuda") for _ in range(len(l1))]
        ms_m1 = timer(lambda i: l1[i % len(l1)].gemv_tiled(x1, y1[i % len(l1)]), a.steps // 4,
                      a.warmup // 4, len(l1))
        del l1
        for M in ((a.m,) if a.m else (2, 4, 8, 16)):
            nbytes = base.nbytes(M)
            layers = rotated(DeviceLayer, base, nbytes)
            nc = len(layers)
            X = torch.from_numpy(np.ascontiguousarray(Lb.x[:M]).view(np.int16)).cuda()
            Y = [torch.empty((M, N), dtype=torch.int16, device="cuda") for _ in range(nc)]
            xrow = [X[m].contiguous() for m in range(M)]
            ms_tiled = timer(lambda i: layers[i % nc].gemm_tiled(X, Y[i % nc]), a.steps // 4,
                             a.warmup // 4, nc)
            ms_gemm = timer(lambda i: layers[i % nc].gemm(X, Y[i % nc]), a.steps // 4, a.warmup // 4, nc)

            def rep(i):
                for m in range(M):
                    layers[i % nc].gemv(xrow[m], Y[i % nc][m])
            ms_rep = timer(rep, max(1, a.steps // (4 * M)), max(1, a.warmup // (4 * M)), nc)
            flops = 2.0 * M * N * K
            rows.append({"workload": f"w{'4p' if w4_fmt(a) == 5 else '4'}_{N}x{K}_m{M}",
                         "bytes": nbytes,
                         "tiled_us": round(ms_tiled * 1e3, 3),
                         "tiled_GB/s": round(nbytes / (ms_tiled * 1e-3) / 1e9, 1),
                         "tiled_over_m1": round(ms_tiled / ms_m1, 3),
                         "m1_tiled_us": round(ms_m1 * 1e3, 3),
                         "rowmajor_us": round(ms_gemm * 1e3, 3),
                         "rowmajor_GB/s": round(nbytes / (ms_gemm * 1e-3) / 1e9, 1),
                         "TFLOP/s": round(flops / (min(ms_tiled, ms_gemm) * 1e-3) / 1e12, 2),
                         "repeated_gemv_us": round(ms_rep * 1e3, 3)})
            del layers
    return rows


def w2_70b_workload(a, torch, timer):
    import synthetic
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    rows = []
    for (N, K) in ((28672, 8192), (8192, 28672)):
        L8 = synthetic.config5(N, K, 8)
        base = DeviceLayer(pack_host(2, L8.W, L8.profile, L8.ratio), tiled=True)
        for M, layout in ((1, "rowmajor"), (1, "tiled"), (8, "rowmajor"), (8, "tiled")):
            nbytes = base.nbytes(M)
            layers = rotated(DeviceLayer, base, nbytes)
            nc = len(layers)
            X = torch.from_numpy(np.ascontiguousarray(L8.x[:M]).view(np.int16)).cuda()
            Y = [torch.empty((M, N), dtype=torch.int16, device="cuda") for _ in range(nc)]
            if M == 1 and layout == "tiled":
                fn = lambda i: layers[i % nc].gemv_tiled(X[0], Y[i % nc][0])  # noqa: E731
            elif M == 1:
                fn = lambda i: layers[i % nc].gemv(X[0], Y[i % nc][0])  # noqa: E731
            elif layout == "tiled":
                fn = lambda i: layers[i % nc].gemm_tiled(X, Y[i % nc])  # noqa: E731
            else:
                fn = lambda i: layers[i % nc].gemm(X, Y[i % nc])  # noqa: E731
            ms = timer(fn, a.steps // 4, a.warmup // 4, nc)
            rows.append({"workload": f"w2_{N}x{K}_outliers{base.n_out}_m{M}", "layout": layout,
                         "bytes": nbytes, "us": round(ms * 1e3, 3),
                         "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "pct_of_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)})
            del layers
    return rows


def embed_workload(a, torch, timer):
    """Embedding row gather (SPECTRA section 4.3) from a W4 (or W4P) table of
    131072 x 4096 (the page's example vocabulary): n_ids uniformly drawn token
    ids per launch, a fresh id set each launch (rotated), rows dequantized
    straight into FP16 output rows.  Bytes = the gathered rows' codes, scales,
    zeros and ids read plus the FP16 rows written."""
    import synthetic
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    V, K = 131072, 4096
    fmt = w4_fmt(a)
    W = synthetic.gaussian_weights(V, K, 0.02, 6, 0, fmt)
    dl = DeviceLayer(pack_host(fmt, W))
    del W
    G = K // 32
    zrow = (G + 1) // 2 if fmt == 5 else 2 * G
    rows = []
    for n_ids in (1, 64, 4096):
        nsets = 64
        rng = np.random.default_rng(n_ids)
        ids = [torch.from_numpy(rng.integers(0, V, n_ids).astype(np.int32)).cuda()
               for _ in range(nsets)]
        outs = [torch.empty((n_ids, K), dtype=torch.int16, device="cuda") for _ in range(4)]
        fn = lambda i: dl.embed(ids[i % nsets], outs[i % 4])  # noqa: E731
        ms = timer(fn, a.steps // 4, a.warmup // 4, nsets)
        nbytes = n_ids * (K // 2 + 2 * G + zrow + 4) + n_ids * K * 2
        rows.append({"workload": f"embed_gather_{V}x{K}_w{'4p' if fmt == 5 else '4'}_ids{n_ids}",
                     "bytes": nbytes, "us": round(ms * 1e3, 3),
                     "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "pct_of_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)})
    return rows


def kurtosis_workload(a, torch, timer):
    """The kurtosis-adaptive outlier policy (SPECTRA sections 3.1-3.3) on the W2
    layers of the other workloads: kappa, the ratio and n_out it picks (host
    time), and the tiled W2 GEMV with those outliers next to the profile-guided
    3.5% of the default workloads."""
    import synthetic
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    import bit_weight_only_gemv_amd as B
    rows = []
    for label, L in (("w2_14336x4096", synthetic.config2()),
                     ("w2_28672x8192", synthetic.config5(28672, 8192, 1))):
        t0 = time.time()
        idx, r, kappa = B.wq_select_outliers_kurtosis(L.W)
        t_sel = time.time() - t0
        row = {"workload": f"kurtosis_policy_{label}", "kappa": round(kappa, 4), "ratio": round(r, 5),
               "n_out": int(len(idx)), "host_select_s": round(t_sel, 3)}
        for pol in ("kurtosis", "profile_3.5pct"):
            hl = pack_host(2, L.W, kurtosis=True) if pol == "kurtosis" else \
                pack_host(2, L.W, L.profile, L.ratio)
            base = DeviceLayer(hl, tiled=True)
            nbytes = base.nbytes(1)
            layers = rotated(DeviceLayer, base, nbytes)
            nc = len(layers)
            x = torch.from_numpy(L.x[:1].reshape(-1).view(np.int16)).cuda()
            ys = [torch.empty(base.N, dtype=torch.int16, device="cuda") for _ in range(nc)]
            ms = timer(lambda i: layers[i % nc].gemv_tiled(x, ys[i % nc]), a.steps // 4,
                       a.warmup // 4, nc)
            row[pol] = {"n_out": base.n_out, "bytes": nbytes, "us": round(ms * 1e3, 3),
                        "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
            del layers
        rows.append(row)
    return rows


def refine_workload(a, torch, timer):
    """Runtime top-k refinement (StrataFlux section 3.2.1, Eq. 2) after the tiled
    GEMV: per 1024-channel chunk the k = 32 largest |x_i| are selected on the GPU
    and their 4-bit residual columns added to y.  Each launch times the
    selection, the add, the GEMV, the three in sequence, and the GEMV with the
    selection and the add in the same launch; the layer and its
    refinement columns are rotated like the GEMV's.  Refinement bytes = the
    selected columns' codes, scales and zeros, the indices and x entries read,
    and y read and written."""
    import synthetic
    import bit_weight_only_gemv_amd as B
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host, refinement_host
    rows = []
    k, chunk = 32, 1024
    for label, L in (("w2_14336x4096_outliers143", synthetic.config2()),
                     ("w4_4096x14336", synthetic.config3_layer(0, 6, 4096, 14336, "down"))):
        hl = pack_host(L.fmt, L.W, L.profile, L.ratio)
        rf = refinement_host(L.W, hl)
        base = DeviceLayer(hl, tiled=True)
        base.set_refinement(rf)
        nbytes = base.nbytes(1)
        rbytes_table = base.r_codes.numel() + 2 * base.r_scales.numel() + 2 * base.r_zeros.numel()
        layers = rotated(DeviceLayer, base, nbytes + rbytes_table)
        for c in layers[1:]:
            c.r_codes, c.r_scales, c.r_zeros = (base.r_codes.clone(), base.r_scales.clone(),
                                                base.r_zeros.clone())
        nc = len(layers)
        N, K = base.N, base.K
        n_sel = B.wq_topk_count(K, chunk, k)
        x = torch.from_numpy(L.x[:1].reshape(-1).view(np.int16)).cuda()
        ys = [torch.empty(N, dtype=torch.int16, device="cuda") for _ in range(nc)]
        sels = [torch.empty(n_sel, dtype=torch.int32, device="cuda") for _ in range(nc)]
        for i in range(nc):
            B.wq_topk_chunks(x, K, chunk, k, sels[i])
        st = a.steps // 4
        wu = a.warmup // 4
        t_topk = timer(lambda i: B.wq_topk_chunks(x, K, chunk, k, sels[i % nc]), st, wu, nc)
        t_ref = timer(lambda i: layers[i % nc].refine(x, ys[i % nc], sels[i % nc], n_sel), st, wu, nc)
        t_gemv = timer(lambda i: layers[i % nc].gemv_tiled(x, ys[i % nc]), st, wu, nc)

        def chain(i):
            lay, y, sel = layers[i % nc], ys[i % nc], sels[i % nc]
            lay.gemv_tiled(x, y)
            B.wq_topk_chunks(x, K, chunk, k, sel)
            lay.refine(x, y, sel, n_sel)

        t_all = timer(chain, st, wu, nc)
        t_fused = timer(lambda i: layers[i % nc].refine_topk(x, ys[i % nc], k, chunk), st, wu, nc)
        # the same call given a selection buffer (two kernels past 8 chunks)
        t_call = timer(lambda i: layers[i % nc].refine_topk(x, ys[i % nc], k, chunk, sels[i % nc]),
                       st, wu, nc)

        def chain_fused(i):
            layers[i % nc].gemv_tiled(x, ys[i % nc])
            layers[i % nc].refine_topk(x, ys[i % nc], k, chunk)

        t_all_fused = timer(chain_fused, st, wu, nc)

        def chain_call(i):
            layers[i % nc].gemv_tiled(x, ys[i % nc])
            layers[i % nc].refine_topk(x, ys[i % nc], k, chunk, sels[i % nc])

        t_all_call = timer(chain_call, st, wu, nc)
        # the product with the selection and the add in the same launch
        t_one = timer(lambda i: layers[i % nc].gemv_tiled_refine(x, ys[i % nc], k, chunk), st, wu, nc)
        Gn = N // 32
        rbytes = n_sel * (N // 2 + 4 * Gn) + 4 * n_sel + 2 * n_sel + 4 * N
        rows.append({"workload": f"refine_topk{k}_per{chunk}_{label}", "N": N, "K": K,
                     "n_sel": n_sel, "topk_us": round(t_topk * 1e3, 3),
                     "refine_us": round(t_ref * 1e3, 3), "refine_bytes": rbytes,
                     "refine_GB/s": round(rbytes / (t_ref * 1e-3) / 1e9, 1),
                     "gemv_us": round(t_gemv * 1e3, 3),
                     "fused_topk_refine_us": round(t_fused * 1e3, 3),
                     "gemv_topk_refine_us": round(t_all * 1e3, 3),
                     "gemv_fused_refine_us": round(t_all_fused * 1e3, 3),
                     "refine_topk_with_sel_out_us": round(t_call * 1e3, 3),
                     "gemv_refine_topk_with_sel_out_us": round(t_all_call * 1e3, 3),
                     "two_launch_overhead_pct": round(100 * (t_all_call - t_gemv) / t_gemv, 1),
                     "gemv_refine_one_launch_us": round(t_one * 1e3, 3),
                     "one_launch_overhead_pct": round(100 * (t_one - t_gemv) / t_gemv, 1)})
        del layers
    return rows


def stream_workload(a, torch, timer, copy):
    import bit_weight_only_gemv_amd as B
    nb = (a.bytes + 15) // 16 * 16
    ncopy = max(1, -(-ROTATE_BYTES // nb))
    bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
    if copy:
        dsts = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
        fn = lambda i: B.wq_copy_probe(bufs[i % ncopy], dsts[i % ncopy], nb)  # noqa: E731
    else:
        sink = torch.empty(B.wq_read_probe_sink_words(nb), dtype=torch.int32, device="cuda")
        fn = lambda i: B.wq_read_probe(bufs[i % ncopy], nb, sink)  # noqa: E731
    ms = timer(fn, a.steps, a.warmup, ncopy)
    moved = nb * (2 if copy else 1)
    return {"workload": "copy_probe" if copy else "read_probe", "bytes": nb, "copies": ncopy,
            "us": round(ms * 1e3, 3), "GB/s": round(moved / (ms * 1e-3) / 1e9, 1)}


def probe_sweep_workload(a, torch, timer):
    """The attainable streaming-read rate per launch at the layers' sizes: the
    geometry-swept read kernel (workgroups x threads x loads in flight per
    lane; each wave reads one contiguous run) over rotated buffers, every
    geometry timed like the GEMV.  One line per size, with the best geometry
    and the whole table."""
    import bit_weight_only_gemv_amd as B
    rows = []
    sizes = [int(v) for v in a.probe_sizes.split(",")] if a.probe_sizes else \
        [26157628, 10502144, 104555640, 37289984]
    for nbytes in sizes:
        nb = (nbytes + 15) // 16 * 16
        ncopy = max(1, -(-ROTATE_BYTES // nb))
        bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
        sink = torch.empty(65536, dtype=torch.int32, device="cuda")
        table = []
        for blocks in (256, 512, 768, 1024, 2048, 4096):
            for threads in (256, 512, 1024):
                waves = blocks * threads // 64
                span_kb = -(-nb // 1024 // waves)
                for ring in (1, 2, 4, 8, 16):
                    if ring > 2 * max(1, span_kb):
                        continue
                    ms = timer(lambda i: B.wq_read_probe_geom(bufs[i % ncopy], nb, sink, blocks,
                                                               threads, ring),
                               max(ncopy, a.steps // 10), max(ncopy, a.warmup // 10), ncopy)
                    table.append({"blocks": blocks, "threads": threads, "ring": ring,
                                  "span_kb": span_kb, "us": round(ms * 1e3, 3),
                                  "GB/s": round(nb / (ms * 1e-3) / 1e9, 1)})
        ms = timer(lambda i: B.wq_read_probe(bufs[i % ncopy], nb, sink[:B.wq_read_probe_sink_words(nb)]),
                   max(ncopy, a.steps // 10), max(ncopy, a.warmup // 10), ncopy)
        best = min(table, key=lambda r: r["us"])
        rows.append({"workload": f"read_probe_sweep_{nb}B", "bytes": nb, "copies": ncopy,
                     "best": best, "pct_of_hbm_peak": round(best["GB/s"] / HBM_PEAK_GBS * 100, 2),
                     "grid_stride_probe": {"us": round(ms * 1e3, 3),
                                           "GB/s": round(nb / (ms * 1e-3) / 1e9, 1)},
                     "table": sorted(table, key=lambda r: r["us"])[:25]})
        del bufs
        torch.cuda.synchronize()
    return rows


def cpu_baseline(L, nbytes):
    """The oracle, as it stands, on the same layer: dequantization of the packed
    weights followed by the float64 product (median of 3)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    ref = O.quantize_layer(L.fmt, L.W, L.profile, L.ratio)
    times, t_deq, t_mv = [], [], []
    for _ in range(3):
        t0 = time.perf_counter()
        w_hat = ref.w_hat()
        t1 = time.perf_counter()
        O.matvec_ref(w_hat, L.x, ref.idx, ref.wout)
        t2 = time.perf_counter()
        times.append(t2 - t0)
        t_deq.append(t1 - t0)
        t_mv.append(t2 - t1)
    t = float(np.median(times))
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                       "unknown")
    except OSError:
        pass
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "dequant_s": round(float(np.median(t_deq)), 3),
            "matvec_s": round(float(np.median(t_mv)), 3),
            "cpu_model": cpu,
            "sample": (f"the whole {ref.N}x{ref.K} layer: oracle dequantization + float64 product, "
                       f"median of 3 runs ({t:.2f} s each); numpy elementwise work is single-threaded, "
                       f"the BLAS product used {blas_threads} threads of "
                       f"{len(os.sched_getaffinity(0))} host cores")}


def main():
    a = _parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): the path is a "
              "single-GPU kernel; sharding across GPUs is described, not built.", file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import torch
    import synthetic
    import bit_weight_only_gemv_amd as B

    B.load()
    torch.cuda.init()
    timer = Timer(torch, eager=a.eager)
    if a.workload == "w2_14336":
        out = gemv_workload(a, torch, synthetic.config2(), "w2_14336x4096_outliers143_m1", timer)
    elif a.workload == "w4_4096":
        L1 = synthetic.config1()
        if a.w4_zeros == "packed":
            L1 = _with_fmt(L1, 5)
        out = gemv_workload(a, torch, L1, "w4_4096x4096_m1" + ("_w4p" if L1.fmt == 5 else ""), timer)
    elif a.workload == "sweep":
        out = sweep_workload(a, torch, timer)
    elif a.workload == "batched":
        out = batched_workload(a, torch, timer)
    elif a.workload == "w2_70b":
        out = w2_70b_workload(a, torch, timer)
    elif a.workload == "embed":
        out = embed_workload(a, torch, timer)
    elif a.workload == "kurtosis":
        out = kurtosis_workload(a, torch, timer)
    elif a.workload == "refine":
        out = refine_workload(a, torch, timer)
    elif a.workload == "probe_sweep":
        out = probe_sweep_workload(a, torch, timer)
    else:
        out = stream_workload(a, torch, timer, copy=(a.workload == "copy"))
    for o in (out if isinstance(out, list) else [out]):
        print(json.dumps(o), flush=True)


if __name__ == "__main__":
    main()
