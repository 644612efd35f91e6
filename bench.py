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
* exactly --steps launches are timed: captured into HIP graphs (the kernels
  are launched through the library's C ABI during capture) and replayed, with
  hipEvents on the replay stream between replays (median and 10th / 90th
  percentiles over the replays); --eager times Python-side launches instead;
* value = algorithmic bytes per step (codes + FP16 scales + FP16 zeros + FP16
  outlier slab + int32 indices + x + y) / median time per step;
* every line carries `roofline` (achieved rate against MI355X's published
  peak, plus HBM bytes per launch from rocprofv3 counters where they were taken
  on the current kernel sources) and `cpu_baseline` (the CPU oracle timed on
  the host on the same layer, or a stated sample of it).

Other workloads (--workload): w4_4096 (W4 4096x4096), sweep (Llama-3-8B-shaped
decode in one graph -> tokens/s: 225 separate W4 GEMVs per token, and 129 with
q|k|v and gate|up stacked along N), batched (W4 small-M products on both
layouts vs M repeated GEMVs), w2_70b (W2 + outliers at 28672x8192 and
8192x28672, M = 1 and 8), embed (row gather from a 131072 x 4096 W4 table),
kurtosis (the kurtosis-adaptive outlier policy on the W2 layers), refine
(runtime top-k refinement), read / copy (plain streaming kernels: the
attainable HBM rate and the byte-counter calibration), probe_sweep (the read
probe's launch geometries at the layers' sizes).
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
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16 matrix cores, published
ROTATE_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["wq_gemv.hip", "wq_mma.hip", "wq_mma.h", "wq_common.cuh", "wq_device.h",
                  "wq_select.cuh"]
DATA = "synthetic (seeded Gaussian weights and activations; no checkpoint)"


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
    """Hash of the kernels' code with comments and layout removed, so that
    counters stay attached to the code they were taken on and survive edits of
    comments only."""
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


class Timing(float):
    """Milliseconds per step (the median over replays) with the spread."""

    def __new__(cls, median, p10, p90, mean, steps):
        o = super().__new__(cls, median)
        o.p10, o.p90, o.mean, o.steps = p10, p90, mean, steps
        return o

    def us(self):
        return {"median": round(self * 1e3, 3), "p10": round(self.p10 * 1e3, 3),
                "p90": round(self.p90 * 1e3, 3), "mean": round(self.mean * 1e3, 3)}


class Timer:
    """Times exactly `steps` calls of fn(i) after `warmup` untimed ones.  The
    steps are captured into a HIP graph of `per` launches (the library is
    called through its C ABI during capture), a whole multiple of `period` (the
    number of rotated buffer copies, so that every replay walks all of them),
    replayed R times with an event on the launching stream between replays; a
    second graph holds the steps - R per left over.  Before the timed replays
    the first graph is replayed back to back for WARM_S seconds (the clocks
    ramp down while the host prepares a workload).  A bounded spin on the
    stream (about 0.1 ms) comes first, so that the launches are queued on the
    GPU before the first event fires and the timed region holds the kernels,
    not the host's latency to submit the first of them.  One synchronization
    ends the timed region.  Returns a Timing."""

    REPLAYS = 20
    LEAD_CYCLES = 250_000
    WARM_S = 0.05     # graph replays before the timed ones, at least this long

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
            # the GPU's clocks drop while the host prepares a workload: replay
            # the graph back to back for WARM_S first, so that the timed
            # replays do not include the ramp
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < self.WARM_S:
                for _ in range(4):
                    g_main.replay()
                torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
        torch.cuda.synchronize()
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


def gbs(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def roofline_hbm(nbytes, ms, traffic=None):
    g = gbs(nbytes, ms)
    return {"bound": "hbm", "achieved": round(g, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(g / HBM_PEAK_GBS, 4), "traffic": traffic}


def line(metric, value, unit, a, ms, config, roofline, **extra):
    """One JSON record in the shape every workload line shares."""
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": float(ms), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": DATA,
           "config": config}
    if isinstance(ms, Timing):
        out["timing_us"] = ms.us()
    out["roofline"] = roofline
    out.update(extra)
    return out


ATTAINABLE_GEOMETRIES = ((0, 256, 1), (0, 256, 2), (0, 256, 4))


def attainable_read(torch, timer, nbytes, steps, warmup):
    """The attainable streaming-read rate at this many bytes per launch: the
    one-shot grid-stride read kernel at the geometries that measured fastest
    at the layers' sizes (256-thread workgroups, 1, 2 or 4 loads in flight per
    lane), over rotated buffers, timed like the GEMV; the best one (GB/s)."""
    import bit_weight_only_gemv_amd as B
    nb = (nbytes + 15) // 16 * 16
    ncopy = max(1, -(-ROTATE_BYTES // nb))
    bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
    sink = torch.empty(65536, dtype=torch.int32, device="cuda")
    best = None
    for blocks, threads, ring in ATTAINABLE_GEOMETRIES:
        ms = timer(lambda i: B.wq_read_probe_geom(bufs[i % ncopy], nb, sink, blocks, threads, ring),
                   max(steps, ncopy), max(warmup, ncopy), ncopy)
        rate = gbs(nb, ms)
        if best is None or rate > best[0]:
            best = (rate, {"blocks": "one-shot", "threads": threads, "loads_in_flight": ring})
    del bufs
    return best


# ------------------------------------------------------------ CPU baseline


def host_info():
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                       "unknown")
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return {"cores": len(os.sched_getaffinity(0)), "blas_threads": int(blas), "cpu_model": cpu}


def oracle_times(ref, X, runs, min_s=0.0):
    """Wall times of the oracle's dequantization and float64 product of one
    packed layer against X (median of `runs`, or of as many runs as fill
    `min_s` seconds)."""
    import oracle as O
    t_deq, t_mv = [], []
    t_start = time.perf_counter()
    while len(t_deq) < runs or time.perf_counter() - t_start < min_s:
        t0 = time.perf_counter()
        w_hat = ref.w_hat()
        t1 = time.perf_counter()
        O.matvec_ref(w_hat, X, ref.idx, ref.wout)
        t2 = time.perf_counter()
        t_deq.append(t1 - t0)
        t_mv.append(t2 - t1)
    return float(np.median(t_deq)), float(np.median(t_mv))


def cpu_baseline_rate(value, unit, t_deq, t_mv, sample, **extra):
    info = host_info()
    out = {"value": value, "unit": unit, "cores": info["cores"], "kind": "oracle",
           "blas_threads": info["blas_threads"], "dequant_s": round(t_deq, 3),
           "matvec_s": round(t_mv, 3), "cpu_model": info["cpu_model"],
           "sample": sample + (f"; numpy elementwise work is single-threaded, the BLAS product "
                               f"used {info['blas_threads']} threads of {info['cores']} host cores")}
    out.update(extra)
    return out


def cpu_baseline_layer(ref, X, nbytes, runs=3, what="the whole layer"):
    """The oracle, as it stands, on the same packed layer and activations:
    dequantization followed by the float64 product; rate in the same
    algorithmic bytes as the GPU line."""
    t_deq, t_mv = oracle_times(ref, X, runs)
    t = t_deq + t_mv
    return cpu_baseline_rate(round(nbytes / t / 1e9, 4), "GB/s", t_deq, t_mv,
                             f"{what} ({ref.N}x{ref.K}, M={np.atleast_2d(X).shape[0]}): oracle "
                             f"dequantization + float64 product, median of {runs} runs "
                             f"({t:.2f} s each)")


# ---------------------------------------------------------------- workloads


FMT_NAME = {4: "W4", 2: "W2", 5: "W4P (packed zero points)"}


def gemv_workload(a, torch, L, label, timer):
    """The M = 1 fused GEMV of one layer on both layouts (tiled and row-major);
    `value` is the faster one unless --layout says which."""
    import bit_weight_only_gemv_amd as B  # noqa: F401
    import oracle as O
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
    g = gbs(nbytes, ms)
    bpt = sweep_bytes_per_token(L.fmt, L.ratio)
    del layers
    probe, geom = attainable_read(torch, timer, nbytes, max(a.steps // 4, 1), max(a.warmup // 4, 1))
    out = line(METRIC, round(g, 2), "GB/s", a, ms,
               {"workload": label, "N": base.N, "K": base.K, "M": 1, "n_out": base.n_out,
                "format": FMT_NAME[L.fmt] + " group-32", "accumulate": "f32",
                "bytes_per_step": nbytes, "rotated_copies": ncopy, "layout": layout,
                "timing": "eager launches" if a.eager else "hip graph replay"},
               roofline_hbm(nbytes, ms, traffic_for(f"{label}_{layout}")),
               pct_of_hbm_peak=round(100 * g / HBM_PEAK_GBS, 2),
               attainable={"read_probe_GB/s": round(probe, 1),
                           "pct_of_read_probe": round(100 * g / probe, 2),
                           "read_probe_geometry": geom,
                           "about": "the best of the one-shot grid-stride read kernels over the "
                                    "same bytes per launch, rotated and graph-replayed in the "
                                    "same run"},
               eq_tokens_per_s=round(g * 1e9 / bpt, 1),
               eq_tokens_basis_bytes_per_token=bpt,
               host_pack_s=round(pack_s, 2))
    out[f"{other}_layout"] = {"us": round(ms_other * 1e3, 3), "GB/s": round(gbs(nbytes, ms_other), 2),
                              "timing_us": ms_other.us()}
    if not a.no_cpu_baseline:
        ref = O.quantize_layer(L.fmt, L.W, L.profile, L.ratio)
        out["cpu_baseline"] = cpu_baseline_layer(ref, L.x, nbytes)
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


def sweep_cpu_baseline(fmt, bytes_per_token):
    """The oracle on a bounded sample of the decode step: the 7 GEMVs of the
    first layer (their own weights and activations), dequantization + float64
    product, scaled to tokens/s by bytes."""
    import oracle as O
    import synthetic
    shapes = [s for s in synthetic.config3_shapes() if s[0] == 0]
    t_deq = t_mv = 0.0
    nb = 0
    for (layer, p, name, N, K) in shapes:
        L = synthetic.config3_layer(layer, p, N, K, name)
        ref = O.quantize_layer(fmt, L.W)
        d, m = oracle_times(ref, L.x, 1)
        t_deq += d
        t_mv += m
        G = K // 32
        nb += N * K // 2 + 2 * N * G + (N * ((G + 1) // 2) if fmt == 5 else 2 * N * G) + 2 * K + 2 * N
    t = t_deq + t_mv
    tps = (nb / t) / bytes_per_token
    return cpu_baseline_rate(round(tps, 4), "tokens/s", t_deq, t_mv,
                             f"the 7 GEMVs of the first layer ({nb / 1e6:.0f} MB of the "
                             f"{bytes_per_token / 1e9:.2f} GB per token), oracle dequantization "
                             f"+ float64 product in {t:.2f} s, scaled to a whole token by bytes",
                             GB_per_s=round(nb / t / 1e9, 4))


def sweep_workload(a, torch, timer):
    """One Llama-3-8B-shaped W4 decode step per graph replay, two ways:
    225 separate GEMVs, and 129 GEMVs with q|k|v and gate|up stacked along N
    (same weights, same bytes, fewer launches).  Each group of GEMVs runs on
    the layout (row-major or tiled) measured faster for it over its 32 layers;
    `value` is the stacked step's rate in tokens/s."""
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
    res = {}
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
        reads = []   # the buffer each GEMV streams (its tiled copy: codes and metadata)
        for li in range(nlayers):
            for g in groups:
                d = layers[g][li]
                calls.append((d.gemv_tiled if pick[g] == "tiled" else d.gemv, xs[g], ys[g]))
                reads.append(d.tiled)
        calls.append((head_layer.gemv_tiled if pick["head"] == "tiled" else head_layer.gemv, xh, yh))
        reads.append(head_layer.tiled)
        total = sum(layers[g][0].nbytes(1) for g in groups) * nlayers + head_layer.nbytes(1)

        def step(i, calls=calls):
            for fn, x, y in calls:
                fn(x, y)

        ms = timer(step, steps, min(a.warmup, 5))
        res[label] = {"gemvs_per_token": len(calls), "ms_per_token": round(ms, 4),
                      "tokens_per_s": round(1e3 / ms, 1), "bytes_per_token": total,
                      "GB/s": round(gbs(total, ms), 1), "timing_us": ms.us(), "ms": ms,
                      "layouts": {("|".join(g) if g != "head" else g): pick[g] for g in pick}}
        if label == "fused":
            # The same launch sequence with each GEMV replaced by the one-shot
            # read kernel over that GEMV's weight buffer: the rate a step of
            # these launches reaches when it only streams the bytes.
            import bit_weight_only_gemv_amd as B
            sink = torch.empty(65536, dtype=torch.int32, device="cuda")
            blocks, threads, ring = ATTAINABLE_GEOMETRIES[0]

            def read_step(i, reads=reads):
                for buf in reads:
                    nb = buf.numel() // 16 * 16
                    # one-shot up to 65536 workgroups (268 MB); past that the
                    # same kernel strides over the buffer with 65536
                    bl = blocks if nb <= 65536 * threads * 16 * ring else 65536
                    B.wq_read_probe_geom(buf, nb, sink, bl, threads, ring)

            ms_r = timer(read_step, steps, min(a.warmup, 5))
            rbytes = sum(buf.numel() // 16 * 16 for buf in reads)
            res[label]["read_step"] = {
                "ms_per_token": round(ms_r, 4), "tokens_per_s": round(1e3 / ms_r, 1),
                "bytes_per_token": rbytes, "GB/s": round(gbs(rbytes, ms_r), 1),
                "about": "the same launch sequence, each GEMV replaced by the one-shot read kernel "
                         "over its tiled weight buffer (256-thread workgroups, one load in flight "
                         "per lane; the 328 MB LM head strided over 65536 workgroups)"}
        del layers, calls, reads
        torch.cuda.synchronize()
    best = res["fused"]
    ms = best.pop("ms")
    res["unfused"].pop("ms")
    roof_tps = HBM_PEAK_GBS * 1e9 / best["bytes_per_token"]
    tps = 1e3 / ms
    out = line("decode step tokens/s (Llama-3-8B-shaped W4 sweep, M=1)", round(tps, 1), "tokens/s",
               a, ms,
               {"workload": "w4_llama3_8b_decode_step" + ("_w4p" if w4_fmt(a) == 5 else ""),
                "gemvs_per_token": best["gemvs_per_token"], "bytes_per_token": best["bytes_per_token"],
                "format": FMT_NAME[w4_fmt(a)] + " group-32"},
               {"bound": "hbm", "achieved": round(tps, 1), "peak": round(roof_tps, 1),
                "unit": "tokens/s", "frac": round(tps / roof_tps, 4),
                "achieved_GB/s": best["GB/s"], "peak_GB/s": HBM_PEAK_GBS, "traffic": None},
               steps_timed=steps, fused=best, unfused=res["unfused"],
               pct_of_hbm_peak=round(100 * best["GB/s"] / HBM_PEAK_GBS, 2),
               attainable={"read_step_tokens_per_s": best["read_step"]["tokens_per_s"],
                           "pct_of_read_step": round(100 * tps / best["read_step"]["tokens_per_s"], 2),
                           "about": best["read_step"]["about"]})
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = sweep_cpu_baseline(w4_fmt(a), best["bytes_per_token"])
    return out


def batched_workload(a, torch, timer):
    """Small-M products (SPECTRA section 4.2) on the W4 14336 x 4096 and
    4096 x 14336 layers: the tiled layout's kernels (the same buffer as the
    M = 1 kernel), the row-major arrays' batched kernel, M repeated GEMVs,
    and the tiled M = 1 GEMV of the same layer in the same run."""
    import oracle as O
    import synthetic
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    rows = []
    shapes = [(14336, 4096), (4096, 14336)]
    if a.shape:
        shapes = [tuple(int(v) for v in a.shape.lower().split("x"))]
    st, wu = max(1, a.steps // 4), max(1, a.warmup // 4)
    for (N, K) in shapes:
        Lb = synthetic.config4(16, N, K)
        base = DeviceLayer(pack_host(w4_fmt(a), Lb.W), tiled=True)
        ref = None if a.no_cpu_baseline else O.quantize_layer(w4_fmt(a), Lb.W)
        n1 = base.nbytes(1)
        l1 = rotated(DeviceLayer, base, n1)
        x1 = torch.from_numpy(np.ascontiguousarray(Lb.x[0]).view(np.int16)).cuda()
        y1 = [torch.empty(N, dtype=torch.int16, device="cuda") for _ in range(len(l1))]
        ms_m1 = timer(lambda i: l1[i % len(l1)].gemv_tiled(x1, y1[i % len(l1)]), st, wu, len(l1))
        del l1
        for M in ((a.m,) if a.m else (2, 4, 8, 16)):
            nbytes = base.nbytes(M)
            layers = rotated(DeviceLayer, base, nbytes)
            nc = len(layers)
            X = torch.from_numpy(np.ascontiguousarray(Lb.x[:M]).view(np.int16)).cuda()
            Y = [torch.empty((M, N), dtype=torch.int16, device="cuda") for _ in range(nc)]
            xrow = [X[m].contiguous() for m in range(M)]
            ms_tiled = timer(lambda i: layers[i % nc].gemm_tiled(X, Y[i % nc]), st, wu, nc)
            ms_gemm = timer(lambda i: layers[i % nc].gemm(X, Y[i % nc]), st, wu, nc)

            def rep(i):
                for m in range(M):
                    layers[i % nc].gemv(xrow[m], Y[i % nc][m])
            ms_rep = timer(rep, max(1, st // M), max(1, wu // M), nc)
            ms = min(ms_tiled, ms_gemm)
            flops = 2.0 * M * N * K
            tfl = flops / (ms * 1e-3) / 1e12
            layout = "tiled" if ms_tiled <= ms_gemm else "rowmajor"
            roof = roofline_hbm(nbytes, ms, traffic_for(f"w4_{N}x{K}_m{M}_{layout}")
                                if w4_fmt(a) == 4 else None)
            roof["mfma"] = {"achieved": round(tfl, 2), "peak": MFMA_FP16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tfl / MFMA_FP16_PEAK_TFLOPS, 5)}
            out = line(f"batched M={M} W4A16 product effective HBM GB/s", round(gbs(nbytes, ms), 2),
                       "GB/s", a, ms,
                       {"workload": f"w{'4p' if w4_fmt(a) == 5 else '4'}_{N}x{K}_m{M}", "N": N,
                        "K": K, "M": M, "format": FMT_NAME[w4_fmt(a)] + " group-32",
                        "bytes_per_step": nbytes, "rotated_copies": nc, "layout": layout},
                       roof,
                       tiled={"us": round(ms_tiled * 1e3, 3), "GB/s": round(gbs(nbytes, ms_tiled), 1),
                              "over_m1": round(ms_tiled / ms_m1, 3)},
                       rowmajor={"us": round(ms_gemm * 1e3, 3), "GB/s": round(gbs(nbytes, ms_gemm), 1)},
                       m1_tiled_us=round(ms_m1 * 1e3, 3),
                       repeated_gemv_us=round(ms_rep * 1e3, 3),
                       speedup_vs_repeated_gemv=round(ms_rep / ms, 2))
            if ref is not None:
                out["cpu_baseline"] = cpu_baseline_layer(ref, Lb.x[:M], nbytes, runs=1)
            rows.append(out)
            del layers
    return rows


def w2_70b_workload(a, torch, timer):
    """70B-class W2 layers with 3.5% FP16 outlier columns (28672 x 8192 and
    8192 x 28672) at M = 1 and M = 8, on both layouts."""
    import synthetic
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    rows = []
    st, wu = max(1, a.steps // 4), max(1, a.warmup // 4)
    for (N, K) in ((28672, 8192), (8192, 28672)):
        L8 = synthetic.config5(N, K, 8)
        base = DeviceLayer(pack_host(2, L8.W, L8.profile, L8.ratio), tiled=True)
        cpu = {}
        att = attainable_read(torch, timer, base.nbytes(1), st, wu)
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
            ms = timer(fn, st, wu, nc)
            g = gbs(nbytes, ms)
            out = line("M=%d W2 + outliers effective HBM GB/s" % M, round(g, 2), "GB/s", a, ms,
                       {"workload": f"w2_{N}x{K}_outliers{base.n_out}_m{M}", "N": N, "K": K, "M": M,
                        "n_out": base.n_out, "format": "W2 group-32", "layout": layout,
                        "bytes_per_step": nbytes, "rotated_copies": nc},
                       roofline_hbm(nbytes, ms, traffic_for(f"w2_{N}x{K}_m{M}_{layout}")),
                       pct_of_hbm_peak=round(100 * g / HBM_PEAK_GBS, 2),
                       attainable={"read_probe_GB/s": round(att[0], 1),
                                   "pct_of_read_probe": round(100 * g / att[0], 2),
                                   "read_probe_geometry": att[1],
                                   "about": "the best of the one-shot read kernels over the layer's "
                                            "M = 1 bytes per launch, rotated and graph-replayed in "
                                            "the same run"})
            if not a.no_cpu_baseline:
                if M not in cpu:
                    cpu[M] = cpu_baseline_rows(2, L8.W, L8.profile, L8.ratio, L8.x[:M], 2048,
                                               f"the {N}x{K} W2 layer")
                out["cpu_baseline"] = cpu[M]
            rows.append(out)
            del layers
    return rows


def cpu_baseline_rows(fmt, W, profile, ratio, X, rows, what):
    """The oracle on a bounded sample of a large layer: its first `rows`
    output rows, quantized by the oracle beforehand (untimed), then the timed
    dequantization + float64 product; GB/s in the sample's algorithmic bytes
    (codes, scales, zeros, outlier slab and indices, X and the sample's Y)."""
    import oracle as O
    X = np.atleast_2d(X)
    ref = O.quantize_layer(fmt, W[:rows], profile, ratio)
    M, K = X.shape
    G = K // 32
    zb = rows * ((G + 1) // 2) if fmt == 5 else 2 * rows * G
    nb = ref.codes.nbytes + 2 * rows * G + zb + 2 * rows * ref.n_out + 4 * ref.n_out + 2 * M * K \
        + 2 * M * rows
    t_deq, t_mv = oracle_times(ref, X, 1, min_s=5.0)
    t = t_deq + t_mv
    return cpu_baseline_rate(round(nb / t / 1e9, 4), "GB/s", t_deq, t_mv,
                             f"{what}: the first {rows} of {W.shape[0]} output rows "
                             f"({rows}x{K}, M={M}), oracle dequantization + float64 product, "
                             f"median over at least 5 s of runs ({t:.2f} s each)")


def host_read_baseline(nbytes):
    """Host-side reference for the plain streaming kernels (which have no
    oracle): numpy's sum over a buffer of the same size, as uint64 words."""
    buf = np.ones(nbytes // 8, np.uint64)
    t0 = time.perf_counter()
    reps = 0
    while True:
        int(buf.sum())
        reps += 1
        if time.perf_counter() - t0 > 1.0:
            break
    t = (time.perf_counter() - t0) / reps
    info = host_info()
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "numpy read",
            "cpu_model": info["cpu_model"],
            "sample": f"numpy sum over {nbytes} bytes of uint64 words, {reps} passes in "
                      f"{t * reps:.2f} s, one thread of {info['cores']} host cores"}


def embed_workload(a, torch, timer):
    """Embedding row gather (SPECTRA section 4.3) from a W4 (or W4P) table of
    131072 x 4096 (the page's example vocabulary): n_ids uniformly drawn token
    ids per launch, a fresh id set each launch (rotated), rows dequantized
    straight into FP16 output rows.  Bytes = the gathered rows' codes, scales,
    zeros and ids read plus the FP16 rows written."""
    import oracle as O
    import synthetic
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    V, K = 131072, 4096
    fmt = w4_fmt(a)
    W = synthetic.gaussian_weights(V, K, 0.02, 6, 0, fmt)
    dl = DeviceLayer(pack_host(fmt, W))
    # the oracle's table for the CPU baseline: the first 8192 rows (quantized untimed)
    ref = None if a.no_cpu_baseline else O.quantize_layer(fmt, W[:8192])
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
        ms = timer(fn, max(1, a.steps // 4), max(1, a.warmup // 4), nsets)
        nbytes = n_ids * (K // 2 + 2 * G + zrow + 4) + n_ids * K * 2
        g = gbs(nbytes, ms)
        out = line(f"embedding gather ({n_ids} ids) effective HBM GB/s", round(g, 2), "GB/s", a, ms,
                   {"workload": f"embed_gather_{V}x{K}_w{'4p' if fmt == 5 else '4'}_ids{n_ids}",
                    "V": V, "K": K, "n_ids": n_ids, "bytes_per_step": nbytes,
                    "id_sets": nsets},
                   roofline_hbm(nbytes, ms), pct_of_hbm_peak=round(100 * g / HBM_PEAK_GBS, 2))
        if ref is not None:
            rid = np.random.default_rng(7 + n_ids).integers(0, 8192, n_ids)
            reps, t0 = 0, time.perf_counter()
            while True:
                q = O.unpack_w4(ref.codes[rid])
                O.dequant_w4(q, ref.scale[rid], ref.zero[rid])
                reps += 1
                if time.perf_counter() - t0 > 2.0:
                    break
            t = (time.perf_counter() - t0) / reps
            info = host_info()
            out["cpu_baseline"] = {
                "value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": info["cores"],
                "kind": "oracle", "cpu_model": info["cpu_model"],
                "sample": f"{n_ids} ids drawn from the first 8192 rows of the table (the oracle's "
                          f"packed codes, scales and zeros): code unpacking + dequantization of the "
                          f"gathered rows, {reps} runs in {t * reps:.2f} s, numpy single-threaded"}
        rows.append(out)
    return rows


def kurtosis_workload(a, torch, timer):
    """The kurtosis-adaptive outlier policy (SPECTRA sections 3.1-3.3) on the W2
    layers of the other workloads: kappa, the ratio and n_out it picks (host
    time), and the tiled W2 GEMV with those outliers next to the profile-guided
    3.5% of the default workloads; `value` is the kurtosis-picked layer's rate."""
    import synthetic
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host
    import bit_weight_only_gemv_amd as B
    rows = []
    for label, L in (("w2_14336x4096", synthetic.config2()),
                     ("w2_28672x8192", synthetic.config5(28672, 8192, 1))):
        t0 = time.time()
        idx, r, kappa = B.wq_select_outliers_kurtosis(L.W)
        t_sel = time.time() - t0
        res = {}
        for pol in ("kurtosis", "profile_3.5pct"):
            hl = pack_host(2, L.W, kurtosis=True) if pol == "kurtosis" else \
                pack_host(2, L.W, L.profile, L.ratio)
            base = DeviceLayer(hl, tiled=True)
            nbytes = base.nbytes(1)
            layers = rotated(DeviceLayer, base, nbytes)
            nc = len(layers)
            x = torch.from_numpy(L.x[:1].reshape(-1).view(np.int16)).cuda()
            ys = [torch.empty(base.N, dtype=torch.int16, device="cuda") for _ in range(nc)]
            ms = timer(lambda i: layers[i % nc].gemv_tiled(x, ys[i % nc]), max(1, a.steps // 4),
                       max(1, a.warmup // 4), nc)
            res[pol] = {"n_out": base.n_out, "bytes": nbytes, "us": round(ms * 1e3, 3),
                        "GB/s": round(gbs(nbytes, ms), 2), "timing_us": ms.us(), "ms": ms}
            del layers
        k = res["kurtosis"]
        ms = k.pop("ms")
        res["profile_3.5pct"].pop("ms")
        out = line("M=1 W2 GEMV with kurtosis-picked outliers, effective HBM GB/s", k["GB/s"], "GB/s",
                   a, ms,
                   {"workload": f"kurtosis_policy_{label}", "N": L.W.shape[0], "K": L.W.shape[1],
                    "M": 1, "n_out": k["n_out"], "format": "W2 group-32", "layout": "tiled",
                    "bytes_per_step": k["bytes"]},
                   roofline_hbm(k["bytes"], ms),
                   kappa=round(kappa, 4), ratio=round(r, 5), host_select_s=round(t_sel, 3),
                   kurtosis=k, profile_3_5pct=res["profile_3.5pct"])
        if not a.no_cpu_baseline:
            out["cpu_baseline"] = _kurtosis_cpu(L, idx)
        rows.append(out)
    return rows


def _kurtosis_cpu(L, idx):
    """The oracle on the kurtosis-picked layer: its first 2048 output rows with
    the same outlier columns, dequantization + float64 product."""
    import oracle as O
    rows = 2048
    ref = O.quantize_layer(2, L.W[:rows], idx=idx)
    K = L.W.shape[1]
    G = K // 32
    nb = ref.codes.nbytes + 4 * rows * G + 2 * rows * ref.n_out + 4 * ref.n_out + 2 * K + 2 * rows
    t_deq, t_mv = oracle_times(ref, L.x[:1], 1, min_s=5.0)
    t = t_deq + t_mv
    return cpu_baseline_rate(round(nb / t / 1e9, 4), "GB/s", t_deq, t_mv,
                             f"the first {rows} of {L.W.shape[0]} output rows with the "
                             f"{len(idx)} kurtosis-picked outlier columns, oracle dequantization + "
                             f"float64 product, median over at least 5 s of runs ({t:.2f} s each)")


def refine_workload(a, torch, timer):
    """Runtime top-k refinement (StrataFlux section 3.2.1, Eq. 2) after the tiled
    GEMV: per 1024-channel chunk the k = 32 largest |x_i| are selected on the GPU
    and their 4-bit residual columns added to y.  Times the selection, the add,
    the GEMV, the three in sequence, and the GEMV with the selection and the add
    in the same launch (`value`, in the layer's and the refinement's bytes); the
    layer and its refinement columns are rotated like the GEMV's.  Refinement
    bytes = the selected columns' codes, scales and zeros, the indices and x
    entries read, and y read and written."""
    import oracle as O
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
        st = max(1, a.steps // 4)
        wu = max(1, a.warmup // 4)
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

        def chain_fused(i):
            layers[i % nc].gemv_tiled(x, ys[i % nc])
            layers[i % nc].refine_topk(x, ys[i % nc], k, chunk)

        t_all_fused = timer(chain_fused, st, wu, nc)
        t_one = timer(lambda i: layers[i % nc].gemv_tiled_refine(x, ys[i % nc], k, chunk), st, wu, nc)
        Gn = N // 32
        rbytes = n_sel * (N // 2 + 4 * Gn) + 4 * n_sel + 2 * n_sel + 4 * N
        total = nbytes + rbytes - 4 * N + 2 * N     # y is written once in the one-launch form
        g = gbs(total, t_one)
        out = line("M=1 GEMV + top-k refinement in one launch, effective HBM GB/s", round(g, 2),
                   "GB/s", a, t_one,
                   {"workload": f"refine_topk{k}_per{chunk}_{label}", "N": N, "K": K, "M": 1,
                    "n_sel": n_sel, "bytes_per_step": total, "layer_bytes": nbytes,
                    "refine_bytes": rbytes, "layout": "tiled"},
                   roofline_hbm(total, t_one),
                   topk_us=round(t_topk * 1e3, 3), refine_us=round(t_ref * 1e3, 3),
                   refine_GB_per_s=round(gbs(rbytes, t_ref), 1),
                   gemv_us=round(t_gemv * 1e3, 3),
                   fused_topk_refine_us=round(t_fused * 1e3, 3),
                   gemv_topk_refine_us=round(t_all * 1e3, 3),
                   gemv_fused_refine_us=round(t_all_fused * 1e3, 3),
                   two_launch_overhead_pct=round(100 * (t_all_fused - t_gemv) / t_gemv, 1),
                   one_launch_overhead_pct=round(100 * (t_one - t_gemv) / t_gemv, 1))
        if not a.no_cpu_baseline:
            ref = O.quantize_layer(L.fmt, L.W, L.profile, L.ratio)
            rq = O.refinement_w4(L.W, ref.w_hat(), ref.idx)
            c_hat = O.dequant_w4(*rq)
            t0 = time.perf_counter()
            w_hat = ref.w_hat()
            y0, _ = O.matvec_ref(w_hat, L.x[:1], ref.idx, ref.wout)
            t1 = time.perf_counter()
            sel = O.topk_chunks(L.x[0], k, chunk)
            O.refine_ref(y0[0], L.x[0], sel, c_hat)
            t2 = time.perf_counter()
            out["cpu_baseline"] = cpu_baseline_rate(
                round(total / (t2 - t0) / 1e9, 4), "GB/s", t1 - t0, t2 - t1,
                f"the whole {N}x{K} layer: oracle dequantization + float64 product, then the "
                f"oracle's top-k selection and refinement add over the dequantized residual "
                f"columns ({t2 - t0:.2f} s; the refinement's time is in matvec_s)")
        rows.append(out)
        del layers
    return rows


def stream_workload(a, torch, timer, copy):
    """Plain streaming kernels: the attainable read rate (read) and the
    byte-counter calibration (copy)."""
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
    out = line(("copy" if copy else "read") + " probe HBM GB/s", round(gbs(moved, ms), 2), "GB/s", a,
               ms, {"workload": "copy_probe" if copy else "read_probe", "bytes_per_step": moved,
                    "rotated_copies": ncopy},
               roofline_hbm(moved, ms))
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = host_read_baseline(nb)
    return out


PROBE_SIZES = [26157628, 10502144, 104555640, 37289984, 147849216, 265056256]


def probe_sweep_workload(a, torch, timer):
    """The attainable streaming-read rate per launch at the layers' sizes: the
    grid-stride read kernel over a table of launch geometries (workgroups x
    threads x loads in flight per lane, blocks 0 = one-shot) over rotated
    buffers, every geometry timed like the GEMV.  One line per size, with the
    best geometry and the fastest rows of the table."""
    import bit_weight_only_gemv_amd as B
    rows = []
    sizes = [int(v) for v in a.probe_sizes.split(",")] if a.probe_sizes else PROBE_SIZES
    for nbytes in sizes:
        nb = (nbytes + 15) // 16 * 16
        ncopy = max(1, -(-ROTATE_BYTES // nb))
        bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
        sink = torch.empty(65536, dtype=torch.int32, device="cuda")
        table = []
        for blocks in (0, 256, 512, 1024, 2048, 4096):
            for threads in (256, 512, 1024):
                for ring in (1, 2, 4, 8):
                    per_block = threads * 16 * ring
                    nblk = blocks if blocks else -(-nb // per_block)
                    if nblk > 65536 or nblk * per_block > 0x80000000:
                        continue
                    if blocks and blocks * per_block >= nb:
                        continue       # the same single round as the one-shot launch
                    ms = timer(lambda i: B.wq_read_probe_geom(bufs[i % ncopy], nb, sink, blocks,
                                                               threads, ring),
                               max(ncopy, a.steps // 10), max(ncopy, a.warmup // 10), ncopy)
                    table.append({"blocks": blocks or f"one-shot ({nblk})", "threads": threads,
                                  "ring": ring, "us": round(ms * 1e3, 3),
                                  "GB/s": round(gbs(nb, ms), 1), "_ms": ms})
        ms_gs = timer(lambda i: B.wq_read_probe(bufs[i % ncopy], nb,
                                                 sink[:B.wq_read_probe_sink_words(nb)]),
                      max(ncopy, a.steps // 10), max(ncopy, a.warmup // 10), ncopy)
        best = min(table, key=lambda r: r["us"])
        ms = best["_ms"]
        for r in table:
            del r["_ms"]
        out = line("attainable streaming read (best launch geometry) HBM GB/s", best["GB/s"], "GB/s",
                   a, ms, {"workload": f"read_probe_sweep_{nb}B", "bytes_per_step": nb,
                           "rotated_copies": ncopy},
                   roofline_hbm(nb, ms), best=best,
                   library_read_probe={"us": round(ms_gs * 1e3, 3), "GB/s": round(gbs(nb, ms_gs), 1)},
                   table=sorted(table, key=lambda r: r["us"])[:25])
        if not a.no_cpu_baseline:
            out["cpu_baseline"] = host_read_baseline(min(nb, 64 << 20))
        rows.append(out)
        del bufs
        torch.cuda.synchronize()
    return rows


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
