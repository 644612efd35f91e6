#!/usr/bin/env python3
"""Benchmark of the fused low-bit weight-only GEMV on one MI355X.

Default workload (one JSON line): M = 1 W2 GEMV of a 14336 x 4096 layer
(Llama-3-8B MLP gate/up shape), Lloyd-Max 2-bit codes with OLS group-32
scale/zero and 143 (3.5%) FP16 outlier columns, x FP16 with 1% of channels
x100.  One step = one launch of the whole fused path (stream codes, scales,
zeros and the outlier slab; decode; multiply; reduce; add outliers; store y).

Weights are rotated through >= 512 MB of distinct device copies so that
neither the 256 MB Infinity Cache nor the L2s serve repeats; inputs are
resident in HBM before the timed region.  Timing: hipEvents on the stream
the kernels run on, around exactly --steps launches, bracketed by device
synchronization.

``value`` is GB/s of algorithmic bytes (codes + FP16 scales + FP16 zeros +
FP16 outlier slab + int32 indices + x + y) per second of wall time per step.

Other workloads (``--workload``): w4_4096 (W4 4096x4096), sweep (Llama-3-8B
shaped decode: 225 W4 GEMVs replayed as one HIP graph, tokens/s), batched
(W4 small-M MFMA path), w2_70b (W2 + outliers 28672x8192 / 8192x28672).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "M=1 dequant-GEMV effective HBM GB/s (% of MI355X peak); eq. tokens/s"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 512 << 20


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="w2_14336",
                   choices=["w2_14336", "w4_4096", "sweep", "batched", "w2_70b", "read"])
    p.add_argument("--read-bytes", type=int, default=26157628,
                   help="bytes per launch of the read-probe workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true", help="replay the timed launches as a HIP graph")
    return p.parse_args()


def sweep_bytes_per_token(fmt: int, ratio: float) -> int:
    """Algorithmic bytes of one Llama-3-8B-shaped decode step (32 layers x 7
    projections + LM head) in the given format."""
    import synthetic
    tot = 0
    for (_, _, _, N, K) in synthetic.config3_shapes():
        n_out = int(np.floor(ratio * K)) if ratio > 0 else 0
        codes = N * K // (2 if fmt == 4 else 4)
        tot += codes + 4 * N * (K // 32) + 2 * N * n_out + 4 * n_out + 2 * K + 2 * N
    return tot


def main():
    a = _parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the path is a "
              "single-GPU kernel and multi-GPU sharding is not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synthetic
    import bit_weight_only_gemv_amd as B
    from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host

    B.load()
    torch.cuda.init()
    dev = torch.cuda.get_device_name(0)
    stream = torch.cuda.current_stream()

    if a.workload == "read":
        return read_probe(a, torch, B)
    if a.workload == "w2_14336":
        L = synthetic.config2()
        label = "w2_14336x4096_outliers143_m1"
    elif a.workload == "w4_4096":
        L = synthetic.config1()
        label = "w4_4096x4096_m1"
    else:
        print("workload not implemented yet", file=sys.stderr)
        sys.exit(3)

    t0 = time.time()
    hl = pack_host(L.fmt, L.W, L.profile, L.ratio)
    pack_s = time.time() - t0
    base = DeviceLayer(hl)
    nbytes = base.nbytes(1)
    ncopy = max(1, -(-ROTATE_BYTES // nbytes))
    layers = [base]
    for _ in range(ncopy - 1):
        c = DeviceLayer.__new__(DeviceLayer)
        c.__dict__.update(base.__dict__)
        c.codes, c.scales, c.zeros = base.codes.clone(), base.scales.clone(), base.zeros.clone()
        if base.n_out:
            c.idx, c.wout = base.idx.clone(), base.wout.clone()
        layers.append(c)
    x = torch.from_numpy(L.x.reshape(-1).view(np.int16)).cuda()
    ys = [torch.empty(base.N, dtype=torch.int16, device="cuda") for _ in range(ncopy)]
    torch.cuda.synchronize()

    def step(i):
        layers[i % ncopy].gemv(x, ys[i % ncopy])

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if a.graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(a.steps):
                    step(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(a.steps):
            step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / a.steps
    gbs = nbytes / (ms_step * 1e-3) / 1e9

    bpt = sweep_bytes_per_token(L.fmt, L.ratio)
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded Gaussian weights and activations, no checkpoint)",
        "config": {"workload": label, "N": base.N, "K": base.K, "M": 1, "n_out": base.n_out,
                   "format": f"W{L.fmt} group-32", "accumulate": "f32",
                   "bytes_per_step": nbytes, "rotated_copies": ncopy,
                   "timing": "hip graph replay" if graph is not None else "eager launches"},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "eq_tokens_per_s": round(gbs * 1e9 / bpt, 1),
        "eq_tokens_basis_bytes_per_token": bpt,
        "device": dev,
        "host_pack_s": round(pack_s, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }

    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(L, nbytes)
    print(json.dumps(out), flush=True)


def read_probe(a, torch, B):
    """Attainable HBM read rate: a plain streaming-read kernel over rotated
    buffers of the given size (no decode, no arithmetic)."""
    nb = (a.read_bytes + 15) // 16 * 16
    ncopy = max(1, -(-ROTATE_BYTES // nb))
    bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
    for b in bufs:
        b.fill_(1)
    sink = torch.empty(B.wq_read_probe_sink_words(nb), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        B.wq_read_probe(bufs[i % ncopy], nb, sink)

    for i in range(a.warmup):
        step(i)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(stream)
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for i in range(a.steps):
                step(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / a.steps
    print(json.dumps({"workload": "read_probe", "bytes": nb, "copies": ncopy, "ms_per_step": ms,
                      "GB/s": round(nb / (ms * 1e-3) / 1e9, 1)}), flush=True)


def cpu_baseline(L, nbytes):
    """The oracle, as it stands, on the same layer: float64 dequantization of
    the packed weights followed by the float64 product (median of 3)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    ref = O.quantize_layer(L.fmt, L.W, L.profile, L.ratio)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        w_hat = ref.w_hat()
        O.matvec_ref(w_hat, L.x, ref.idx, ref.wout)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"whole {ref.N}x{ref.K} layer: oracle dequant + float64 product, median of 3 "
                      f"({t:.2f} s each); host has {len(os.sched_getaffinity(0))} cores"}


if __name__ == "__main__":
    main()
