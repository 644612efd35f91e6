"""GPU parity at the full sizes of the larger workloads, in the launch
configuration the benchmark times, on every output element:

* 70B-class W2 + outlier layers (28672 x 8192 and 8192 x 28672; M = 1 and
  M = 8, each on the row-major and the tiled layout): the oracle selects the
  outlier columns from the whole matrix, then splits, quantizes and multiplies
  the rows in chunks of 4096 (the encoding of a row does not depend on other
  rows once the outlier columns are fixed), covering every row;
* the Llama-3-8B-shaped W4 decode sweep (225 GEMVs) captured in one HIP
  graph: every replay (with eager work in between) equals the eager result
  bit for bit, and every distinct projection of the first layer and the
  whole LM head (128256 rows) match the oracle;
* the stacked projections the fused sweep runs (q|k|v 6144 x 4096, gate|up
  28672 x 4096), on both layouts, on every row.
"""

import sys

import numpy as np
import pytest

import oracle as O
import synthetic

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host  # noqa: E402


def say(*a):
    print(*a, flush=True, file=sys.stderr)


CHUNK = 4096


def row_chunks(N, chunk=CHUNK):
    """Every row, in consecutive chunks of at most `chunk` rows."""
    return [np.arange(r0, min(N, r0 + chunk), dtype=np.int64) for r0 in range(0, N, chunk)]


def check_all_rows(outputs, fmt, W, profile, ratio, X):
    """Each GPU output (a label and its [M, N] FP16 array) against the oracle on
    every row, chunk by chunk."""
    N = W.shape[0]
    idx = O.select_outliers(W, profile, ratio) if profile is not None else np.zeros(0, np.int32)
    worst = {label: 0.0 for label, _ in outputs}
    for rows in row_chunks(N):
        dense, wout = O.split_outliers(W[rows], idx)
        if fmt == 4:
            q, s, z, _ = O.quantize_w4(dense)
            w_hat = O.dequant_w4(q, s, z)
        else:
            q, s, z = O.quantize_w2(dense)
            w_hat = O.dequant_w2(q, s, z)
        for label, y in outputs:
            Xm = X[:y.shape[0]]
            y_ref, a = O.matvec_ref(w_hat, Xm, idx if len(idx) else None,
                                    wout if len(idx) else None)
            ok, wr = O.check_tolerance(y[:, rows].astype(np.float64), y_ref, a)
            assert ok, f"{label}: rows {rows[0]}..{rows[-1]}: worst |err|/bound = {wr}"
            worst[label] = max(worst[label], wr)
    for label, wr in worst.items():
        say(f"  {label}: all {N} rows, worst |err|/bound = {wr:.4f}")
    return idx


@pytest.mark.parametrize("N,K", [(28672, 8192), (8192, 28672)])
def test_w2_70b_class_outliers(N, K):
    say(f"W2 70B-class {N}x{K} + outliers")
    L = synthetic.config5(N, K, 8)
    dl = DeviceLayer(pack_host(2, L.W, L.profile, L.ratio), tiled=True)
    assert dl.n_out == int(np.floor(0.035 * K))
    X = torch.from_numpy(np.ascontiguousarray(L.x).view(np.int16)).cuda()
    y1 = torch.empty(N, dtype=torch.int16, device="cuda")
    dl.gemv(X[0].contiguous(), y1)
    yt = torch.empty(N, dtype=torch.int16, device="cuda")
    dl.gemv_tiled(X[0].contiguous(), yt)
    Y8 = torch.empty((8, N), dtype=torch.int16, device="cuda")
    dl.gemm(X, Y8)
    Y8t = torch.empty((8, N), dtype=torch.int16, device="cuda")
    dl.gemm_tiled(X, Y8t)
    torch.cuda.synchronize()

    def h(t):
        return t.cpu().numpy().view(np.float16).reshape(-1, N)
    idx = check_all_rows([(f"M=1 {N}x{K}", h(y1)), (f"M=1 tiled {N}x{K}", h(yt)),
                          (f"M=8 {N}x{K}", h(Y8)), (f"M=8 tiled {N}x{K}", h(Y8t))],
                         2, L.W, L.profile, L.ratio, L.x)
    # spiked channels carry |N(0,1)| x 300 in the profile: all but the ones whose
    # draw was tiny land among the top 3.5% of scores
    hit = len(set(L.spikes.tolist()) & set(idx.tolist()))
    assert hit >= 0.95 * len(L.spikes)


def test_llama_sweep_graph_replay_and_oracle():
    shapes = synthetic.config3_shapes()
    assert len(shapes) == 225
    key = {"q": "sq", "o": "sq", "k": "kv", "v": "kv", "gate": "mlp", "up": "mlp",
           "down": "down", "lm_head": "lm_head"}
    proto, Ws = {}, {}
    for (layer, proj, name, N, K) in shapes:
        k = key[name]
        if k not in proto:
            L = synthetic.config3_layer(layer, proj, N, K, name)
            Ws[k] = L.W
            proto[k] = DeviceLayer(pack_host(4, L.W))
    xs, ys, ls = [], [], []
    for (layer, proj, name, N, K) in shapes:
        x = synthetic.gaussian_x_fp16(1, K, 3, layer, proj)
        xs.append(x)
        ls.append(proto[key[name]])
        ys.append(torch.empty(N, dtype=torch.int16, device="cuda"))
    xd = [torch.from_numpy(x.reshape(-1).view(np.int16)).cuda() for x in xs]

    def run():
        for d, x, y in zip(ls, xd, ys):
            d.gemv(x, y)

    run()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for y in ys:
        y.fill_(-1)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for rep in range(3):
        for y in ys:
            y.fill_(-1)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(ys, eager)):
            assert torch.equal(y, e), f"replay {rep}: GEMV {i} differs from the eager run"
    say("  225-GEMV graph: 3 replays equal the eager run")
    # every distinct projection of the first layer (q, k, v, o, gate, up, down)
    # and the LM head against the oracle, on every row
    for i in list(range(7)) + [224]:
        layer, proj, name, N, K = shapes[i]
        W = Ws[key[name]]   # the graph runs each shape class on one prototype layer
        check_all_rows([(f"sweep GEMV {i} ({name} {N}x{K})",
                         eager[i].cpu().numpy().view(np.float16)[None, :])],
                       4, W, None, 0.0, xs[i])


@pytest.mark.parametrize("names", [("q", "k", "v"), ("gate", "up")])
def test_stacked_projections_both_layouts(names):
    shapes = {name: (p, N, K) for (layer, p, name, N, K) in synthetic.config3_shapes() if layer == 0}
    Ws = [synthetic.config3_layer(0, shapes[n][0], shapes[n][1], shapes[n][2], n).W for n in names]
    W = np.concatenate(Ws, axis=0)
    N, K = W.shape
    say(f"stacked {'|'.join(names)} {N}x{K}")
    dl = DeviceLayer(pack_host(4, W), tiled=True)
    x = synthetic.gaussian_x_fp16(1, K, 3, 0, 0)
    xd = torch.from_numpy(x.reshape(-1).view(np.int16)).cuda()
    y1 = torch.empty(N, dtype=torch.int16, device="cuda")
    y2 = torch.empty(N, dtype=torch.int16, device="cuda")
    dl.gemv(xd, y1)
    dl.gemv_tiled(xd, y2)
    torch.cuda.synchronize()
    check_all_rows([(f"stacked {N}x{K} row-major", y1.cpu().numpy().view(np.float16)[None, :]),
                    (f"stacked {N}x{K} tiled", y2.cpu().numpy().view(np.float16)[None, :])],
                   4, W, None, 0.0, x)
