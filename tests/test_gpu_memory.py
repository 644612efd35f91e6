"""The library allocates no device memory: ten thousand launches of every
kind of call (M = 1 GEMV on both layouts, the batched products, the dequantizer,
the embedding gather, the top-k selection, the refinement add and the GEMV
with the refinement in its launch) leave the device's free memory where it
was after the first round of them.  The first round loads the code objects
and lets the runtime set up its launch queues."""

import sys

import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bit_weight_only_gemv_amd as B  # noqa: E402
from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host, refinement_host  # noqa: E402

ROUNDS = 10
PER_ROUND = 1000


def test_launch_loop_keeps_device_memory_flat():
    print("memory-flat launch loop", flush=True, file=sys.stderr)
    N, K = 1024, 2048
    rng = np.random.default_rng(11)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    prof = np.abs(rng.standard_normal(K)) + 0.5
    layers = {fmt: DeviceLayer(pack_host(fmt, W, prof, 0.035), tiled=True) for fmt in (4, 2, 5)}
    ref_layer = layers[4]
    ref_layer.set_refinement(refinement_host(W, pack_host(4, W, prof, 0.035)))
    x = torch.from_numpy(synthetic.gaussian_x_fp16(1, K, 1, 0, 0).reshape(-1).view(np.int16)).cuda()
    X = torch.from_numpy(synthetic.gaussian_x_fp16(8, K, 2, 0, 0).view(np.int16)).cuda()
    y = torch.empty(N, dtype=torch.int16, device="cuda")
    Y = torch.empty((8, N), dtype=torch.int16, device="cuda")
    W_hat = torch.empty((N, K), dtype=torch.int16, device="cuda")
    ids = torch.from_numpy(rng.integers(0, N, 64).astype(np.int32)).cuda()
    rows = torch.empty((64, K), dtype=torch.int16, device="cuda")
    n_sel = B.wq_topk_count(K, 1024, 32)
    sel = torch.empty(n_sel, dtype=torch.int32, device="cuda")

    calls = []
    for fmt, d in layers.items():
        calls += [lambda d=d: d.gemv(x, y), lambda d=d: d.gemv_tiled(x, y),
                  lambda d=d: d.gemm(X, Y), lambda d=d: d.gemm_tiled(X, Y),
                  lambda d=d: d.dequant(W_hat)]
        if fmt != 2:
            calls.append(lambda d=d: d.embed(ids, rows))
    calls += [lambda: B.wq_topk_chunks(x, K, 1024, 32, sel),
              lambda: ref_layer.refine(x, y, sel, n_sel),
              lambda: ref_layer.refine_topk(x, y, 32, 1024),
              lambda: ref_layer.gemv_tiled_refine(x, y, 32, 1024)]

    def one_round():
        for i in range(PER_ROUND):
            calls[i % len(calls)]()
        torch.cuda.synchronize()

    one_round()
    torch_alloc = torch.cuda.memory_allocated()
    free = []
    for r in range(ROUNDS):
        one_round()
        free.append(torch.cuda.mem_get_info()[0])
        print(f"round {r}: free {free[-1]}", flush=True, file=sys.stderr)
    assert torch.cuda.memory_allocated() == torch_alloc
    # flat: no growth over 10^4 launches (the runtime's own bookkeeping may
    # move by a page or two; a per-call allocation would show as steady loss)
    assert max(free) - min(free) <= 2 << 20, free
