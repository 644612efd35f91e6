"""GPU parity: every device entry point of the C ABI against the CPU oracle on
the same seeded inputs.

* packed bytes and dequantized FP16 weights: bit-exact;
* formats W4, W2 and W4P (W4 with its zero points packed two per byte);
* products: every output element within |y - y_ref| <= 2e-3 sum|w x| + 1e-5
  (y_ref and sum|w x| in float64 from the oracle's own quantization).

Small cases span several workgroup tiles and ragged tails in N, K and n_out;
full-size cases use the workloads' real shapes in the launch configuration
the benchmark times.
"""

import sys

import numpy as np
import pytest

import oracle as O
import synthetic

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():   # collected but skipped off the GPU machine
    pytest.skip("no GPU", allow_module_level=True)

import bit_weight_only_gemv_amd as B  # noqa: E402
from bit_weight_only_gemv_amd.layer import DeviceLayer, pack_host  # noqa: E402


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def dev_fp16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16).view(np.int16)).cuda()


def host_fp16(t):
    return t.cpu().numpy().view(np.float16)


def build(fmt, W, profile=None, ratio=0.0):
    """Oracle layer, and the library's packing of the same W on the GPU (the
    two are byte-identical; checked here too)."""
    ref = O.quantize_layer(fmt, W, profile, ratio)
    hl = pack_host(fmt, W, profile, ratio)
    assert np.array_equal(hl.codes, ref.codes) and np.array_equal(hl.idx, ref.idx)
    if fmt == 5:
        assert np.array_equal(hl.zeros, ref.zero_packed)
    return ref, DeviceLayer(hl)


def check_product(ref, y, x, label):
    y_ref, a = O.matvec_ref(ref.w_hat(), x, ref.idx, ref.wout)
    ok, worst = O.check_tolerance(host_fp16(y).astype(np.float64).reshape(y_ref.shape), y_ref, a)
    say(f"  {label}: worst |err|/bound = {worst:.4f}")
    assert ok, f"{label}: worst |err|/bound = {worst}"
    return worst


def run_gemv(dl, x, flags=B.WQ_FUSE_OUTLIERS, variant=None):
    xd = dev_fp16(x.reshape(-1))
    y = torch.full((dl.N,), -1, dtype=torch.int16, device="cuda")
    dl.gemv(xd, y, flags, variant=variant)
    torch.cuda.synchronize()
    return y, xd


# --------------------------------------------------------------- dequant


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("N,K,scale", [(5, 96, 0.02), (37, 4096, 0.02), (130, 14336, 0.02),
                                       (64, 1024, 1e-5), (16, 512, 300.0)])
def test_dequant_device_bit_exact(fmt, N, K, scale):
    say(f"dequant fmt={fmt} N={N} K={K} sigma={scale}")
    W = synthetic.gaussian_weights(N, K, scale, 300, N, K)
    ref, dl = build(fmt, W)
    out = torch.empty((N, K), dtype=torch.int16, device="cuda")
    dl.dequant(out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(host_fp16(out)), _bits(ref.w_hat()))


# ------------------------------------------------------------------ gemv

SHAPES = [(1, 32), (7, 96), (129, 4096), (300, 14336), (77, 28672), (64, 8192), (33, 2080),
          (1000, 1024), (17, 65536), (5000, 4224)]


class Path(str):
    """A named kernel choice: the variant passed with each call."""

    def __new__(cls, name, variant):
        o = super().__new__(cls, name)
        o.variant = variant
        return o


@pytest.fixture(params=["valu", "mfma"])
def gemv_path(request):
    """Runs a GEMV test on the VALU kernels and again with the matrix-core
    kernel chosen wherever it supports the shape (K % 128 == 0 and its LDS
    fits); the library otherwise picks it only for large N."""
    return Path(request.param, B.variant(gemv_kernel=0 if request.param == "valu" else 2))


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("outl", [False, True])
def test_gemv_small(fmt, N, K, outl, gemv_path):
    say(f"gemv fmt={fmt} N={N} K={K} outliers={outl} path={gemv_path}")
    L = synthetic.small_layer(fmt, N, K, with_outliers=outl, seed=N % 17)
    ref, dl = build(fmt, L.W, L.profile, L.ratio)
    y, _ = run_gemv(dl, L.x, variant=gemv_path.variant)
    check_product(ref, y, L.x, f"w{fmt} {N}x{K} n_out={ref.n_out}")


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("n_out", [1, 31, 32, 33, 64, 65, 129, 500])
def test_gemv_outlier_counts(fmt, n_out, gemv_path):
    K = 4096
    say(f"gemv fmt={fmt} n_out={n_out} path={gemv_path}")
    L = synthetic.small_layer(fmt, 200, K, with_outliers=True, seed=n_out,
                              ratio=(n_out + 0.5) / K)
    ref, dl = build(fmt, L.W, L.profile, L.ratio)
    assert ref.n_out == n_out
    y, _ = run_gemv(dl, L.x, variant=gemv_path.variant)
    check_product(ref, y, L.x, f"w{fmt} n_out={n_out}")


@pytest.mark.parametrize("fmt", [4, 2, 5])
def test_gemv_unfused_then_outlier_add(fmt):
    say(f"gemv unfused + outlier_add fmt={fmt}")
    L = synthetic.small_layer(fmt, 333, 4096, with_outliers=True, seed=5)
    ref, dl = build(fmt, L.W, L.profile, L.ratio)
    y, xd = run_gemv(dl, L.x, flags=0)
    dl.outlier_add(xd.view(1, -1), y.view(1, -1))
    torch.cuda.synchronize()
    check_product(ref, y, L.x, "unfused")


# ------------------------------------------------------------- tiled gemv

# row blocks vs 256 compute units: 5000 rows -> 313 blocks (57 left over, cut in 4 row ranges);
# 5376 -> 336 (80 left, cut in 3); 300 -> 19 (fewer blocks than units, each cut in 4)
TILED_SHAPES = [(1, 32), (7, 96), (129, 4096), (300, 14336), (77, 28672), (33, 2080),
                (1000, 1024), (5000, 4224), (16, 512), (40, 32768), (5376, 1024)]


def build_tiled(fmt, W, profile=None, ratio=0.0):
    ref = O.quantize_layer(fmt, W, profile, ratio)
    hl = pack_host(fmt, W, profile, ratio)
    assert np.array_equal(hl.codes, ref.codes) and np.array_equal(hl.idx, ref.idx)
    return ref, DeviceLayer(hl, tiled=True)


def run_gemv_tiled(dl, x):
    xd = dev_fp16(x.reshape(-1))
    y = torch.full((dl.N,), -1, dtype=torch.int16, device="cuda")
    dl.gemv_tiled(xd, y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("N,K", TILED_SHAPES)
@pytest.mark.parametrize("outl", [False, True])
def test_gemv_tiled(fmt, N, K, outl):
    say(f"gemv tiled fmt={fmt} N={N} K={K} outliers={outl}")
    L = synthetic.small_layer(fmt, N, K, with_outliers=outl, seed=N % 17)
    ref, dl = build_tiled(fmt, L.W, L.profile, L.ratio)
    y = run_gemv_tiled(dl, L.x)
    check_product(ref, y, L.x, f"tiled w{fmt} {N}x{K} n_out={ref.n_out}")
    if K % 128 == 0:
        # the row-major matrix-core kernel performs the same operations in the
        # same order on the same values: identical bits
        y2, _ = run_gemv(dl, L.x, variant=B.variant(gemv_kernel=2))
        assert torch.equal(y, y2)


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("N,K", TILED_SHAPES)
@pytest.mark.parametrize("outl", [False, True])
@pytest.mark.parametrize("M", [2, 3, 4, 5, 8, 13, 16])
def test_gemm_tiled_rows(fmt, N, K, outl, M):
    """Up to 16 activation rows on the tiled layer: every row within the
    bound, on the kernel the library picks (the shared-slot kernel up to 4
    rows where it fits, else the batched kernel on the same tiles) and, up to
    4 rows, on the batched kernel too; M = 1 through the same entry equals the
    tiled GEMV."""
    say(f"gemm tiled M={M} fmt={fmt} N={N} K={K} outliers={outl}")
    L = synthetic.small_layer(fmt, N, K, M=M, with_outliers=outl, seed=N % 13 + M)
    ref, dl = build_tiled(fmt, L.W, L.profile, L.ratio)
    X = dev_fp16(L.x)
    paths = [("default", None)] + ([("batched", B.variant(gemm_rows=0))] if M <= 4 else [])
    for name, var in paths:
        Y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
        try:
            dl.gemm_tiled(X, Y, variant=var)
        except B.WQError as e:   # the batched kernel takes at most 1024 outlier columns
            assert e.status == -2 and ref.n_out > 1024, (e.status, fmt, M, K, ref.n_out)
            continue
        torch.cuda.synchronize()
        check_product(ref, Y, L.x, f"tiled M={M} w{fmt} {N}x{K} n_out={ref.n_out} {name}")
    if M == 2:
        Y1 = torch.full((1, N), -1, dtype=torch.int16, device="cuda")
        dl.gemm_tiled(dev_fp16(L.x[:1]), Y1)
        y = run_gemv_tiled(dl, L.x[0])
        assert torch.equal(Y1[0], y)


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("N,K,outl", [(129, 4096, True), (5000, 4224, True), (300, 14336, False)])
@pytest.mark.parametrize("M", [2, 3, 4])
def test_gemm_rows_paths(fmt, N, K, outl, M):
    """M = 2..4 on the row-major arrays: the shared-slot matrix-core kernel (the
    default where it applies) and the batched kernel (gemm_rows 0) both
    within the bound."""
    L = synthetic.small_layer(fmt, N, K, M=M, with_outliers=outl, seed=K % 11 + M)
    ref, dl = build(fmt, L.W, L.profile, L.ratio)
    X = dev_fp16(L.x)
    for rows in (1, 0):
        say(f"gemm M={M} fmt={fmt} {N}x{K} shared-slot kernel={rows}")
        Y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
        dl.gemm(X, Y, variant=B.variant(gemm_rows=rows))
        torch.cuda.synchronize()
        check_product(ref, Y, L.x, f"M={M} w{fmt} {N}x{K} rows={rows}")


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("n_out", [1, 7, 8, 9, 31, 33, 64, 65, 129, 256])
def test_gemv_tiled_outlier_counts(fmt, n_out):
    K = 4096
    say(f"gemv tiled fmt={fmt} n_out={n_out}")
    L = synthetic.small_layer(fmt, 200, K, with_outliers=True, seed=n_out,
                              ratio=(n_out + 0.5) / K)
    ref, dl = build_tiled(fmt, L.W, L.profile, L.ratio)
    assert ref.n_out == n_out
    y = run_gemv_tiled(dl, L.x)
    check_product(ref, y, L.x, f"tiled w{fmt} n_out={n_out}")


def test_gemv_tiled_unsupported_shapes():
    # 257 outlier positions over 8 slices of 512 channels: one slice would need 5 chunks
    L = synthetic.small_layer(2, 64, 4096, with_outliers=True, seed=3, ratio=257.5 / 4096)
    _, dl = build_tiled(2, L.W, L.profile, L.ratio)
    assert dl.n_out == 257
    y = torch.empty(64, dtype=torch.int16, device="cuda")
    with pytest.raises(B.WQError) as e:
        dl.gemv_tiled(dev_fp16(L.x.reshape(-1)), y)
    assert e.value.status == -2
    L = synthetic.small_layer(4, 16, 65536, seed=1)
    _, dl = build_tiled(4, L.W)
    with pytest.raises(B.WQError) as e:
        dl.gemv_tiled(dev_fp16(L.x.reshape(-1)), torch.empty(16, dtype=torch.int16, device="cuda"))
    assert e.value.status == -2


def test_gemv_deterministic(gemv_path):
    L = synthetic.small_layer(2, 1500, 4096, with_outliers=True, seed=9)
    ref, dl = build(2, L.W, L.profile, L.ratio)
    y1, _ = run_gemv(dl, L.x, variant=gemv_path.variant)
    y2, _ = run_gemv(dl, L.x, variant=gemv_path.variant)
    assert torch.equal(y1, y2)


def test_outlier_add_standalone():
    say("outlier_add M=3")
    L = synthetic.small_layer(4, 100, 2048, M=3, with_outliers=True, seed=2)
    ref = O.quantize_layer(4, L.W, L.profile, L.ratio)
    hl = pack_host(4, L.W, L.profile, L.ratio)
    dl = DeviceLayer(hl)
    rng = np.random.default_rng(0)
    y0 = rng.standard_normal((3, 100)).astype(np.float16)
    Y = dev_fp16(y0)
    dl.outlier_add(dev_fp16(L.x), Y)
    torch.cuda.synchronize()
    Xo = L.x.astype(np.float64)[:, ref.idx]
    exp = y0.astype(np.float64) + Xo @ ref.wout.astype(np.float64).T
    bound = O.TOL_REL * (np.abs(y0.astype(np.float64)) + np.abs(Xo) @ np.abs(ref.wout.astype(np.float64)).T) + O.TOL_ABS
    assert np.all(np.abs(host_fp16(Y).astype(np.float64) - exp) <= bound)


# ------------------------------------------------------------------ gemm


@pytest.fixture(params=["tile", "mfma"])
def gemm_path(request):
    """Runs a batched test on the per-group tile kernel and on the persistent
    matrix-core kernel (the library's choice wherever the latter supports the
    shape: K % 128 == 0, fused outliers, its LDS fits)."""
    return Path(request.param, B.variant(gemm_kernel=0 if request.param == "tile" else 1))


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 13, 16])
@pytest.mark.parametrize("N,K,outl", [(129, 4096, False), (200, 2080, True), (64, 14336, True),
                                      (5000, 4224, True), (300, 8192, True), (40, 28672, True)])
def test_gemm_small(fmt, M, N, K, outl, gemm_path):
    say(f"gemm fmt={fmt} M={M} N={N} K={K} outliers={outl} path={gemm_path}")
    L = synthetic.small_layer(fmt, N, K, M=M, with_outliers=outl, seed=M)
    ref, dl = build(fmt, L.W, L.profile, L.ratio)
    X = dev_fp16(L.x)
    Y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    dl.gemm(X, Y, variant=gemm_path.variant)
    torch.cuda.synchronize()
    check_product(ref, Y, L.x, f"gemm w{fmt} M={M} {N}x{K} n_out={ref.n_out}")


@pytest.mark.parametrize("qg", ["2", "4"])
@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("M", [2, 5, 16])
@pytest.mark.parametrize("N,K", [(129, 4096), (300, 8192), (5000, 4224), (64, 2176), (48, 384)])
def test_gemm_slice_widths(fmt, M, N, K, qg):
    """The matrix-core batched kernel with 256- and 512-channel slices (no
    outliers), including a short last slice (K % 512 = 128) and K below one
    slice."""
    say(f"gemm slices of {128 * int(qg)} fmt={fmt} M={M} N={N} K={K}")
    L = synthetic.small_layer(fmt, N, K, M=M, seed=M + N)
    ref, dl = build(fmt, L.W)
    X = dev_fp16(L.x)
    Y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    dl.gemm(X, Y, variant=B.variant(gemm_kernel=1, batch_slice_groups=int(qg)))
    torch.cuda.synchronize()
    check_product(ref, Y, L.x, f"gemm w{fmt} M={M} {N}x{K} slices {128 * int(qg)}")


@pytest.mark.parametrize("qg", ["2", "4"])
@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("M", [2, 5, 8, 16])
@pytest.mark.parametrize("N,K,outl", [(129, 4096, True), (300, 8320, False), (64, 2176, True),
                                      (1000, 10240, False), (96, 384, False)])
def test_gemm_row_transpose(fmt, M, N, K, outl, qg):
    """The batched kernel with its activation rows loaded whole and transposed
    in LDS (batch_row_transpose 1, where the LDS fits) or loaded in the lane
    layout directly (0): the same fragments, so bit-identical Y, within the
    bound; 256- and 512-channel slices (outlier layers always take 256), short
    last slices and rows past M included."""
    say(f"gemm row transpose fmt={fmt} M={M} N={N} K={K} outliers={outl} slices={128 * int(qg)}")
    L = synthetic.small_layer(fmt, N, K, M=M, with_outliers=outl, seed=M + N + 1)
    ref, dl = build(fmt, L.W, L.profile, L.ratio) if outl else build(fmt, L.W)
    X = dev_fp16(L.x)
    ys = []
    for xt in (1, 0):
        Y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
        dl.gemm(X, Y, variant=B.variant(gemm_kernel=2, gemm_rows=0, batch_slice_groups=int(qg),
                                        batch_row_transpose=xt))
        torch.cuda.synchronize()
        ys.append(Y.cpu().numpy())
    assert np.array_equal(ys[0], ys[1])
    check_product(ref, torch.from_numpy(ys[0]), L.x, f"gemm w{fmt} M={M} {N}x{K} row transpose")


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("M", [3, 8, 16])
@pytest.mark.parametrize("N,K,outl", [(129, 4096, True), (5000, 2048, False), (20000, 512, True),
                                      (33000, 256, False)])
def test_gemm_register_partials(fmt, M, N, K, outl):
    """The batched kernel with each wave's partial tiles in registers
    (batch_register_partials 1, where a workgroup has at most 8 row blocks)
    or in LDS (0): the same additions in the same order, so bit-identical Y
    on both layouts, within the bound; 1, 2, 5 and 9 row blocks per
    workgroup (the last keeps the LDS tiles)."""
    say(f"gemm register partials fmt={fmt} M={M} N={N} K={K} outliers={outl}")
    L = synthetic.small_layer(fmt, N, K, M=M, with_outliers=outl, seed=M + N + 2)
    ref = O.quantize_layer(fmt, L.W, L.profile if outl else None, L.ratio if outl else 0.0)
    dl = DeviceLayer(pack_host(fmt, L.W, L.profile if outl else None, L.ratio if outl else 0.0),
                     tiled=True)
    X = dev_fp16(L.x)
    for layout in ("rowmajor", "tiled"):
        ys = []
        for pr in (1, 0):
            Y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
            v = B.variant(gemm_kernel=2, gemm_rows=0, batch_register_partials=pr)
            if layout == "tiled":
                dl.gemm_tiled(X, Y, variant=v)
            else:
                dl.gemm(X, Y, variant=v)
            torch.cuda.synchronize()
            ys.append(Y.cpu().numpy())
        assert np.array_equal(ys[0], ys[1]), layout
        check_product(ref, torch.from_numpy(ys[0]), L.x,
                      f"gemm w{fmt} M={M} {N}x{K} register partials {layout}")


# ------------------------------------------------------- full-size layers


@pytest.mark.parametrize("fmt", [4, 5])
def test_full_w4_4096x4096_m1(fmt):
    L = synthetic.config1()
    say(f"full W{'4P' if fmt == 5 else '4'} 4096x4096 M=1")
    ref, dl = build(fmt, L.W)
    y, _ = run_gemv(dl, L.x)
    check_product(ref, y, L.x, f"fmt {fmt} 4096x4096")


def test_full_w2_14336x4096_outliers_m1():
    L = synthetic.config2()
    say("full W2 14336x4096 + outliers M=1")
    ref = O.quantize_layer(2, L.W, L.profile, L.ratio)
    dl = DeviceLayer(pack_host(2, L.W, L.profile, L.ratio), tiled=True)
    assert ref.n_out == 143
    y, _ = run_gemv(dl, L.x)
    check_product(ref, y, L.x, "W2 14336x4096")
    yt = run_gemv_tiled(dl, L.x)
    check_product(ref, yt, L.x, "W2 14336x4096 tiled")


@pytest.mark.parametrize("N,K", [(14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("M", [2, 4, 8, 16])
def test_full_w4_batched(N, K, M):
    say(f"full W4 batched {N}x{K} M={M}")
    L = synthetic.config4(M, N, K)
    ref = O.quantize_layer(4, L.W)
    dl = DeviceLayer(pack_host(4, L.W), tiled=True)
    X = dev_fp16(L.x)
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    dl.gemm(X, Y)
    Yt = torch.empty((M, N), dtype=torch.int16, device="cuda")
    dl.gemm_tiled(X, Yt)
    torch.cuda.synchronize()
    check_product(ref, Y, L.x, f"W4 {N}x{K} M={M}")
    check_product(ref, Yt, L.x, f"W4 {N}x{K} M={M} tiled")
    # M repeated GEMVs agree with the oracle too
    for m in range(M):
        y, _ = run_gemv(dl, L.x[m])
        check_product(ref, y, L.x[m:m + 1], f"W4 {N}x{K} gemv row {m}")


@pytest.mark.parametrize("fmt", [4, 5])
@pytest.mark.parametrize("N", [12300, 16400])
@pytest.mark.parametrize("M", [5, 8, 13])
def test_batched_several_row_blocks(fmt, N, M):
    """K = 4096 (8 slices on 8 waves) with 3 or 4 row blocks per workgroup
    and a ragged last one: every row within the bound on both layouts, with
    the rows staged in one round or in two (M = 13 on the tiled layout), and
    with the partial tiles in LDS or in registers."""
    K = 4096
    say(f"batched several row blocks fmt={fmt} {N}x{K} M={M}")
    L = synthetic.small_layer(fmt, N, K, M=M, with_outliers=False, seed=N % 97 + M)
    ref, dl = build_tiled(fmt, L.W, L.profile, L.ratio)
    X = dev_fp16(L.x)
    for name, var in (("default", B.variant(gemm_rows=0)),
                      ("register partials", B.variant(gemm_rows=0, batch_register_partials=1))):
        for layout in ("tiled", "rowmajor"):
            Y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
            if layout == "tiled":
                dl.gemm_tiled(X, Y, variant=var)
            else:
                dl.gemm(X, Y, variant=var)
            torch.cuda.synchronize()
            check_product(ref, Y, L.x, f"row blocks w{fmt} {N}x{K} M={M} {layout} {name}")


# ------------------------------------------------------ embedding row gather


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("V,K", [(1000, 4096), (77, 96), (300, 2080)])
def test_embed_gather_bit_exact(fmt, V, K):
    say(f"embed gather fmt={fmt} V={V} K={K}")
    W = synthetic.gaussian_weights(V, K, 0.02, 310, V, K)
    ref, dl = build(fmt, W)
    w_hat = ref.w_hat()
    rng = np.random.default_rng(V + K + fmt)
    ids = np.concatenate([[0, V - 1, 5, 5], rng.integers(0, V, 200), [-1, V, 2**31 - 1]])
    ids = ids.astype(np.int32)
    idd = torch.from_numpy(ids).cuda()
    out = torch.full((len(ids), K), -1, dtype=torch.int16, device="cuda")
    dl.embed(idd, out)
    torch.cuda.synchronize()
    got = _bits(host_fp16(out))
    valid = (ids >= 0) & (ids < V)
    assert np.array_equal(got[valid], _bits(w_hat[ids[valid]]))
    assert np.all(got[~valid] == 0)
    # an empty batch is a no-op
    dl.embed(idd[:0], out[:0])


# --------------------------------------- kurtosis-adaptive outlier policy


@pytest.mark.parametrize("fmt", [2, 4])
def test_gemv_kurtosis_policy_layer(fmt):
    say(f"gemv with kurtosis-selected outliers fmt={fmt}")
    rng = np.random.default_rng(12)
    N, K = 700, 4096
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    W[:, rng.choice(K, 60, replace=False)] *= 20.0      # leptokurtic column norms
    idx, r, kappa = O.select_outliers_kurtosis(W)
    assert r > 0.01 and len(idx) == int(np.floor(r * K))
    ref = O.quantize_layer(fmt, W, idx=idx)
    hl = pack_host(fmt, W, kurtosis=True)
    assert np.array_equal(hl.idx, ref.idx) and np.array_equal(hl.codes, ref.codes)
    dl = DeviceLayer(hl, tiled=True)
    x = synthetic.gaussian_x_fp16(1, K, 12, 0, fmt)
    y, _ = run_gemv(dl, x)
    check_product(ref, y, x, f"kurtosis policy w{fmt} n_out={ref.n_out} (row-major)")
    check_product(ref, run_gemv_tiled(dl, x), x, f"kurtosis policy w{fmt} (tiled)")


# ---------------------------------------------- runtime top-k refinement


@pytest.mark.parametrize("K,chunk,k", [(4096, 1024, 32), (14336, 1024, 32), (4096, 1024, 1),
                                       (2080, 1024, 64), (1024, 256, 255), (96, 64, 200),
                                       (4096, 512, 0), (28672, 1024, 128)])
def test_topk_chunks_exact(K, chunk, k):
    say(f"topk K={K} chunk={chunk} k={k}")
    rng = np.random.default_rng(K + k)
    x = rng.standard_normal(K).astype(np.float16)
    x[rng.choice(K, K // 8)] = x[1]        # exact ties in |x|
    x[rng.choice(K, K // 16)] = -x[1]
    x[::37] *= -40                          # large negative values
    n = B.wq_topk_count(K, chunk, k)
    exp = O.topk_chunks(x, k, chunk)
    assert n == len(exp)
    sel = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    B.wq_topk_chunks(dev_fp16(x), K, chunk, k, sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy()[:n], exp)


@pytest.mark.parametrize("fmt", [4, 2])
@pytest.mark.parametrize("N,K,k", [(14336 // 4, 4096, 32), (512, 2048, 8), (96, 1088, 100)])
def test_gemv_then_refine(fmt, N, K, k):
    say(f"gemv + top-k refinement fmt={fmt} N={N} K={K} k={k}")
    from bit_weight_only_gemv_amd.layer import refinement_host
    L = synthetic.small_layer(fmt, N, K, with_outliers=True, seed=k)
    ref, dl = build(fmt, L.W, L.profile, L.ratio)
    hl = pack_host(fmt, L.W, L.profile, L.ratio)
    rf = refinement_host(L.W, hl)
    rq, rs, rz = O.refinement_w4(L.W, ref.w_hat(), ref.idx)
    assert np.array_equal(rf.codes, O.pack_w4(rq))
    assert np.array_equal(_bits(rf.scales), _bits(rs)) and np.array_equal(_bits(rf.zeros), _bits(rz))
    dl.set_refinement(rf)
    x = L.x.reshape(-1)
    y, xd = run_gemv(dl, x)
    y_base = host_fp16(y).astype(np.float64).copy()
    n = B.wq_topk_count(K, 1024, k)
    sel = torch.empty(n, dtype=torch.int32, device="cuda")
    B.wq_topk_chunks(xd, K, 1024, k, sel)
    dl.refine(xd, y, sel, n)
    torch.cuda.synchronize()
    S = O.topk_chunks(x, k)
    assert np.array_equal(sel.cpu().numpy(), S)
    c_hat = O.dequant_w4(rq, rs, rz)
    # the add itself, on top of the GPU's own base output
    y_ref, a = O.refine_ref(y_base.astype(np.float16), x, S, c_hat)
    ok, worst = O.check_tolerance(host_fp16(y).astype(np.float64), y_ref, a)
    say(f"  refine add: worst |err|/bound = {worst:.4f}")
    assert ok
    # and the whole refined product against the oracle's
    y0, a0 = O.matvec_ref(ref.w_hat(), x, ref.idx, ref.wout)
    terms = x.astype(np.float64)[S][:, None] * c_hat.astype(np.float64)[S]
    ok2, worst2 = O.check_tolerance(host_fp16(y).astype(np.float64), y0[0] + terms.sum(0),
                                    a0[0] + np.abs(terms).sum(0))
    say(f"  refined product: worst |err|/bound = {worst2:.4f}")
    assert ok2
    # refinement moves the product toward the unquantized layer
    exact = L.W.astype(np.float64) @ x.astype(np.float64)
    assert np.abs(host_fp16(y) - exact).mean() < np.abs(y_base - exact).mean()


@pytest.mark.parametrize("fmt", [4, 2])
@pytest.mark.parametrize("N,K,chunk,k", [(14336 // 4, 4096, 1024, 32), (4096, 14336, 1024, 32),
                                         (512, 2048, 1024, 8), (96, 1088, 1024, 100),
                                         (64, 1024, 64, 64), (128, 4096, 1024, 1024)])
def test_refine_topk_fused(fmt, N, K, chunk, k):
    """One-launch selection + add: the same selection as wq_topk_chunks (copied
    out) and bit-identical y to wq_topk_chunks followed by wq_refine_add."""
    say(f"fused top-k refinement fmt={fmt} N={N} K={K} chunk={chunk} k={k}")
    from bit_weight_only_gemv_amd.layer import refinement_host
    L = synthetic.small_layer(fmt, N, K, with_outliers=True, seed=k + 1)
    hl = pack_host(fmt, L.W, L.profile, L.ratio)
    rf = refinement_host(L.W, hl)
    dl = DeviceLayer(hl)
    dl.set_refinement(rf)
    x = L.x.reshape(-1)
    y1, xd = run_gemv(dl, x)
    y2 = y1.clone()
    y_base = host_fp16(y1).astype(np.float64).copy()
    n = B.wq_topk_count(K, chunk, k)
    sel_out = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    dl.refine_topk(xd, y1, k, chunk, sel_out)
    sel = torch.empty(n, dtype=torch.int32, device="cuda")
    B.wq_topk_chunks(xd, K, chunk, k, sel)
    dl.refine(xd, y2, sel, n)
    torch.cuda.synchronize()
    S = O.topk_chunks(x, k, chunk)
    assert np.array_equal(sel_out.cpu().numpy(), S)
    assert np.array_equal(y1.cpu().numpy(), y2.cpu().numpy())
    rq, rs, rz = O.refinement_w4(L.W, O.quantize_layer(fmt, L.W, L.profile, L.ratio).w_hat(),
                                 hl.idx)
    y_ref, a = O.refine_ref(y_base.astype(np.float16), x, S, O.dequant_w4(rq, rs, rz))
    ok, worst = O.check_tolerance(host_fp16(y1).astype(np.float64), y_ref, a)
    say(f"  fused refine add: worst |err|/bound = {worst:.4f}")
    assert ok


def test_refine_topk_limits():
    """More than 4096 selected channels is refused before any launch; k = 0 is a no-op."""
    x = torch.zeros(8192, dtype=torch.int16, device="cuda")
    y = torch.zeros(64, dtype=torch.int16, device="cuda")
    c = torch.zeros(8192 * 32, dtype=torch.uint8, device="cuda")
    m = torch.zeros(8192 * 2, dtype=torch.int16, device="cuda")
    with pytest.raises(B.WQError):
        B.wq_refine_topk(c, m, m, 64, 8192, 64, 64, x, y)
    B.wq_refine_topk(c, m, m, 64, 8192, 1024, 0, x, y)
    B.wq_refine_topk(c, m, m, 64, 8192, 1024, 32, x, y)   # 256 channels of x = 0: adds 0
    torch.cuda.synchronize()
    assert int(y.abs().sum()) == 0


@pytest.mark.parametrize("fmt", [4, 2])
def test_refine_topk_with_selection_buffer(fmt):
    """Given a selection buffer, the call also takes more than 4096 selected
    channels (and more than 8 chunks) through the two-kernel path: same y as the
    two calls, S(x) as the oracle's, the add within the bound."""
    from bit_weight_only_gemv_amd.layer import refinement_host
    N, K, chunk, k = 64, 8192, 64, 40
    say(f"refine_topk with sel_out fmt={fmt} N={N} K={K} chunk={chunk} k={k}")
    L = synthetic.small_layer(fmt, N, K, with_outliers=True, seed=11)
    hl = pack_host(fmt, L.W, L.profile, L.ratio)
    dl = DeviceLayer(hl)
    dl.set_refinement(refinement_host(L.W, hl))
    x = L.x.reshape(-1)
    y1, xd = run_gemv(dl, x)
    y2 = y1.clone()
    y_base = host_fp16(y1).astype(np.float64).copy()
    n = B.wq_topk_count(K, chunk, k)
    assert n > 4096
    sel_out = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    dl.refine_topk(xd, y1, k, chunk, sel_out)
    sel = torch.empty(n, dtype=torch.int32, device="cuda")
    B.wq_topk_chunks(xd, K, chunk, k, sel)
    dl.refine(xd, y2, sel, n)
    torch.cuda.synchronize()
    S = O.topk_chunks(x, k, chunk)
    assert np.array_equal(sel_out.cpu().numpy(), S)
    assert np.array_equal(y1.cpu().numpy(), y2.cpu().numpy())
    rq, rs, rz = O.refinement_w4(L.W, O.quantize_layer(fmt, L.W, L.profile, L.ratio).w_hat(),
                                 hl.idx)
    y_ref, a = O.refine_ref(y_base.astype(np.float16), x, S, O.dequant_w4(rq, rs, rz))
    ok, worst = O.check_tolerance(host_fp16(y1).astype(np.float64), y_ref, a)
    say(f"  refine add: worst |err|/bound = {worst:.4f}")
    assert ok


# (fmt, N, K, chunk, k, outliers, fused): whether the one-launch kernel takes the
# shape (at most 4 units of chunk x 32 picks x row block per helper lane) or the
# call runs the product and then the selection and add
TILED_REFINE_CASES = [
    (2, 14336, 4096, 1024, 32, True, True),     # the default W2 layer: 2 row blocks per lane half
    (4, 4096, 14336, 1024, 32, True, True),     # 14 chunks on 5 helper waves
    (5, 3584, 4096, 1024, 32, True, True),      # fewer row blocks than compute units
    (4, 7168, 4096, 512, 48, False, True),      # two 32-pick groups per chunk
    (4, 28672, 1024, 1024, 16, True, True),     # 7 row blocks per workgroup: 4 per lane half
    (2, 512, 2048, 1024, 8, True, True),
    (4, 96, 1088, 1024, 100, True, True),       # k above a short last chunk (64 channels)
    (2, 64, 1024, 64, 64, True, True),          # 16 chunks on 10 helper waves
    (5, 96, 1088, 64, 1, True, True),           # 17 chunks of 64, one pick each
    (2, 32, 512, 64, 7, False, True),           # one 512-channel slice, smallest N
    (4, 256, 8192, 1024, 32, False, True),      # W4 without outliers: 16 waves, 8 helpers
    (5, 4096, 14336, 1024, 32, False, True),    # 14 chunks on 9 helpers of a 16-wave workgroup
    (4, 40960, 1024, 1024, 16, True, False),    # 10 row blocks per workgroup: two launches
    (4, 128, 4096, 1024, 1024, False, False),   # every channel picked: two launches
]


@pytest.mark.parametrize("fmt,N,K,chunk,k,outl,fused", TILED_REFINE_CASES)
def test_gemv_tiled_refine(fmt, N, K, chunk, k, outl, fused):
    """The tiled product with the refinement in the same launch: S(x) equal to the
    oracle's, y within the bound of the refined product, and the same
    selection and bound on the two-launch path (refine_fuse 0), which must be
    bit-identical to wq_gemv_tiled followed by wq_refine_topk.  Where the fused
    kernel runs, y is rounded once and differs from the two-launch y."""
    from bit_weight_only_gemv_amd.layer import refinement_host
    say(f"tiled gemv + refinement fmt={fmt} N={N} K={K} chunk={chunk} k={k} outliers={outl}")
    L = synthetic.small_layer(fmt, N, K, with_outliers=outl, seed=k + 3)
    ref, dl = build_tiled(fmt, L.W, L.profile, L.ratio)
    hl = pack_host(fmt, L.W, L.profile, L.ratio)
    dl.set_refinement(refinement_host(L.W, hl))
    x = L.x.reshape(-1)
    xd = dev_fp16(x)
    n = B.wq_topk_count(K, chunk, k)
    S = O.topk_chunks(x, k, chunk)
    rq, rs, rz = O.refinement_w4(L.W, ref.w_hat(), ref.idx)
    c_hat = O.dequant_w4(rq, rs, rz)
    y0, a0 = O.matvec_ref(ref.w_hat(), x, ref.idx, ref.wout)
    terms = x.astype(np.float64)[S][:, None] * c_hat.astype(np.float64)[S]
    outs = {}
    # W4 / W4P layers without outliers also run their 12-wave kernel (refine_wide 0)
    modes = ("1", "1w0", "0") if fmt != 2 and not outl else ("1", "0")
    for mode in modes:
        var = B.variant(refine_fuse=int(mode[0]), refine_wide=0 if mode == "1w0" else 1)
        y = torch.full((N,), -1, dtype=torch.int16, device="cuda")
        sel = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        dl.gemv_tiled_refine(xd, y, k, chunk, sel, variant=var)
        torch.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), S)
        ok, worst = O.check_tolerance(host_fp16(y).astype(np.float64), y0[0] + terms.sum(0),
                                      a0[0] + np.abs(terms).sum(0))
        say(f"  mode {mode}: worst |err|/bound = {worst:.4f}")
        assert ok
        outs[mode] = y.cpu().numpy()
    # the two-launch path is exactly the product followed by the fused selection + add
    y2 = torch.full((N,), -1, dtype=torch.int16, device="cuda")
    dl.gemv_tiled(xd, y2)
    dl.refine_topk(xd, y2, k, chunk)
    torch.cuda.synchronize()
    assert np.array_equal(outs["0"], y2.cpu().numpy())
    if not fused:
        assert np.array_equal(outs["1"], outs["0"])
    elif N >= 2048:
        assert not np.array_equal(outs["1"], outs["0"])
    # refinement moves the product toward the unquantized layer wherever it does
    # so clearly in float64 (a few picks among thousands of channels, or picks
    # that are all outlier columns with zero refinement, barely move it)
    exact = L.W.astype(np.float64) @ x.astype(np.float64)
    y_ref = outs["1"].view(np.float16).astype(np.float64)
    base = torch.full((N,), -1, dtype=torch.int16, device="cuda")
    dl.gemv_tiled(xd, base)
    torch.cuda.synchronize()
    y_base = host_fp16(base).astype(np.float64)
    gain = np.abs(y0[0] + terms.sum(0) - exact).mean() / np.abs(y0[0] - exact).mean()
    say(f"  float64 refined / base mean error = {gain:.4f}")
    if gain < 0.98:
        assert np.abs(y_ref - exact).mean() < np.abs(y_base - exact).mean()


@pytest.mark.parametrize("fmt", [4, 2])
def test_gemv_tiled_refine_zero_chunk(fmt):
    """A chunk of x that is all zeros (and one of all-equal magnitudes): the
    picks are its lowest indices (ties go to the lower index), and their
    refinement adds nothing (zero activations) or exactly the oracle's terms."""
    from bit_weight_only_gemv_amd.layer import refinement_host
    N, K, chunk, k = 256, 3072, 1024, 16
    say(f"tiled gemv + refinement with a zero chunk fmt={fmt}")
    L = synthetic.small_layer(fmt, N, K, with_outliers=True, seed=5)
    ref, dl = build_tiled(fmt, L.W, L.profile, L.ratio)
    hl = pack_host(fmt, L.W, L.profile, L.ratio)
    dl.set_refinement(refinement_host(L.W, hl))
    x = L.x.reshape(-1).copy()
    x[:chunk] = 0.0
    x[chunk:2 * chunk] = np.where(np.arange(chunk) % 2, 0.5, -0.5).astype(np.float16)
    n = B.wq_topk_count(K, chunk, k)
    S = O.topk_chunks(x, k, chunk)
    assert np.array_equal(S[:k], np.arange(k)) and np.array_equal(S[k:2 * k], chunk + np.arange(k))
    y = torch.full((N,), -1, dtype=torch.int16, device="cuda")
    sel = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    dl.gemv_tiled_refine(dev_fp16(x), y, k, chunk, sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), S)
    rq, rs, rz = O.refinement_w4(L.W, ref.w_hat(), ref.idx)
    c_hat = O.dequant_w4(rq, rs, rz)
    y0, a0 = O.matvec_ref(ref.w_hat(), x, ref.idx, ref.wout)
    terms = x.astype(np.float64)[S][:, None] * c_hat.astype(np.float64)[S]
    ok, worst = O.check_tolerance(host_fp16(y).astype(np.float64), y0[0] + terms.sum(0),
                                  a0[0] + np.abs(terms).sum(0))
    say(f"  worst |err|/bound = {worst:.4f}")
    assert ok


@pytest.mark.parametrize("gpw", ["1", "2", "4"])
@pytest.mark.parametrize("N,K", [(96, 2048), (14336 // 4, 4096), (4096, 14336 // 2)])
def test_refine_groups_per_workgroup(gpw, N, K):
    """Workgroups of 1, 2 or 4 row groups (a ragged last workgroup included) sum
    every group in the same order: the fused and two-call paths stay
    bit-identical to each other and to the one-group default."""
    say(f"refinement with {gpw} groups per workgroup N={N} K={K}")
    from bit_weight_only_gemv_amd.layer import refinement_host
    L = synthetic.small_layer(4, N, K, with_outliers=True, seed=3)
    hl = pack_host(4, L.W, L.profile, L.ratio)
    dl = DeviceLayer(hl)
    dl.set_refinement(refinement_host(L.W, hl))
    x = L.x.reshape(-1)
    y0, xd = run_gemv(dl, x)
    n = B.wq_topk_count(K, 1024, 32)
    sel = torch.empty(n, dtype=torch.int32, device="cuda")
    B.wq_topk_chunks(xd, K, 1024, 32, sel)
    ya = y0.clone()
    dl.refine(xd, ya, sel, n)                  # default grouping
    var = B.variant(refine_groups=int(gpw))
    yb, yc = y0.clone(), y0.clone()
    dl.refine(xd, yb, sel, n, variant=var)
    dl.refine_topk(xd, yc, 32, variant=var)
    torch.cuda.synchronize()
    assert np.array_equal(ya.cpu().numpy(), yb.cpu().numpy())
    assert np.array_equal(ya.cpu().numpy(), yc.cpu().numpy())


# ------------------------------------------- degenerate values and boundaries


def _special_layer(fmt, N, K, seed):
    """Weights with constant groups (the scale floor flushes to FP16 0), all-zero
    rows, groups of a huge range next to tiny ones; activations with exact
    zeros, negative zeros and FP16 subnormals; outlier columns at 0, K - 1 and
    on both sides of 32-, 256- and 512-channel boundaries."""
    rng = np.random.default_rng(seed)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    W[1, :] = 0.0
    W[2, 64:96] = 0.37                       # one constant group
    W[3, :] = -1.25                          # constant row
    W[4, 128:160] *= 1e4                     # a huge-range group
    W[5, 160:192] *= 1e-6                    # a tiny one
    x = rng.standard_normal(K).astype(np.float16)
    x[::7] = 0.0
    x[3::11] = np.float16(-0.0)
    x[5::13] = np.float16(2.0 ** -20)        # subnormal
    x[6::17] = np.float16(-(2.0 ** -24))     # smallest subnormal
    cols = np.array(sorted({0, 31, 32, 255, 256, 511, 512, 513, K - 1}), np.int64)
    profile = np.full(K, 1e-9)
    profile[cols] = 1e9
    ratio = (len(cols) + 0.5) / K
    return W, x, profile, ratio, cols


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("N,K", [(48, 1024), (160, 4096)])
def test_special_values_and_boundary_outliers(fmt, N, K):
    say(f"special values fmt={fmt} N={N} K={K}")
    W, x, profile, ratio, cols = _special_layer(fmt, N, K, seed=N + K)
    ref = O.quantize_layer(fmt, W, profile, ratio)
    assert np.array_equal(ref.idx, cols)
    hl = pack_host(fmt, W, profile, ratio)
    assert np.array_equal(hl.codes, ref.codes) and np.array_equal(hl.idx, ref.idx)
    dl = DeviceLayer(hl, tiled=True)
    # bit-exact dequantization, constant and zero groups included
    out = torch.empty((N, K), dtype=torch.int16, device="cuda")
    dl.dequant(out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16),
                          np.asarray(ref.w_hat(), np.float16).view(np.uint16))
    for mode in (0, 2):
        y, _ = run_gemv(dl, x, variant=B.variant(gemv_kernel=mode))
        check_product(ref, y, x, f"special w{fmt} gemv mode {mode}")
    check_product(ref, run_gemv_tiled(dl, x), x, f"special w{fmt} tiled")
    X = np.stack([x, -x, x[::-1].copy()])
    for mode in (0, 1):
        Y = torch.full((3, N), -1, dtype=torch.int16, device="cuda")
        dl.gemm(dev_fp16(X), Y, variant=B.variant(gemm_kernel=mode))
        torch.cuda.synchronize()
        check_product(ref, Y, X, f"special w{fmt} gemm M=3 mode {mode}")


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("N,K", [(48, 1024), (160, 4096), (37, 14336)])
@pytest.mark.parametrize("M", [5, 8, 10, 16])
def test_batched_boundary_outliers(fmt, N, K, M):
    """The batched kernels (both layouts, rows staged or not) on the special
    layer: outlier columns at 0 and K - 1, odd and even, on both sides of the
    32-, 256- and 512-channel boundaries, so each gathered activation comes
    from either half of its aligned 4-byte word."""
    say(f"batched boundary outliers fmt={fmt} N={N} K={K} M={M}")
    W, x, profile, ratio, cols = _special_layer(fmt, N, K, seed=N + K + M)
    ref = O.quantize_layer(fmt, W, profile, ratio)
    dl = DeviceLayer(pack_host(fmt, W, profile, ratio), tiled=True)
    rng = np.random.default_rng(M)
    X = np.stack([x] + [(x * np.float16(rng.uniform(-2, 2))).astype(np.float16)
                        for _ in range(M - 1)])
    Xd = dev_fp16(X)
    for layout in ("tiled", "rowmajor"):
        for xt in (0, 1):
            var = B.variant(gemm_rows=0, batch_row_transpose=xt)
            Y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
            if layout == "tiled":
                dl.gemm_tiled(Xd, Y, variant=var)
            else:
                dl.gemm(Xd, Y, variant=var)
            torch.cuda.synchronize()
            check_product(ref, Y, X, f"boundary w{fmt} M={M} {layout} xt={xt}")


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("lds_path", ["0", "1"])
@pytest.mark.parametrize("rpw", ["1", "2", "4"])
@pytest.mark.parametrize("N,K,outl", [(129, 4096, True), (37, 14336, False), (300, 2080, True)])
def test_gemv_valu_launch_variants(fmt, lds_path, rpw, N, K, outl):
    """The VALU M = 1 kernels with x staged in LDS or kept in registers, and
    1, 2 or 4 rows per wave step."""
    var = B.variant(gemv_kernel=0, gemv_lds_x=int(lds_path), gemv_rows_per_wave=int(rpw))
    say(f"gemv VALU fmt={fmt} lds={lds_path} rows/wave={rpw} N={N} K={K} outliers={outl}")
    L = synthetic.small_layer(fmt, N, K, with_outliers=outl, seed=N + int(rpw))
    ref, dl = build(fmt, L.W, L.profile, L.ratio)
    y, _ = run_gemv(dl, L.x, variant=var)
    check_product(ref, y, L.x, f"valu w{fmt} lds={lds_path} rpw={rpw} {N}x{K}")


@pytest.mark.parametrize("nbytes", [4096, 26157632, 104555648])
def test_read_probe_geometries(nbytes):
    """The streaming-read probes the benchmark times against: every geometry it
    uses launches, returns, and leaves the sink as it was (the probe writes a
    word only for data that a buffer of ones cannot hold)."""
    say(f"read probe {nbytes} B")
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    for blocks, threads, ring in [(0, 256, 1), (0, 256, 2), (0, 256, 4), (0, 1024, 8),
                                  (256, 256, 1), (512, 512, 16), (4096, 64, 2)]:
        B.wq_read_probe_geom(buf, nbytes, sink, blocks, threads, ring)
    B.wq_read_probe(buf, nbytes, sink[:B.wq_read_probe_sink_words(nbytes)])
    torch.cuda.synchronize()
    assert int(sink[B.wq_read_probe_sink_words(nbytes):].abs().sum()) == 0
