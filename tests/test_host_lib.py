"""The library's host encoder (C ABI, CPU) against the oracle: byte-for-byte
equality of codes, FP16 scales/zeros, outlier indices, the FP16 outlier slab
and host-dequantized FP16 weights.  Also: the shared library loads and exports
every symbol include/wq.h declares, and argument errors come back as codes."""

import ctypes
import os
import re

import numpy as np
import pytest

import bit_weight_only_gemv_amd as B
import oracle as O
import synthetic
from conftest import ROOT


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def _same_layer(fmt, W, profile=None, ratio=0.0):
    ref = O.quantize_layer(fmt, W, profile, ratio)
    from bit_weight_only_gemv_amd.layer import pack_host
    lib = pack_host(fmt, W, profile, ratio)
    assert np.array_equal(lib.idx, ref.idx)
    assert np.array_equal(_bits(lib.wout), _bits(ref.wout))
    assert np.array_equal(lib.codes, ref.codes)
    assert np.array_equal(_bits(lib.scales), _bits(ref.scale))
    assert np.array_equal(_bits(lib.zeros), _bits(ref.zero))
    wh = B.wq_dequant_host(fmt, lib.codes, lib.scales, lib.zeros, ref.N, ref.K)
    assert np.array_equal(_bits(wh), _bits(ref.w_hat()))
    return ref, lib


# ---------------------------------------------------------------- exports


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "wq.h")).read()
    declared = set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", hdr))
    assert declared, "no declarations parsed"
    lib = B.load()
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(B.SIGNATURES), declared ^ set(B.SIGNATURES)
    assert lib.wq_status_str(0) == b"ok"


# ------------------------------------------------------- encoder equality


@pytest.mark.parametrize("fmt", [4, 2])
@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (37, 4096), (64, 14336 // 4)])
def test_encoder_matches_oracle_plain(fmt, N, K):
    W = synthetic.gaussian_weights(N, K, 0.02, 200, N, K)
    _same_layer(fmt, W)


@pytest.mark.parametrize("fmt", [4, 2])
def test_encoder_matches_oracle_with_outliers(fmt):
    L = synthetic.small_layer(fmt, 300, 4096, with_outliers=True, seed=7)
    ref, lib = _same_layer(fmt, L.W, L.profile, L.ratio)
    assert ref.n_out == 143


def test_encoder_edge_groups():
    """Constant, all-zero, one-sided, heavy-tailed and tiny groups (subnormal
    FP16 scales) encode identically."""
    rng = np.random.default_rng(4)
    W = rng.standard_normal((16, 256), dtype=np.float32) * np.float32(0.02)
    W[0, :32] = 0.0
    W[1, :32] = 0.37
    W[2, :32] = -np.abs(W[2, :32]) - 0.1
    W[3, :] *= rng.standard_cauchy(256).astype(np.float32)
    W[4, :] *= np.float32(1e-5)                  # FP16 scales in the subnormal range
    W[5, :] *= np.float32(1e3)
    W[6, ::7] = 0.0
    for fmt in (4, 2):
        _same_layer(fmt, W)


def test_fp16_rounding_of_outlier_slab_exhaustive():
    """The host converter rounds float32 to FP16 to nearest-even exactly like
    numpy: every FP16 value, every midpoint, and their float32 neighbours."""
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    mids = (h[:-1].astype(np.float64) + h[1:].astype(np.float64)) / 2
    mids = mids.astype(np.float32)
    vals = np.concatenate([h, mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf)),
                           np.array([65504, 65519.99, 65520, 7e4, 1e-8, 3e-8, 2.98e-8], np.float32)])
    vals = np.concatenate([vals, -vals])
    pad = (-len(vals)) % 32
    vals = np.concatenate([vals, np.zeros(pad, np.float32)])
    W = vals.reshape(-1, 32)
    idx = np.arange(32, dtype=np.int32)
    dense, wout = B.wq_split_outliers(W, idx)
    assert np.array_equal(_bits(wout), _bits(W.astype(np.float16)))
    assert np.all(dense == 0)


@pytest.mark.slow
def test_encoder_matches_oracle_w4_4096x4096():
    L = synthetic.config1()
    _same_layer(4, L.W)


@pytest.mark.slow
def test_encoder_matches_oracle_w2_14336x4096_outliers():
    L = synthetic.config2()
    ref, lib = _same_layer(2, L.W, L.profile, L.ratio)
    assert ref.n_out == 143 and set(L.spikes.tolist()) <= set(ref.idx.tolist())


def _same_layer_chunked(fmt, W, profile=None, ratio=0.0, chunk=4096):
    """Byte equality of the library's encoding of the whole layer with the
    oracle's, the oracle taking the rows in chunks (outlier columns chosen from
    the whole matrix; a row's encoding depends on nothing else)."""
    from bit_weight_only_gemv_amd.layer import pack_host
    lib = pack_host(fmt, W, profile, ratio)
    idx = O.select_outliers(W, profile, ratio) if profile is not None else np.zeros(0, np.int32)
    assert np.array_equal(lib.idx, idx)
    for r0 in range(0, W.shape[0], chunk):
        rows = slice(r0, min(W.shape[0], r0 + chunk))
        dense, wout = O.split_outliers(W[rows], idx)
        if fmt == 4:
            q, sc, ze, _ = O.quantize_w4(dense)
            codes = O.pack_w4(q)
        else:
            q, sc, ze = O.quantize_w2(dense)
            codes = O.pack_w2(q)
        assert np.array_equal(lib.codes[rows], codes), f"codes, rows {r0}.."
        assert np.array_equal(_bits(lib.scales[rows]), _bits(sc)), f"scales, rows {r0}.."
        assert np.array_equal(_bits(lib.zeros[rows]), _bits(ze)), f"zeros, rows {r0}.."
        if len(idx):
            assert np.array_equal(_bits(lib.wout[rows]), _bits(wout)), f"slab, rows {r0}.."
    return lib


@pytest.mark.slow
@pytest.mark.parametrize("N,K", [(14336, 4096), (4096, 14336)])
def test_encoder_matches_oracle_config4_full(N, K):
    _same_layer_chunked(4, synthetic.config4(2, N, K).W)


@pytest.mark.slow
@pytest.mark.parametrize("N,K", [(28672, 8192), (8192, 28672)])
def test_encoder_matches_oracle_config5_full(N, K):
    L = synthetic.config5(N, K, 1)
    lib = _same_layer_chunked(2, L.W, L.profile, L.ratio)
    assert lib.n_out == int(np.floor(0.035 * K))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["q", "k", "gate", "down", "lm_head"])
def test_encoder_matches_oracle_config3_shapes(name):
    """One layer of each distinct shape of the Llama-3-8B-shaped sweep
    (q and o 4096 x 4096, k and v 1024 x 4096, gate and up 14336 x 4096, down
    4096 x 14336, the LM head 128256 x 4096)."""
    layer, proj, nm, N, K = next(s for s in synthetic.config3_shapes() if s[2] == name)
    _same_layer_chunked(4, synthetic.config3_layer(layer, proj, N, K, nm).W)


# ------------------------------------------------------------- error codes


def test_error_codes():
    lib = B.load()
    W = np.zeros((4, 64), np.float32)
    out = np.zeros(4096, np.uint8)
    p = W.ctypes.data_as(ctypes.c_void_p)
    o = out.ctypes.data_as(ctypes.c_void_p)
    assert lib.wq_quantize_w4(p, 4, 64, 64, o, o, o) == B._lib.WQ_ERR_UNSUPPORTED
    assert lib.wq_quantize_w4(p, 4, 48, 32, o, o, o) == B._lib.WQ_ERR_UNSUPPORTED
    assert b"K" in lib.wq_last_error()
    assert lib.wq_quantize_w2(None, 4, 64, 32, o, o, o) == B._lib.WQ_ERR_INVALID_ARG
    assert lib.wq_quantize_w2(p, 0, 64, 32, o, o, o) == B._lib.WQ_ERR_INVALID_ARG
    bad = np.array([3, 3], np.int32)
    with pytest.raises(B.WQError) as e:
        B.wq_split_outliers(W, bad)
    assert e.value.status == B._lib.WQ_ERR_INVALID_ARG
    with pytest.raises(B.WQError):
        B.wq_split_outliers(W, np.array([64], np.int32))
    with pytest.raises(B.WQError):
        B.wq_select_outliers(W, np.ones(64), 1.5)
    with pytest.raises(B.WQError):
        B.wq_dequant_host(3, out, out, out, 4, 64)
    # device entry points reject bad arguments before touching the GPU
    fake = ctypes.c_void_p(4096)
    assert lib.wq_gemv_w4(fake, fake, fake, 0, 64, None, None, 0, 1, fake, fake, None) == -1
    assert lib.wq_gemv_w2(fake, fake, fake, 8, 40, None, None, 0, 1, fake, fake, None) == -2
    assert lib.wq_gemv_w2(fake, fake, fake, 8, 64, None, None, 3, 1, fake, fake, None) == -1
    assert lib.wq_gemv_w4(fake, fake, fake, 8, 64, None, None, 0, 1, ctypes.c_void_p(4098),
                          fake, None) == -1
    assert lib.wq_gemm_wq(4, fake, fake, fake, 8, 64, None, None, 0, 1, fake, 17, fake, None) == -2
    assert lib.wq_gemm_wq(4, fake, fake, fake, 8, 64, None, None, 0, 1, fake, 0, fake, None) == -1
    assert lib.wq_gemm_wq(3, fake, fake, fake, 8, 64, None, None, 0, 1, fake, 2, fake, None) == -1
    assert lib.wq_gemv_w4(fake, fake, fake, 8, 65536 + 32, None, None, 0, 1, fake, fake, None) == -2
    assert lib.wq_read_probe(fake, 15, fake, None) == -1
    # the geometry probe: bad thread counts, ring, sizes and grids fail before any launch
    assert lib.wq_read_probe_geom(fake, 4096, fake, 0, 96, 1, None) == -1
    assert lib.wq_read_probe_geom(fake, 4096, fake, 0, 256, 3, None) == -1
    assert lib.wq_read_probe_geom(fake, 4100, fake, 0, 256, 1, None) == -1
    assert lib.wq_read_probe_geom(fake, 1 << 31, fake, 0, 256, 1, None) == -1
    assert lib.wq_read_probe_geom(fake, 4096, fake, -1, 256, 1, None) == -1
    assert lib.wq_read_probe_geom(fake, (1 << 31) - 4096, fake, 0, 64, 1, None) == -1
    assert lib.wq_read_probe_geom(fake, 4096, fake, 65536, 1024, 16, None) == -1
    assert lib.wq_embed_gather(3, fake, fake, fake, 8, 64, fake, 1, fake, None) == -1
    assert lib.wq_embed_gather(4, fake, fake, fake, 8, 40, fake, 1, fake, None) == -2
    assert lib.wq_embed_gather(4, fake, fake, fake, 8, 64, fake, -1, fake, None) == -1
    assert lib.wq_embed_gather(4, fake, fake, fake, 8, 64, None, 0, None, None) == 0
    assert lib.wq_embed_gather(4, fake, fake, fake, 8, 64, None, 2, fake, None) == -1
    # top-k selection and refinement add
    assert B.wq_topk_count(4096, 1024, 32) == 128 and B.wq_topk_count(2080, 1024, 64) == 160
    assert B.wq_topk_count(100, 64, 200) == 100 and B.wq_topk_count(64, 64, 0) == 0
    assert lib.wq_topk_count(10, 0, 1) < 0
    assert lib.wq_topk_chunks(fake, 4096, 1000, 8, fake, None) == -2
    assert lib.wq_topk_chunks(fake, 4096, 2048, 8, fake, None) == -2
    assert lib.wq_topk_chunks(fake, 4010, 1024, 8, fake, None) == -2
    assert lib.wq_topk_chunks(fake, 4096, 1024, -1, fake, None) == -1
    assert lib.wq_topk_chunks(None, 4096, 1024, 0, None, None) == 0
    assert lib.wq_refine_add(fake, fake, fake, 48, 64, fake, 1, fake, fake, None) == -2
    assert lib.wq_refine_add(fake, fake, fake, 64, 64, fake, 65, fake, fake, None) == -1
    assert lib.wq_refine_add(None, None, None, 64, 64, None, 0, None, None, None) == 0
    assert lib.wq_refine_topk(fake, fake, fake, 48, 64, 64, 1, fake, fake, None, None) == -2
    assert lib.wq_refine_topk(fake, fake, fake, 64, 64, 32, 1, fake, fake, None, None) == -2
    assert lib.wq_refine_topk(fake, fake, fake, 64, 8192, 64, 64, fake, fake, None, None) == -2
    assert lib.wq_refine_topk(fake, fake, fake, 64, 64, 64, -1, fake, fake, None, None) == -1
    assert lib.wq_refine_topk(None, None, None, 64, 64, 64, 0, None, None, None, None) == 0
    assert lib.wq_refine_topk(fake, fake, fake, 64, 64, 64, 1, None, fake, None, None) == -1
    # two-row tiled product
    assert lib.wq_gemm_tiled(4, fake, 64, 512, None, 0, fake, 5, fake, None) == -2
    assert lib.wq_gemm_tiled(2, fake, 64, 512, None, 0, fake, 3, fake, None) == -2
    assert lib.wq_gemm_tiled(4, fake, 64, 512, None, 0, fake, 0, fake, None) == -1
    assert lib.wq_gemm_tiled(4, None, 64, 512, None, 0, fake, 2, fake, None) == -1
    assert lib.wq_gemm_tiled(3, fake, 64, 512, None, 0, fake, 2, fake, None) == -1
    # tiled product with the refinement fused in
    R = lib.wq_gemv_tiled_refine
    assert R(3, fake, 64, 512, None, 0, fake, fake, fake, fake, fake, 1024, 8, None, None) == -1
    assert R(4, fake, 48, 512, None, 0, fake, fake, fake, fake, fake, 1024, 8, None, None) == -2
    assert R(4, fake, 64, 512, None, 0, fake, fake, fake, fake, fake, 32, 8, None, None) == -2
    assert R(4, fake, 64, 512, None, 0, fake, fake, fake, fake, fake, 2048, 8, None, None) == -2
    assert R(4, fake, 64, 512, None, 0, fake, fake, fake, fake, fake, 1024, -1, None, None) == -1
    assert R(4, fake, 64, 512, None, -1, fake, fake, fake, fake, fake, 1024, 8, None, None) == -1
    assert R(4, fake, 64, 512, None, 0, fake, fake, None, fake, fake, 1024, 8, None, None) == -1
    assert R(4, fake, 64, 512, None, 0, None, fake, fake, fake, fake, 1024, 0, None, None) == -1


# ------------------------------------------------- W4P packed zero points


@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (37, 4096), (5, 224)])
def test_packed_zeros_match_oracle(N, K):
    W = synthetic.gaussian_weights(N, K, 0.02, 201, N, K)
    W[:, :32] -= 1.0     # all-negative first group: its zero point clamps to 15
    ref = O.quantize_layer(5, W)
    from bit_weight_only_gemv_amd.layer import pack_host
    lib = pack_host(5, W)
    assert np.array_equal(lib.codes, ref.codes)
    assert np.array_equal(lib.zeros, ref.zero_packed)
    assert lib.zeros.shape == (N, (K // 32 + 1) // 2)
    wh = B.wq_dequant_host(5, lib.codes, lib.scales, lib.zeros, N, K)
    assert np.array_equal(_bits(wh), _bits(ref.w_hat()))
    # and the same values as the W4 layer with FP16 zero points
    w4 = B.wq_dequant_host(4, ref.codes, ref.scale, ref.zero, N, K)
    assert np.array_equal(_bits(wh), _bits(w4))


def test_packed_zeros_reject_non_integer():
    z = np.array([[3.0, 2.5]], np.float16)
    with pytest.raises(B.WQError):
        B.wq_pack_zeros_w4(z, 1, 64)
    with pytest.raises(B.WQError):
        B.wq_pack_zeros_w4(np.array([[16.0, 0.0]], np.float16), 1, 64)
    assert B.wq_pack_zeros_w4(np.array([[15.0, 0.0]], np.float16), 1, 64).tolist() == [[15]]


# ------------------------------------------ kurtosis-adaptive outlier policy


@pytest.mark.parametrize("case", ["gaussian", "heavy", "gamma", "tiny", "constant"])
def test_kurtosis_policy_matches_oracle(case):
    rng = np.random.default_rng(11)
    N, K = 48, 2048
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    gamma = None
    if case == "heavy":
        W[:, rng.choice(K, 30, replace=False)] *= 25.0
    elif case == "gamma":
        gamma = np.abs(rng.standard_normal(K)) + 0.1
        gamma[rng.choice(K, 8, replace=False)] = 60.0
    elif case == "tiny":
        W = W[:3, :64].copy()
    elif case == "constant":
        W = np.ones((5, 256), np.float32)    # equal saliencies: kappa 0, r = r_base
    idx, r, kappa = B.wq_select_outliers_kurtosis(W, gamma)
    ridx, rr, rk = O.select_outliers_kurtosis(W, gamma)
    assert np.array_equal(idx, ridx)
    assert r == rr and kappa == rk        # the same float64 operations in the same order
    # and a layer packed with it equals the oracle's layer with those columns
    from bit_weight_only_gemv_amd.layer import pack_host
    lib = pack_host(2, W, kurtosis=True, kurtosis_gamma=gamma)
    ref = O.quantize_layer(2, W, idx=ridx)
    assert np.array_equal(lib.idx, ref.idx) and np.array_equal(lib.codes, ref.codes)
    assert np.array_equal(_bits(lib.wout), _bits(ref.wout))


def test_kurtosis_policy_errors():
    W = np.zeros((4, 64), np.float32)
    with pytest.raises(B.WQError):
        B.wq_select_outliers_kurtosis(W, None, r_base=0.0)
    lib = B.load()
    n = ctypes.c_int64(0)
    p = W.ctypes.data_as(ctypes.c_void_p)
    assert lib.wq_select_outliers_kurtosis(None, 4, 64, None, 0.01, None, 0, ctypes.byref(n),
                                           None, None) == -1
    # a capacity below floor(r K) is rejected (r >= 0.01 -> at least 10 of 1024 columns)
    W2 = np.random.default_rng(0).standard_normal((4, 1024)).astype(np.float32)
    idx = np.zeros(4, np.int32)
    assert lib.wq_select_outliers_kurtosis(W2.ctypes.data_as(ctypes.c_void_p), 4, 1024, None,
                                           0.01, idx.ctypes.data_as(ctypes.c_void_p), 4,
                                           ctypes.byref(n), None, None) == -1
    assert p is not None


# ------------------------------------------------ refinement columns (C ABI)


@pytest.mark.parametrize("fmt", [4, 5, 2])
@pytest.mark.parametrize("N,K,outl", [(32, 64, False), (96, 1088, True), (256, 4096, True),
                                      (64, 2080, False)])
def test_refinement_columns_match_oracle(fmt, N, K, outl):
    """wq_refinement_w4 (StrataFlux section 3.2.1): the residual of the packed
    layer with the outlier columns zeroed, W4-encoded transposed, byte for byte
    the oracle's refinement_w4."""
    from bit_weight_only_gemv_amd.layer import pack_host, refinement_host
    L = synthetic.small_layer(fmt, N, K, with_outliers=outl, seed=N + K)
    hl = pack_host(fmt, L.W, L.profile, L.ratio)
    ref = O.quantize_layer(fmt, L.W, L.profile, L.ratio)
    assert (ref.n_out > 0) == outl
    rq, rs, rz = O.refinement_w4(L.W, ref.w_hat(), ref.idx if outl else None)
    rf = refinement_host(L.W, hl)
    assert np.array_equal(rf.codes, O.pack_w4(rq))
    assert np.array_equal(_bits(rf.scales), _bits(rs))
    assert np.array_equal(_bits(rf.zeros), _bits(rz))
    if outl:   # the outlier channels' refinement rows decode to exactly 0
        c_hat = O.dequant_w4(O.unpack_w4(rf.codes), rf.scales, rf.zeros)
        assert np.all(c_hat[hl.idx] == 0)


def test_refinement_columns_errors():
    W = np.zeros((48, 64), np.float32)
    codes, sc, ze = B.wq_quantize_w4(W)
    with pytest.raises(B.WQError) as e:            # N not a multiple of 32
        B.wq_refinement_w4(4, W, codes, sc, ze)
    assert e.value.status == B._lib.WQ_ERR_UNSUPPORTED
    W = np.zeros((32, 64), np.float32)
    codes, sc, ze = B.wq_quantize_w4(W)
    for bad in ([5, 5], [70], [-1], [9, 3]):       # not strictly increasing in [0, K)
        with pytest.raises(B.WQError) as e:
            B.wq_refinement_w4(4, W, codes, sc, ze, np.array(bad, np.int32))
        assert e.value.status == B._lib.WQ_ERR_INVALID_ARG
    with pytest.raises(B.WQError):
        B.wq_refinement_w4(3, W, codes, sc, ze)
