"""The tiled M = 1 layout (include/wq.h, "Tiled layout"): the library's host
rearrangement against an independent numpy construction written from the
header's index formulas, byte for byte, on ragged shapes (N not a multiple of
16, K not a multiple of 512, n_out not a multiple of 8, no outliers).  The
layout moves bytes only, so random arrays serve as inputs.  Also: the size
query and the argument errors."""

import ctypes

import numpy as np
import pytest

import bit_weight_only_gemv_amd as B


def ceil_div(a, b):
    return -(-a // b)


def expected_tiled(fmt, codes, scales, zeros, wout, N, K):
    n_out = 0 if wout is None else wout.shape[1]
    nrb, nks, nch = ceil_div(N, 16), ceil_div(K, 512), ceil_div(n_out, 8)
    sb = 128 if fmt == 2 else 256
    up = lambda v: ceil_div(v, 256) * 256  # noqa: E731
    meta_off = up(nrb * nks * 16 * sb)
    slab_off = meta_off + up(nrb * nks * (640 if fmt == 5 else 1024))
    total = slab_off + up(nrb * nch * 256)
    out = np.zeros(total, np.uint8)
    # codes: tile (b, s) byte 1024 u + 16 (n + 16 r) + c = codes[16 b + n][s sb + 64 u + 16 r + c]
    cp = np.zeros((nrb * 16, nks * sb), np.uint8)
    cp[:N, :codes.shape[1]] = codes
    t = cp.reshape(nrb, 16, nks, sb // 64, 4, 16)          # b, n, s, u, r, c
    out[:nrb * nks * 16 * sb] = t.transpose(0, 2, 3, 4, 1, 5).reshape(-1)
    # meta: entry 8 (n + 16 r) + i = scales[16 b + n][16 s + 4 r + i], + 4: zeros
    # (W4P: a 640-byte tile, entry 4 (n + 16 r) + i = scales, then bytes
    # 512 + 2 (n + 16 r) + j = zeros_packed[16 b + n][8 s + 2 r + j])
    G = K // 32
    sp = np.zeros((nrb * 16, nks * 16), np.uint16)
    sp[:N, :G] = np.asarray(scales).view(np.uint16)
    s5 = sp.reshape(nrb, 16, nks, 4, 4).transpose(0, 2, 3, 1, 4)            # b, s, r, n, i
    if fmt == 5:
        zp = np.zeros((nrb * 16, nks * 8), np.uint8)
        zp[:N, :zeros.shape[1]] = zeros
        z5 = zp.reshape(nrb, 16, nks, 4, 2).transpose(0, 2, 3, 1, 4)        # b, s, r, n, j
        meta = np.concatenate([s5.reshape(nrb, nks, -1).view(np.uint8),
                               z5.reshape(nrb, nks, -1)], axis=-1)         # 512 + 128 bytes
        out[meta_off:meta_off + nrb * nks * 640] = meta.reshape(-1)
    else:
        zz = np.zeros((nrb * 16, nks * 16), np.uint16)
        zz[:N, :G] = np.asarray(zeros).view(np.uint16)
        z5 = zz.reshape(nrb, 16, nks, 4, 4).transpose(0, 2, 3, 1, 4)
        meta = np.concatenate([s5, z5], axis=-1)
        out[meta_off:meta_off + nrb * nks * 1024] = meta.reshape(-1).view(np.uint8)
    # slab: chunk (b, c) entry 8 n + i = out_w[16 b + n][8 c + i]
    if n_out:
        p = np.zeros((nrb * 16, nch * 8), np.uint16)
        p[:N, :n_out] = np.asarray(wout).view(np.uint16)
        slab = p.reshape(nrb, 16, nch, 8).transpose(0, 2, 1, 3)                # b, c, n, i
        out[slab_off:slab_off + nrb * nch * 256] = slab.reshape(-1).view(np.uint8)
    return out


@pytest.mark.parametrize("fmt", [4, 2, 5])
@pytest.mark.parametrize("N,K,n_out", [(1, 32, 0), (1, 32, 1), (16, 512, 8), (37, 4224, 147),
                                       (33, 1056, 9), (48, 14336, 0), (5, 96, 96)])
def test_tile_host_matches_index_formulas(fmt, N, K, n_out):
    rng = np.random.default_rng(N * 7 + K + n_out)
    codes = rng.integers(0, 256, (N, K // (4 if fmt == 2 else 2)), dtype=np.uint8)
    sc = rng.integers(0, 65536, (N, K // 32), dtype=np.uint16)
    if fmt == 5:   # packed zero points: (K / 32 + 1) / 2 bytes per row
        ze = rng.integers(0, 256, (N, (K // 32 + 1) // 2), dtype=np.uint8)
    else:
        ze = rng.integers(0, 65536, (N, K // 32), dtype=np.uint16)
    wout = rng.integers(0, 65536, (N, n_out), dtype=np.uint16) if n_out else None
    got = B.wq_tile_host(fmt, codes, sc, ze, wout, N, K)
    exp = expected_tiled(fmt, codes, sc, ze, wout, N, K)
    assert got.shape == exp.shape
    assert np.array_equal(got, exp)
    assert B.wq_tiled_bytes(fmt, N, K, n_out) == exp.size


def test_tiled_sizes_and_errors():
    # W2 14336 x 4096 + 143 outliers: 14.68 MB of codes, 7.34 MB of scales and
    # zeros, 896 row blocks x 18 chunks x 256 bytes of slab
    assert B.wq_tiled_bytes(2, 14336, 4096, 143) == 896 * 8 * 2048 + 896 * 8 * 1024 + 896 * 18 * 256
    assert B.wq_tiled_bytes(4, 16, 512, 0) == 4096 + 1024
    assert B.wq_tiled_bytes(5, 16, 512, 0) == 4096 + 768   # 640-byte tile, padded to 256
    lib = B.load()
    assert lib.wq_tiled_bytes(3, 16, 512, 0) == B._lib.WQ_ERR_INVALID_ARG
    assert lib.wq_tiled_bytes(2, 16, 500, 0) == B._lib.WQ_ERR_UNSUPPORTED
    assert lib.wq_tiled_bytes(2, 16, 512, 513) == B._lib.WQ_ERR_INVALID_ARG
    buf = np.zeros(8192, np.uint8)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    # a buffer one byte short of the layout
    assert lib.wq_tile_host(4, p, p, p, None, 16, 512, 0, p, 4096 + 1023) == B._lib.WQ_ERR_INVALID_ARG
    assert b"needed" in lib.wq_last_error()
    assert lib.wq_tile_host(4, p, p, p, None, 16, 512, 1, p, 8192) == B._lib.WQ_ERR_INVALID_ARG
    # the device entry point rejects bad arguments before touching the GPU
    fake = ctypes.c_void_p(4096)
    assert lib.wq_gemv_tiled(3, fake, 16, 512, None, 0, fake, fake, None) == -1
    assert lib.wq_gemv_tiled(2, fake, 16, 512, None, 4, fake, fake, None) == -1
    assert lib.wq_gemv_tiled(2, ctypes.c_void_p(4100), 16, 512, None, 0, fake, fake, None) == -1
    assert lib.wq_gemv_tiled(2, fake, 16, 520, None, 0, fake, fake, None) == -2
