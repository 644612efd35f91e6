"""ctypes binding of ``libwq.so`` (include/wq.h).  Argument marshalling only:
every step of the computation runs in the library.

Host entry points take numpy arrays; device entry points take torch tensors
that live on the GPU (torch is used only for device memory and streams) and
enqueue on ``torch.cuda.current_stream()`` unless a stream is given.

Importing torch before loading the library matters: torch ships its own HIP
runtime under the same soname, and loading it first makes the library bind
to that one runtime instead of a second copy.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwq.so")

WQ_OK = 0
WQ_ERR_INVALID_ARG = -1
WQ_ERR_UNSUPPORTED = -2
WQ_ERR_HIP = -3
WQ_FMT_W4 = 4
WQ_FMT_W2 = 2
WQ_FMT_W4P = 5
WQ_FUSE_OUTLIERS = 1
WQ_GROUP = 32
WQ_MAX_K = 65536
WQ_GEMM_MAX_M = 16

# Every symbol include/wq.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_INT = ctypes.c_int
SIGNATURES = {
    "wq_status_str": (ctypes.c_char_p, [_INT]),
    "wq_last_error": (ctypes.c_char_p, []),
    "wq_version": (ctypes.c_char_p, []),
    "wq_quantize_w4": (_INT, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "wq_quantize_w2": (_INT, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "wq_pack_zeros_w4": (_INT, [_P, _I64, _I64, _P]),
    "wq_select_outliers": (_INT, [_P, _I64, _I64, _P, ctypes.c_double, _P, _I64, _P]),
    "wq_select_outliers_kurtosis": (_INT, [_P, _I64, _I64, _P, ctypes.c_double, _P, _I64, _P,
                                           _P, _P]),
    "wq_split_outliers": (_INT, [_P, _I64, _I64, _P, _I64, _P, _P]),
    "wq_dequant_host": (_INT, [_INT, _P, _P, _P, _I64, _I64, _P]),
    "wq_refinement_w4": (_INT, [_INT, _P, _P, _P, _P, _I64, _I64, _P, _I64, _P, _P, _P]),
    "wq_dequant_device": (_INT, [_INT, _P, _P, _P, _I64, _I64, _P, _P]),
    "wq_gemv_w4": (_INT, [_P, _P, _P, _I64, _I64, _P, _P, _I64, _U32, _P, _P, _P]),
    "wq_gemv_w2": (_INT, [_P, _P, _P, _I64, _I64, _P, _P, _I64, _U32, _P, _P, _P]),
    "wq_gemv_w4p": (_INT, [_P, _P, _P, _I64, _I64, _P, _P, _I64, _U32, _P, _P, _P]),
    "wq_gemm_wq": (_INT, [_INT, _P, _P, _P, _I64, _I64, _P, _P, _I64, _U32, _P, _I64, _P, _P]),
    "wq_outlier_add": (_INT, [_P, _P, _I64, _I64, _P, _I64, _I64, _P, _P]),
    "wq_embed_gather": (_INT, [_INT, _P, _P, _P, _I64, _I64, _P, _I64, _P, _P]),
    "wq_topk_count": (_I64, [_I64, _I64, _I64]),
    "wq_topk_chunks": (_INT, [_P, _I64, _I64, _I64, _P, _P]),
    "wq_refine_add": (_INT, [_P, _P, _P, _I64, _I64, _P, _I64, _P, _P, _P]),
    "wq_refine_topk": (_INT, [_P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P]),
    "wq_tiled_bytes": (_I64, [_INT, _I64, _I64, _I64]),
    "wq_tile_host": (_INT, [_INT, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64]),
    "wq_gemv_tiled": (_INT, [_INT, _P, _I64, _I64, _P, _I64, _P, _P, _P]),
    "wq_gemm_tiled": (_INT, [_INT, _P, _I64, _I64, _P, _I64, _P, _I64, _P, _P]),
    "wq_gemv_tiled_refine": (_INT, [_INT, _P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _I64, _I64,
                                    _P, _P]),
    "wq_gemv_v": (_INT, [_INT, _P, _P, _P, _I64, _I64, _P, _P, _I64, _U32, _P, _P, _P, _P]),
    "wq_gemm_wq_v": (_INT, [_INT, _P, _P, _P, _I64, _I64, _P, _P, _I64, _U32, _P, _I64, _P, _P,
                            _P]),
    "wq_gemm_tiled_v": (_INT, [_INT, _P, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _P]),
    "wq_refine_add_v": (_INT, [_P, _P, _P, _I64, _I64, _P, _I64, _P, _P, _P, _P]),
    "wq_refine_topk_v": (_INT, [_P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "wq_gemv_tiled_refine_v": (_INT, [_INT, _P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _I64,
                                      _I64, _P, _P, _P]),
    "wq_read_probe": (_INT, [_P, _I64, _P, _P]),
    "wq_read_probe_sink_words": (_I64, [_I64]),
    "wq_read_probe_geom": (_INT, [_P, _I64, _P, _INT, _INT, _INT, _P]),
    "wq_copy_probe": (_INT, [_P, _P, _I64, _P]),
}


# Fields of wq_variant (include/wq.h, "kernel-variant selection"), in order.
VARIANT_FIELDS = ("gemv_kernel", "gemv_rows_per_wave", "gemv_lds_x", "gemm_kernel", "gemm_rows",
                  "batch_slice_groups", "batch_row_transpose", "refine_groups", "refine_fuse",
                  "refine_wide", "batch_register_partials")


class Variant(ctypes.Structure):
    """wq_variant: an explicit kernel choice for one call (tests and
    measurements; not part of the method).  A field < 0 keeps the library's
    choice."""
    _fields_ = [(f, ctypes.c_int32) for f in VARIANT_FIELDS]


def variant(**fields) -> Variant:
    """A wq_variant with the given fields set and every other field -1."""
    v = Variant(*([-1] * len(VARIANT_FIELDS)))
    for k, val in fields.items():
        if k not in VARIANT_FIELDS:
            raise ValueError(f"unknown wq_variant field {k!r}")
        setattr(v, k, int(val))
    return v


def _vptr(v):
    return ctypes.addressof(v) if v is not None else None


class WQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{status}]")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Loads the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m bit_weight_only_gemv_amd.build` "
            "(there is no fallback implementation)")
    import torch  # noqa: F401  (see module docstring)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != WQ_OK:
        raise WQError(status, load().wq_last_error().decode())


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ------------------------------------------------------------------ host


def wq_quantize_w4(W: np.ndarray):
    """W float32 [N, K] -> (codes uint8 [N, K/2], scales fp16 [N, K/32], zeros fp16 [N, K/32])."""
    W = _c(W, np.float32)
    N, K = W.shape
    codes = np.empty((N, K // 2), np.uint8)
    sc = np.empty((N, K // WQ_GROUP), np.uint16)
    ze = np.empty((N, K // WQ_GROUP), np.uint16)
    _check(load().wq_quantize_w4(_np_ptr(W), N, K, WQ_GROUP, _np_ptr(codes), _np_ptr(sc), _np_ptr(ze)))
    return codes, sc.view(np.float16), ze.view(np.float16)


def wq_quantize_w2(W: np.ndarray):
    """W float32 [N, K] -> (codes uint8 [N, K/4], scales fp16 [N, K/32], zeros fp16 [N, K/32])."""
    W = _c(W, np.float32)
    N, K = W.shape
    codes = np.empty((N, K // 4), np.uint8)
    sc = np.empty((N, K // WQ_GROUP), np.uint16)
    ze = np.empty((N, K // WQ_GROUP), np.uint16)
    _check(load().wq_quantize_w2(_np_ptr(W), N, K, WQ_GROUP, _np_ptr(codes), _np_ptr(sc), _np_ptr(ze)))
    return codes, sc.view(np.float16), ze.view(np.float16)


def wq_pack_zeros_w4(zeros, N: int, K: int) -> np.ndarray:
    """FP16 W4 zero points [N, K/32] -> packed bytes uint8 [N, ceil(K/64)]."""
    ze = _c(np.asarray(zeros).view(np.uint16), np.uint16)
    out = np.empty((N, (K // WQ_GROUP + 1) // 2), np.uint8)
    _check(load().wq_pack_zeros_w4(_np_ptr(ze), N, K, _np_ptr(out)))
    return out


def wq_select_outliers(W: np.ndarray, profile: np.ndarray, ratio: float) -> np.ndarray:
    W = _c(W, np.float32)
    N, K = W.shape
    prof = _c(profile, np.float64)
    cap = max(1, int(np.floor(ratio * K)) + 1)
    idx = np.empty(cap, np.int32)
    n = ctypes.c_int64(0)
    _check(load().wq_select_outliers(_np_ptr(W), N, K, _np_ptr(prof), float(ratio), _np_ptr(idx),
                                     cap, ctypes.byref(n)))
    return idx[: n.value].copy()


def wq_select_outliers_kurtosis(W: np.ndarray, gamma: Optional[np.ndarray] = None,
                                r_base: float = 0.01):
    """Kurtosis-adaptive selection -> (idx int32 ascending, ratio r, kurtosis)."""
    W = _c(W, np.float32)
    N, K = W.shape
    g = _c(gamma, np.float64) if gamma is not None else None
    cap = max(1, int(np.floor(0.03 * K)) + 1)
    idx = np.empty(cap, np.int32)
    n = ctypes.c_int64(0)
    r = ctypes.c_double(0.0)
    k = ctypes.c_double(0.0)
    _check(load().wq_select_outliers_kurtosis(_np_ptr(W), N, K, _np_ptr(g) if g is not None else None,
                                              float(r_base), _np_ptr(idx), cap, ctypes.byref(n),
                                              ctypes.byref(r), ctypes.byref(k)))
    return idx[: n.value].copy(), r.value, k.value


def wq_split_outliers(W: np.ndarray, idx: np.ndarray):
    W = _c(W, np.float32)
    N, K = W.shape
    idx = _c(idx, np.int32)
    dense = np.empty_like(W)
    wout = np.empty((N, len(idx)), np.uint16)
    _check(load().wq_split_outliers(_np_ptr(W), N, K, _np_ptr(idx), len(idx), _np_ptr(dense),
                                    _np_ptr(wout)))
    return dense, wout.view(np.float16)


def _zeros_arg(fmt, zeros):
    """FP16 zero points (uint16 bits), or the packed bytes of W4P."""
    if fmt == WQ_FMT_W4P:
        return _c(zeros, np.uint8)
    return _c(np.asarray(zeros).view(np.uint16), np.uint16)


def wq_dequant_host(fmt: int, codes, scales, zeros, N: int, K: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    sc = _c(np.asarray(scales).view(np.uint16), np.uint16)
    ze = _zeros_arg(fmt, zeros)
    out = np.empty((N, K), np.uint16)
    _check(load().wq_dequant_host(fmt, _np_ptr(codes), _np_ptr(sc), _np_ptr(ze), N, K, _np_ptr(out)))
    return out.view(np.float16)


def wq_refinement_w4(fmt: int, W: np.ndarray, codes, scales, zeros, idx=None):
    """Refinement columns of a packed layer (W float32 [N, K] before the outlier
    split) -> (rcodes uint8 [K, N/2], rscales fp16 [K, N/32], rzeros fp16 [K, N/32])."""
    W = _c(W, np.float32)
    N, K = W.shape
    codes = _c(codes, np.uint8)
    sc = _c(np.asarray(scales).view(np.uint16), np.uint16)
    ze = _zeros_arg(fmt, zeros)
    idx = _c(idx if idx is not None else np.zeros(0, np.int32), np.int32)
    rc = np.empty((K, N // 2), np.uint8)
    rs = np.empty((K, N // WQ_GROUP), np.uint16)
    rz = np.empty((K, N // WQ_GROUP), np.uint16)
    _check(load().wq_refinement_w4(fmt, _np_ptr(W), _np_ptr(codes), _np_ptr(sc), _np_ptr(ze), N, K,
                                   _np_ptr(idx) if len(idx) else None, len(idx), _np_ptr(rc),
                                   _np_ptr(rs), _np_ptr(rz)))
    return rc, rs.view(np.float16), rz.view(np.float16)


def wq_tiled_bytes(fmt: int, N: int, K: int, n_out: int) -> int:
    n = int(load().wq_tiled_bytes(fmt, N, K, n_out))
    if n < 0:
        _check(n)
    return n


def wq_tile_host(fmt: int, codes, scales, zeros, out_w, N: int, K: int) -> np.ndarray:
    """Row-major packed arrays -> the tiled M = 1 layout (uint8 array)."""
    n_out = 0 if out_w is None else int(np.asarray(out_w).shape[1])
    codes = _c(codes, np.uint8)
    sc = _c(np.asarray(scales).view(np.uint16), np.uint16)
    ze = _zeros_arg(fmt, zeros)
    ow = _c(np.asarray(out_w).view(np.uint16), np.uint16) if n_out else None
    nb = wq_tiled_bytes(fmt, N, K, n_out)
    out = np.empty(nb, np.uint8)
    _check(load().wq_tile_host(fmt, _np_ptr(codes), _np_ptr(sc), _np_ptr(ze),
                               _np_ptr(ow) if n_out else None, N, K, n_out, _np_ptr(out), nb))
    return out


# ---------------------------------------------------------------- device


def _dptr(t) -> int:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("device arguments must be contiguous GPU tensors")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def wq_dequant_device(fmt, codes, scales, zeros, N, K, W_hat, stream=None):
    _check(load().wq_dequant_device(fmt, _dptr(codes), _dptr(scales), _dptr(zeros), N, K,
                                    _dptr(W_hat), _stream(stream)))


def _gemv(fmt, fn, codes, scales, zeros, N, K, x, y, out_idx, out_w, n_out, flags, stream,
          variant):
    args = (_dptr(codes), _dptr(scales), _dptr(zeros), N, K,
            _dptr(out_idx) if n_out else None, _dptr(out_w) if n_out else None, n_out, flags,
            _dptr(x), _dptr(y))
    if variant is None:
        _check(fn(*args, _stream(stream)))
    else:
        _check(load().wq_gemv_v(fmt, *args, _vptr(variant), _stream(stream)))


def wq_gemv_w4(codes, scales, zeros, N, K, x, y, out_idx=None, out_w=None, n_out=0,
               flags=WQ_FUSE_OUTLIERS, stream=None, variant=None):
    _gemv(WQ_FMT_W4, load().wq_gemv_w4, codes, scales, zeros, N, K, x, y, out_idx, out_w, n_out,
          flags, stream, variant)


def wq_gemv_w2(codes, scales, zeros, N, K, x, y, out_idx=None, out_w=None, n_out=0,
               flags=WQ_FUSE_OUTLIERS, stream=None, variant=None):
    _gemv(WQ_FMT_W2, load().wq_gemv_w2, codes, scales, zeros, N, K, x, y, out_idx, out_w, n_out,
          flags, stream, variant)


def wq_gemv_w4p(codes, scales, zeros_packed, N, K, x, y, out_idx=None, out_w=None, n_out=0,
                flags=WQ_FUSE_OUTLIERS, stream=None, variant=None):
    _gemv(WQ_FMT_W4P, load().wq_gemv_w4p, codes, scales, zeros_packed, N, K, x, y, out_idx, out_w,
          n_out, flags, stream, variant)


def wq_gemm_wq(fmt, codes, scales, zeros, N, K, X, M, Y, out_idx=None, out_w=None, n_out=0,
               flags=WQ_FUSE_OUTLIERS, stream=None, variant=None):
    args = (fmt, _dptr(codes), _dptr(scales), _dptr(zeros), N, K,
            _dptr(out_idx) if n_out else None, _dptr(out_w) if n_out else None,
            n_out, flags, _dptr(X), M, _dptr(Y))
    if variant is None:
        _check(load().wq_gemm_wq(*args, _stream(stream)))
    else:
        _check(load().wq_gemm_wq_v(*args, _vptr(variant), _stream(stream)))


def wq_gemm_tiled(fmt, tiled, N, K, X, M, Y, out_idx=None, n_out=0, stream=None, variant=None):
    args = (fmt, _dptr(tiled), N, K, _dptr(out_idx) if n_out else None, n_out, _dptr(X), M,
            _dptr(Y))
    if variant is None:
        _check(load().wq_gemm_tiled(*args, _stream(stream)))
    else:
        _check(load().wq_gemm_tiled_v(*args, _vptr(variant), _stream(stream)))


def wq_gemv_tiled(fmt, tiled, N, K, x, y, out_idx=None, n_out=0, stream=None):
    _check(load().wq_gemv_tiled(fmt, _dptr(tiled), N, K, _dptr(out_idx) if n_out else None, n_out,
                                _dptr(x), _dptr(y), _stream(stream)))


def wq_gemv_tiled_refine(fmt, tiled, N, K, x, y, rcodes, rscales, rzeros, chunk, k, out_idx=None,
                         n_out=0, sel_out=None, stream=None, variant=None):
    args = (fmt, _dptr(tiled), N, K, _dptr(out_idx) if n_out else None, n_out, _dptr(x), _dptr(y),
            _dptr(rcodes), _dptr(rscales), _dptr(rzeros), chunk, k,
            _dptr(sel_out) if sel_out is not None else None)
    if variant is None:
        _check(load().wq_gemv_tiled_refine(*args, _stream(stream)))
    else:
        _check(load().wq_gemv_tiled_refine_v(*args, _vptr(variant), _stream(stream)))


def wq_embed_gather(fmt, codes, scales, zeros, V, K, ids, n_ids, out, stream=None):
    _check(load().wq_embed_gather(fmt, _dptr(codes), _dptr(scales), _dptr(zeros), V, K,
                                  _dptr(ids) if n_ids else None, n_ids,
                                  _dptr(out) if n_ids else None, _stream(stream)))


def wq_topk_count(K: int, chunk: int, k: int) -> int:
    n = int(load().wq_topk_count(K, chunk, k))
    if n < 0:
        _check(n)
    return n


def wq_topk_chunks(x, K, chunk, k, sel, stream=None):
    _check(load().wq_topk_chunks(_dptr(x), K, chunk, k, _dptr(sel) if k else None,
                                 _stream(stream)))


def wq_refine_add(rcodes, rscales, rzeros, N, K, sel, n_sel, x, y, stream=None, variant=None):
    args = (_dptr(rcodes), _dptr(rscales), _dptr(rzeros), N, K, _dptr(sel) if n_sel else None,
            n_sel, _dptr(x), _dptr(y))
    if variant is None:
        _check(load().wq_refine_add(*args, _stream(stream)))
    else:
        _check(load().wq_refine_add_v(*args, _vptr(variant), _stream(stream)))


def wq_refine_topk(rcodes, rscales, rzeros, N, K, chunk, k, x, y, sel_out=None, stream=None,
                   variant=None):
    args = (_dptr(rcodes), _dptr(rscales), _dptr(rzeros), N, K, chunk, k, _dptr(x), _dptr(y),
            _dptr(sel_out) if sel_out is not None else None)
    if variant is None:
        _check(load().wq_refine_topk(*args, _stream(stream)))
    else:
        _check(load().wq_refine_topk_v(*args, _vptr(variant), _stream(stream)))


def wq_outlier_add(idx, out_w, n_out, N, X, M, K, Y, stream=None):
    _check(load().wq_outlier_add(_dptr(idx) if n_out else None, _dptr(out_w) if n_out else None,
                                 n_out, N, _dptr(X), M, K, _dptr(Y), _stream(stream)))


def wq_read_probe_sink_words(nbytes: int) -> int:
    return int(load().wq_read_probe_sink_words(nbytes))


def wq_read_probe(src, nbytes, sink, stream=None):
    _check(load().wq_read_probe(_dptr(src), nbytes, _dptr(sink), _stream(stream)))


def wq_read_probe_geom(src, nbytes, sink, blocks, threads, ring, stream=None):
    _check(load().wq_read_probe_geom(_dptr(src), nbytes, _dptr(sink), blocks, threads, ring,
                                     _stream(stream)))


def wq_copy_probe(src, dst, nbytes, stream=None):
    _check(load().wq_copy_probe(_dptr(src), _dptr(dst), nbytes, _stream(stream)))
