"""Packing a float32 weight matrix with the library's host encoder, and the
packed arrays' home on the GPU.

``pack_host`` is the offline path of the pages (OTF-LLM v4.0 quickstart:
profile -> outlier selection -> split -> per-group quantization -> packing),
entirely through ``libwq.so``'s host entry points.  ``DeviceLayer`` holds the
same arrays in device memory and calls the device entry points on them.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import _lib as L


@dataclasses.dataclass
class HostLayer:
    fmt: int
    N: int
    K: int
    codes: np.ndarray          # uint8 [N, K/2] (W4, W4P) or [N, K/4] (W2)
    scales: np.ndarray         # float16 [N, K/32]
    zeros: np.ndarray          # float16 [N, K/32]; W4P: packed uint8 [N, ceil(K/64)]
    idx: np.ndarray            # int32 [n_out], ascending
    wout: np.ndarray           # float16 [N, n_out]

    @property
    def n_out(self) -> int:
        return int(len(self.idx))


def pack_host(fmt: int, W: np.ndarray, profile: Optional[np.ndarray] = None,
              ratio: float = 0.0, *, kurtosis_gamma: Optional[np.ndarray] = None,
              kurtosis: bool = False) -> HostLayer:
    """Outlier selection, split, quantization and packing.  Outliers come from
    the profile-guided rule (profile, ratio), or with kurtosis=True from the
    kurtosis-adaptive rule (optional normalization gains kurtosis_gamma)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    if kurtosis:
        idx, _, _ = L.wq_select_outliers_kurtosis(W, kurtosis_gamma)
    elif profile is not None and ratio > 0:
        idx = L.wq_select_outliers(W, profile, ratio)
    else:
        idx = np.zeros(0, np.int32)
    if len(idx):
        dense, wout = L.wq_split_outliers(W, idx)
    else:
        dense, wout = W, np.zeros((N, 0), np.float16)
    if fmt in (L.WQ_FMT_W4, L.WQ_FMT_W4P):
        codes, sc, ze = L.wq_quantize_w4(dense)
        if fmt == L.WQ_FMT_W4P:
            ze = L.wq_pack_zeros_w4(ze, N, K)
    elif fmt == L.WQ_FMT_W2:
        codes, sc, ze = L.wq_quantize_w2(dense)
    else:
        raise ValueError("fmt must be 4, 5 (W4P) or 2")
    return HostLayer(fmt, N, K, codes, sc, ze, idx, wout)


@dataclasses.dataclass
class HostRefinement:
    """4-bit refinement columns of a layer, per input channel: the W4 format of
    the residual transposed ([K, N], groups of 32 output rows)."""
    N: int
    K: int
    codes: np.ndarray          # uint8 [K, N/2]
    scales: np.ndarray         # float16 [K, N/32]
    zeros: np.ndarray          # float16 [K, N/32]


def refinement_host(W: np.ndarray, host: "HostLayer") -> HostRefinement:
    """The refinement columns of the packed layer (StrataFlux section 3.2.1):
    the library's host encoder forms the residual of the resident layer, zeroes
    the outlier columns and W4-encodes it transposed (wq_refinement_w4)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    codes, sc, ze = L.wq_refinement_w4(host.fmt, W, host.codes, host.scales, host.zeros,
                                       host.idx if host.n_out else None)
    return HostRefinement(N, K, codes, sc, ze)


class DeviceLayer:
    """Packed arrays in device memory (torch tensors used as plain buffers).
    With ``tiled=True`` the layer also holds the tiled M = 1 layout (built by
    the library's host rearrangement), which ``gemv_tiled`` reads."""

    def __init__(self, host: HostLayer, device="cuda", tiled: bool = False):
        import torch
        self.fmt, self.N, self.K, self.n_out = host.fmt, host.N, host.K, host.n_out

        def up(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)

        self.codes = up(host.codes, np.uint8)
        self.scales = up(host.scales.view(np.int16), np.int16)
        if self.fmt == L.WQ_FMT_W4P:
            self.zeros = up(host.zeros, np.uint8)
        else:
            self.zeros = up(host.zeros.view(np.int16), np.int16)
        if self.n_out:
            self.idx = up(host.idx, np.int32)
            self.wout = up(host.wout.view(np.int16), np.int16)
        else:
            self.idx = self.wout = None
        self.tiled = None
        if tiled:
            t = L.wq_tile_host(self.fmt, host.codes, host.scales, host.zeros,
                               host.wout if self.n_out else None, self.N, self.K)
            self.tiled = up(t, np.uint8)

    def nbytes(self, M: int = 1) -> int:
        """Algorithmic bytes of one product: codes, scales, zeros, outlier slab
        and indices, X and Y."""
        b = self.codes.numel() + 2 * self.scales.numel() + self.zeros.numel() * self.zeros.element_size()
        b += 2 * self.N * self.n_out + 4 * self.n_out
        return b + 2 * M * self.K + 2 * M * self.N

    def gemv(self, x, y, flags=L.WQ_FUSE_OUTLIERS, stream=None, variant=None):
        fn = {L.WQ_FMT_W4: L.wq_gemv_w4, L.WQ_FMT_W2: L.wq_gemv_w2,
              L.WQ_FMT_W4P: L.wq_gemv_w4p}[self.fmt]
        fn(self.codes, self.scales, self.zeros, self.N, self.K, x, y, self.idx, self.wout,
           self.n_out, flags, stream, variant)

    def gemv_tiled(self, x, y, stream=None):
        if self.tiled is None:
            raise ValueError("layer built without tiled=True")
        L.wq_gemv_tiled(self.fmt, self.tiled, self.N, self.K, x, y, self.idx, self.n_out, stream)

    def gemm_tiled(self, X, Y, stream=None, variant=None):
        """Y [M][N] from X [M][K] on the tiled layout, M = 1 .. 16."""
        if self.tiled is None:
            raise ValueError("layer built without tiled=True")
        L.wq_gemm_tiled(self.fmt, self.tiled, self.N, self.K, X, X.shape[0], Y, self.idx,
                        self.n_out, stream, variant)

    def gemm(self, X, Y, flags=L.WQ_FUSE_OUTLIERS, stream=None, variant=None):
        L.wq_gemm_wq(self.fmt, self.codes, self.scales, self.zeros, self.N, self.K, X, X.shape[0],
                     Y, self.idx, self.wout, self.n_out, flags, stream, variant)

    def outlier_add(self, X, Y, stream=None):
        L.wq_outlier_add(self.idx, self.wout, self.n_out, self.N, X, X.shape[0], self.K, Y, stream)

    def embed(self, ids, out, stream=None):
        """Rows ids of the dequantized table into out (FP16 [len(ids), K])."""
        L.wq_embed_gather(self.fmt, self.codes, self.scales, self.zeros, self.N, self.K, ids,
                          ids.numel(), out, stream)

    def set_refinement(self, ref: HostRefinement, device="cuda"):
        import torch

        def up(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)

        self.r_codes = up(ref.codes, np.uint8)
        self.r_scales = up(ref.scales.view(np.int16), np.int16)
        self.r_zeros = up(ref.zeros.view(np.int16), np.int16)

    def refine(self, x, y, sel, n_sel, stream=None, variant=None):
        """y += sum over the selected channels of x_i C[:, i] (StrataFlux Eq. 2)."""
        L.wq_refine_add(self.r_codes, self.r_scales, self.r_zeros, self.N, self.K, sel, n_sel,
                        x, y, stream, variant)

    def refine_topk(self, x, y, k, chunk=1024, sel_out=None, stream=None, variant=None):
        """Selection and add of StrataFlux Eq. 2 in one launch."""
        L.wq_refine_topk(self.r_codes, self.r_scales, self.r_zeros, self.N, self.K, chunk, k, x, y,
                         sel_out, stream, variant)

    def gemv_tiled_refine(self, x, y, k, chunk=1024, sel_out=None, stream=None, variant=None):
        """The tiled product with the selection and add of StrataFlux Eq. 2 in
        the same launch (one FP16 rounding)."""
        if self.tiled is None:
            raise ValueError("layer built without tiled=True")
        L.wq_gemv_tiled_refine(self.fmt, self.tiled, self.N, self.K, x, y, self.r_codes,
                               self.r_scales, self.r_zeros, chunk, k, self.idx, self.n_out, sel_out,
                               stream, variant)

    def dequant(self, W_hat, stream=None):
        L.wq_dequant_device(self.fmt, self.codes, self.scales, self.zeros, self.N, self.K, W_hat,
                            stream)
