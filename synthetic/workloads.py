"""Seeded synthetic layers for the five workloads and for small parity cases.

Nothing here quantizes, packs, selects outliers or multiplies: it returns
float32 weights, FP16 activations, spike sets and float64 activation
profiles.  Shapes follow the models the pages name (Llama-3-8B projection
shapes, a 70B-class MLP), distributions follow the recipe below.

Recipe (all seeds via :func:`rng_for`):

* weights ``W = sigma * standard_normal(float32)``;
* activations ``x = standard_normal(float32)``, optional spike channels
  multiplied in float32, then rounded to FP16 (round-to-nearest-even);
* the W2 layer of the 14336x4096 workload adds a per-(row, group-of-32)
  mean shift ``mu ~ 0.005 * N(0, 1)`` broadcast over each group;
* activation profiles (the "mean |X_c|" a calibration pass would record,
  OTF-LLM v4.0 page, section 4) are either the mean of 128 seeded draws of the
  runtime activation distribution, or ``|N(0, 1)|`` with spiked channels.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

ROLE_W, ROLE_X, ROLE_SHIFT, ROLE_SPIKES, ROLE_PROFILE = 0, 1, 2, 3, 4

# Fraction of input channels kept exact in FP16 (OTF-LLM v4.0 page: "Top-3.5%").
OUTLIER_RATIO = 0.035

# (name, N rows = output features, K = input features) of one Llama-3-8B decoder
# layer, in the order a decode step visits them.
LLAMA3_8B_SWEEP = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
)
LLAMA3_8B_LAYERS = 32
LLAMA3_8B_LM_HEAD = ("lm_head", 128256, 4096)


def rng_for(cfg: int, layer: int, proj: int, role: int) -> np.random.Generator:
    """Generator for one array of one workload."""
    return np.random.default_rng(np.random.SeedSequence([2026, cfg, layer, proj, role]))


def gaussian_weights(N: int, K: int, sigma: float, cfg: int, layer: int = 0,
                     proj: int = 0) -> np.ndarray:
    g = rng_for(cfg, layer, proj, ROLE_W)
    W = g.standard_normal((N, K), dtype=np.float32)
    W *= np.float32(sigma)
    return W


def gaussian_x_fp16(M: int, K: int, cfg: int, layer: int = 0, proj: int = 0,
                    spikes: Optional[np.ndarray] = None, spike_mult: float = 1.0) -> np.ndarray:
    g = rng_for(cfg, layer, proj, ROLE_X)
    x = g.standard_normal((M, K), dtype=np.float32)
    if spikes is not None and len(spikes):
        x[:, spikes] *= np.float32(spike_mult)
    return x.astype(np.float16)


def spike_set(K: int, count: int, cfg: int, layer: int = 0, proj: int = 0) -> np.ndarray:
    """``count`` distinct channels out of ``K``, ascending."""
    g = rng_for(cfg, layer, proj, ROLE_SPIKES)
    return np.sort(g.choice(K, size=count, replace=False)).astype(np.int64)


@dataclasses.dataclass
class Layer:
    """One synthetic linear layer plus its activations.

    ``W`` float32 [N, K]; ``x`` float16 [M, K]; ``profile`` float64 [K] or None
    (None means no outlier channels); ``ratio`` the outlier fraction; ``fmt`` 4
    or 2 (bits per weight code); ``spikes`` the spiked channels (may be empty).
    """

    name: str
    fmt: int
    W: np.ndarray
    x: np.ndarray
    profile: Optional[np.ndarray]
    ratio: float
    spikes: np.ndarray

    @property
    def N(self) -> int:
        return self.W.shape[0]

    @property
    def K(self) -> int:
        return self.W.shape[1]

    @property
    def M(self) -> int:
        return self.x.shape[0]


def _profile_from_draws(K: int, spikes: np.ndarray, mult: float, cfg: int, layer: int,
                        proj: int, draws: int = 128) -> np.ndarray:
    g = rng_for(cfg, layer, proj, ROLE_PROFILE)
    acc = np.zeros(K, dtype=np.float64)
    for _ in range(draws):
        d = g.standard_normal(K, dtype=np.float32)
        d[spikes] *= np.float32(mult)
        acc += np.abs(d.astype(np.float16).astype(np.float64))
    return acc / draws


def small_layer(fmt: int, N: int, K: int, M: int = 1, *, with_outliers: bool = False,
                seed: int = 0, sigma: float = 0.02, spike_frac: float = 0.01,
                spike_mult: float = 100.0, ratio: float = OUTLIER_RATIO) -> Layer:
    """A small layer of the same recipe, for parity tests the oracle finishes quickly."""
    cfg = 100 + seed
    W = gaussian_weights(N, K, sigma, cfg, 0, fmt)
    n_sp = max(1, int(spike_frac * K)) if with_outliers else 0
    sp = spike_set(K, n_sp, cfg, 0, fmt) if n_sp else np.zeros(0, np.int64)
    x = gaussian_x_fp16(M, K, cfg, 0, fmt, sp, spike_mult)
    prof = _profile_from_draws(K, sp, spike_mult, cfg, 0, fmt, draws=16) if with_outliers else None
    return Layer(f"small_w{fmt}_{N}x{K}_m{M}", fmt, W, x, prof, ratio if with_outliers else 0.0, sp)


def config1() -> Layer:
    """W4, 4096x4096, N(0, 0.02^2) weights, x ~ N(0, 1), no outliers, M = 1."""
    W = gaussian_weights(4096, 4096, 0.02, 1)
    x = gaussian_x_fp16(1, 4096, 1)
    return Layer("w4_4096x4096_m1", 4, W, x, None, 0.0, np.zeros(0, np.int64))


def config2() -> Layer:
    """W2, 14336x4096 (Llama-3-8B gate/up shape), M = 1.

    W = 0.02 N(0,1) + a per-(row, group) shift 0.005 N(0,1); 1% of input
    channels spiked x100 in x; the profile is the mean |x| over 128 draws of the
    same distribution; 3.5% outlier columns.
    """
    N, K = 14336, 4096
    W = gaussian_weights(N, K, 0.02, 2)
    mu = rng_for(2, 0, 0, ROLE_SHIFT).standard_normal((N, K // 32), dtype=np.float32)
    mu *= np.float32(0.005)
    W += np.repeat(mu, 32, axis=1)
    sp = spike_set(K, int(0.01 * K), 2)
    x = gaussian_x_fp16(1, K, 2, spikes=sp, spike_mult=100.0)
    prof = _profile_from_draws(K, sp, 100.0, 2, 0, 0)
    return Layer("w2_14336x4096_m1", 2, W, x, prof, OUTLIER_RATIO, sp)


def config3_shapes():
    """(layer, proj, name, N, K) for the 225 GEMVs of one Llama-3-8B-shaped decode step."""
    out = []
    for layer in range(LLAMA3_8B_LAYERS):
        for p, (name, N, K) in enumerate(LLAMA3_8B_SWEEP):
            out.append((layer, p, name, N, K))
    name, N, K = LLAMA3_8B_LM_HEAD
    out.append((LLAMA3_8B_LAYERS, 0, name, N, K))
    return out


def config3_layer(layer: int, proj: int, N: int, K: int, name: str = "") -> Layer:
    """One W4 GEMV of the sweep: N(0, 0.02^2) weights, its own x ~ N(0, 1)."""
    W = gaussian_weights(N, K, 0.02, 3, layer, proj)
    x = gaussian_x_fp16(1, K, 3, layer, proj)
    return Layer(f"w4_sweep_l{layer}_{name}", 4, W, x, None, 0.0, np.zeros(0, np.int64))


def config4(M: int, N: int, K: int) -> Layer:
    """W4 batched small-M: X [M, K] ~ N(0, 1), W N(0, 0.02^2), no outliers."""
    W = gaussian_weights(N, K, 0.02, 4, 0, N)
    x = gaussian_x_fp16(M, K, 4, M, N)
    return Layer(f"w4_{N}x{K}_m{M}", 4, W, x, None, 0.0, np.zeros(0, np.int64))


def config5(N: int, K: int, M: int) -> Layer:
    """70B-class W2 + outliers: W N(0, 0.015^2); profile |N(0,1)| with 0.5% of
    channels x300; runtime X ~ N(0, 1) with the same channels x300."""
    W = gaussian_weights(N, K, 0.015, 5, 0, N)
    sp = spike_set(K, int(0.005 * K), 5, 0, N)
    prof = np.abs(rng_for(5, 0, N, ROLE_PROFILE).standard_normal(K))
    prof[sp] *= 300.0
    x = gaussian_x_fp16(M, K, 5, M, N, spikes=sp, spike_mult=300.0)
    return Layer(f"w2_{N}x{K}_m{M}", 2, W, x, prof, OUTLIER_RATIO, sp)
