"""Plain CPU oracle for group-wise low-bit weight-only GEMV (numpy).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
library (``bit_weight_only_gemv_amd``) never imports, calls or links it, and
this module imports nothing from the product.

Every step is written out in the order the pages give it, vectorised only
across independent (row, group) pairs.  Sums over the 32 weights of a group,
and over the rows of a column, are taken left to right (``_seqsum``) rather
than with numpy's pairwise ``sum``, so that a C implementation that loops in
the natural order gets bit-identical results.

Sources (the three web pages this library is built from):

* [SPECTRA] "Compress Any LLM 3x in One Click, Near-Lossless in Under 50 MB
  RAM" (wpnews.pro).  Section 3.4 "Microscaled Group-32 Quantization with
  Marlin-Interleaved Layout" (the W4 formulas and the nibble interleave);
  Appendix A, Proposition 2 (error bound, and that codes use the scale before
  its rounding to 16 bits); section 4.1 "In-Register Fused W4A16 GEMV with
  Outlier Channel Accumulation" (the product, FP32 accumulation, FP16 store,
  outlier accumulation into the same accumulator); section 3.3 (int32
  outlier indices).
* [OTF] "On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)" (pypi otf-llm
  4.0.0).  Section 2 "The Lloyd-Max Non-Uniform Solution" (codebook),
  section 3 "Closed-Form Group Linear Regression" (S_g, Z_g), section 4
  "Profile-Guided Activation Outliers" (I_c score, top 3.5%), section 5
  "Bit-Packing Mechanics" (4 codes per byte, FP16 centroids, w = S*c + Z),
  "Architecture & Key Innovations" (FP16 outliers + INT2 background).

Readings taken where the pages are silent (each is tested):

* rounding is half-to-even everywhere (``np.rint`` / numpy casts);
* W4 arithmetic is float32 and the codes use the unrounded scale; the
  stored scale is its FP16 rounding and the zero point is stored as FP16;
* a constant group keeps the page's 1e-8 scale floor, which FP16 rounds to
  0, so its reconstruction is exactly 0;
* W2 code assignment: standardise each group by its mean and population
  standard deviation, then take the nearest FP16 centroid (ties go to the
  lower code; a zero-variance group gets code 1);
* the OLS epsilon is 1e-8; W2 scale and zero are stored as FP16;
* the outlier count is floor(ratio * K); ties in the score go to the lower
  column index; indices are stored ascending as int32;
* outlier columns are zeroed in the dense residual before quantization,
  and the quantized background skips them (x is masked at those columns);
* dequantized weights are rounded once to float32 and then to FP16.
"""

from __future__ import annotations

import numpy as np

GROUP = 32

# [OTF] section 2: the 4-level Lloyd-Max codebook, used at its FP16 values
# ([OTF] section 5 maps codes to an "FP16 Lloyd-Max Centroid").
CODEBOOK_DECIMAL = (-1.52, -0.45, 0.45, 1.52)
CODEBOOK_FP16 = np.array(CODEBOOK_DECIMAL, dtype=np.float16)
CODEBOOK_F64 = CODEBOOK_FP16.astype(np.float64)
# Decision thresholds of a nearest-centroid quantizer: midpoints of adjacent levels.
THRESHOLDS_F64 = (CODEBOOK_F64[:-1] + CODEBOOK_F64[1:]) / 2.0

W4_LEVELS = 15          # [SPECTRA] 3.4: s = (wmax - wmin) / 15, codes 0..15
W4_SCALE_FLOOR = np.float32(1e-8)
OLS_EPS = 1e-8


def _seqsum(a: np.ndarray, axis: int = -1) -> np.ndarray:
    """Left-to-right float sum along ``axis`` (no pairwise reordering)."""
    a = np.moveaxis(a, axis, 0)
    acc = np.zeros(a.shape[1:], dtype=a.dtype)
    for i in range(a.shape[0]):
        acc = acc + a[i]
    return acc


def _groups(W: np.ndarray) -> np.ndarray:
    N, K = W.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 32")
    return W.reshape(N, K // GROUP, GROUP)


# --------------------------------------------------------------------------- W4


def quantize_w4(W: np.ndarray):
    """Asymmetric 4-bit group-32 quantization ([SPECTRA] section 3.4).

    Per (row i, group g) of 32 consecutive input channels, in float32:
    wmin, wmax; ``s = max((wmax - wmin) / 15, 1e-8)``;
    ``z = clamp(round(-wmin / s), 0, 15)``; ``q = clamp(round(w / s + z), 0, 15)``
    (the code formula of [SPECTRA] Appendix A, Proposition 2 proof).

    Returns ``(q uint8 [N, K], scale fp16 [N, K/32], zero fp16 [N, K/32],
    s float32 [N, K/32])``; ``s`` is the unrounded scale the codes were made with.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    Wg = _groups(W)
    wmin = Wg.min(axis=2)
    wmax = Wg.max(axis=2)
    s = np.maximum((wmax - wmin) / np.float32(W4_LEVELS), W4_SCALE_FLOOR)
    z = np.clip(np.rint(-wmin / s), np.float32(0), np.float32(W4_LEVELS))
    t = Wg / s[..., None]
    t = t + z[..., None]
    q = np.clip(np.rint(t), np.float32(0), np.float32(W4_LEVELS)).astype(np.uint8)
    return q.reshape(W.shape), s.astype(np.float16), z.astype(np.float16), s


def pack_w4(q: np.ndarray) -> np.ndarray:
    """Nibble interleave of [SPECTRA] section 3.4: within each group, byte k
    (k = 0..15) holds code k in bits 3:0 and code k+16 in bits 7:4."""
    N, K = q.shape
    qg = q.reshape(N, K // GROUP, GROUP).astype(np.uint8)
    lo = qg[:, :, :16] & 0x0F
    hi = qg[:, :, 16:] & 0x0F
    return (lo | (hi << 4)).reshape(N, K // 2).astype(np.uint8)


def unpack_w4(codes: np.ndarray) -> np.ndarray:
    N, KB = codes.shape
    cg = codes.reshape(N, KB // 16, 16)
    lo = cg & 0x0F
    hi = cg >> 4
    return np.concatenate([lo, hi], axis=2).reshape(N, KB * 2).astype(np.uint8)


def dequant_w4(q: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """w_hat = (q - z) * s with the stored FP16 s and z ([SPECTRA] 4.1 kernel body):
    the float32 product is exact (small integer times an FP16 value), then it
    is rounded once to FP16."""
    N, K = q.shape
    qf = q.reshape(N, K // GROUP, GROUP).astype(np.float32)
    d = qf - zero.astype(np.float32)[..., None]
    w = d * scale.astype(np.float32)[..., None]
    return w.astype(np.float16).reshape(N, K)


def pack_zeros_w4(zero: np.ndarray) -> np.ndarray:
    """Packed zero points of [SPECTRA] section 3.4: the zero points of the two
    adjacent groups 2m and 2m + 1 of a row share byte m, group 2m in bits 3:0
    and group 2m + 1 in bits 7:4 (with an odd group count the last byte's high
    nibble is 0).  ``zero`` holds the FP16 zero points, which the W4 quantizer
    makes integers 0..15; anything else is rejected."""
    z = np.asarray(zero).astype(np.float32)
    if z.size and not (np.all(z == np.rint(z)) and z.min() >= 0 and z.max() <= W4_LEVELS):
        raise ValueError("zero points must be integers in 0..15")
    zi = z.astype(np.uint8)
    N, G = zi.shape
    if G % 2:
        zi = np.concatenate([zi, np.zeros((N, 1), np.uint8)], axis=1)
    return (zi[:, 0::2] | (zi[:, 1::2] << 4)).astype(np.uint8)


def unpack_zeros_w4(zpk: np.ndarray, G: int) -> np.ndarray:
    """Inverse of ``pack_zeros_w4``: FP16 zero points [N, G]."""
    zpk = np.asarray(zpk, dtype=np.uint8)
    N = zpk.shape[0]
    z = np.empty((N, 2 * zpk.shape[1]), np.uint8)
    z[:, 0::2] = zpk & 0x0F
    z[:, 1::2] = zpk >> 4
    return z[:, :G].astype(np.float16)


# --------------------------------------------------------------------------- W2


def quantize_w2(W: np.ndarray, return_unrounded: bool = False):
    """2-bit Lloyd-Max codes with a closed-form per-group OLS scale and zero
    ([OTF] sections 2 and 3), float64 throughout.

    Per group of 32: mean mu and population std sigma; standardised
    u = (w - mu) / sigma (0 if sigma = 0); code q = index of the nearest FP16
    centroid; c = C[q]; then
    ``S = sum((w - mean(w)) (c - mean(c))) / (sum((c - mean(c))^2) + eps)``,
    ``Z = mean(w) - S * mean(c)``.

    Returns ``(q uint8 [N, K], S fp16 [N, K/32], Z fp16 [N, K/32])`` and, if
    asked, the float64 ``S`` and ``Z`` before FP16 rounding.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    Wg = _groups(W).astype(np.float64)
    mu = _seqsum(Wg) / GROUP
    d = Wg - mu[..., None]
    sigma = np.sqrt(_seqsum(d * d) / GROUP)
    safe = np.where(sigma > 0, sigma, 1.0)
    u = np.where(sigma[..., None] > 0, d / safe[..., None], 0.0)
    q = ((u > THRESHOLDS_F64[0]).astype(np.uint8) + (u > THRESHOLDS_F64[1]).astype(np.uint8)
         + (u > THRESHOLDS_F64[2]).astype(np.uint8))
    c = CODEBOOK_F64[q]
    cbar = _seqsum(c) / GROUP
    dc = c - cbar[..., None]
    S = _seqsum(d * dc) / (_seqsum(dc * dc) + OLS_EPS)
    Z = mu - S * cbar
    out = (q.reshape(W.shape), S.astype(np.float16), Z.astype(np.float16))
    if return_unrounded:
        return out + (S, Z)
    return out


def pack_w2(q: np.ndarray) -> np.ndarray:
    """[OTF] section 5: byte = q0 | q1 << 2 | q2 << 4 | q3 << 6, four consecutive
    codes along K per byte."""
    N, K = q.shape
    qb = q.reshape(N, K // 4, 4).astype(np.uint8) & 0x03
    return (qb[..., 0] | (qb[..., 1] << 2) | (qb[..., 2] << 4) | (qb[..., 3] << 6)).astype(np.uint8)


def unpack_w2(codes: np.ndarray) -> np.ndarray:
    N, KB = codes.shape
    parts = [(codes >> (2 * j)) & 0x03 for j in range(4)]
    return np.stack(parts, axis=2).reshape(N, KB * 4).astype(np.uint8)


def dequant_w2(q: np.ndarray, S: np.ndarray, Z: np.ndarray) -> np.ndarray:
    """w_hat = S * C[q] + Z ([OTF] section 5, "W = scale * centroid + zero"),
    float32 (the product of two FP16 values is exact), then FP16."""
    N, K = q.shape
    c = CODEBOOK_FP16.astype(np.float32)[q.reshape(N, K // GROUP, GROUP)]
    w = S.astype(np.float32)[..., None] * c
    w = w + Z.astype(np.float32)[..., None]
    return w.astype(np.float16).reshape(N, K)


# --------------------------------------------------------------------- outliers


def outlier_count(K: int, ratio: float) -> int:
    """Number of FP16 outlier columns: floor(ratio * K) ([OTF] section 4, top 3.5%)."""
    return int(np.floor(ratio * K))


def outlier_scores(W: np.ndarray, profile: np.ndarray) -> np.ndarray:
    """I_c = ||W[:, c]||_2 * mean|X_c| ([OTF] section 4), float64, with the
    column norm summed over rows in order."""
    W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    acc = np.zeros(W64.shape[1], dtype=np.float64)
    for n in range(W64.shape[0]):
        acc = acc + W64[n] * W64[n]
    return np.sqrt(acc) * np.asarray(profile, dtype=np.float64)


def select_outliers(W: np.ndarray, profile: np.ndarray, ratio: float) -> np.ndarray:
    """The floor(ratio*K) columns of highest score; ties to the lower index;
    returned ascending as int32 ([SPECTRA] 3.3 stores indices as int32)."""
    K = W.shape[1]
    n = outlier_count(K, ratio)
    score = outlier_scores(W, profile)
    order = np.lexsort((np.arange(K), -score))
    return np.sort(order[:n]).astype(np.int32)


# ------------------------------------------ kurtosis-adaptive outlier policy

KURT_R_BASE = 0.01      # [SPECTRA] 3.3: r stays 0.01 for mesokurtic saliencies
KURT_R_MIN = 0.005      # [SPECTRA] 3.3: clamp(..., 0.005, 0.03)
KURT_R_MAX = 0.03
KURT_SLOPE = 0.15       # [SPECTRA] 3.3: r_base (1 + 0.15 ln(1 + kappa_excess))


def channel_saliency(W: np.ndarray, gamma=None) -> np.ndarray:
    """[SPECTRA] 3.1-3.2: S_j = |gamma_j| ||W[:, j]||_2 (float64, the column norm
    summed over rows in order).  Without a preceding normalization gain the page
    sets gamma_j = 1, the plain column norm."""
    K = W.shape[1]
    g = np.ones(K) if gamma is None else np.abs(np.asarray(gamma, dtype=np.float64))
    return outlier_scores(W, g)


def saliency_kurtosis(S: np.ndarray) -> float:
    """Population kurtosis of the saliencies ([SPECTRA] 3.3, Appendix A Prop. 1):
    mu = (1/K) sum S, sigma^2 = (1/K) sum (S - mu)^2, z = (S - mu) / sigma,
    kappa = (1/K) sum z^4, every sum left to right in float64.  A constant
    vector has no spread; its kappa is taken as 0 (reading)."""
    S = np.asarray(S, dtype=np.float64)
    K = S.size
    mu = float(_seqsum(S)) / K
    d = S - mu
    var = float(_seqsum(d * d)) / K
    if var == 0.0:
        return 0.0
    z = d / np.sqrt(var)
    z2 = z * z
    return float(_seqsum(z2 * z2)) / K


def kurtosis_ratio(kappa: float, r_base: float = KURT_R_BASE) -> float:
    """[SPECTRA] 3.3: r = clamp(r_base (1 + 0.15 ln(1 + max(0, kappa - 3))), 0.005, 0.03)."""
    ex = max(0.0, kappa - 3.0)
    r = r_base * (1.0 + KURT_SLOPE * float(np.log1p(ex)))
    return min(max(r, KURT_R_MIN), KURT_R_MAX)


def select_outliers_kurtosis(W: np.ndarray, gamma=None, r_base: float = KURT_R_BASE):
    """The kurtosis-adaptive outlier policy of [SPECTRA] 3.1-3.3: saliencies,
    their kurtosis, the ratio r, then the floor(r K) most salient columns (ties
    to the lower index), ascending int32.  Returns (idx, r, kappa)."""
    K = W.shape[1]
    S = channel_saliency(W, gamma)
    kappa = saliency_kurtosis(S)
    r = kurtosis_ratio(kappa, r_base)
    n = outlier_count(K, r)
    order = np.lexsort((np.arange(K), -S))
    return np.sort(order[:n]).astype(np.int32), r, kappa


def split_outliers(W: np.ndarray, idx: np.ndarray):
    """Dense residual with the outlier columns zeroed, and the outlier columns
    kept in FP16 as a row-major [N, n_out] slab ([SPECTRA] 3.4 first sentence,
    3.6 payload; [OTF] "Architecture": FP16 outliers + quantized background)."""
    W = np.asarray(W, dtype=np.float32)
    dense = W.copy()
    dense[:, idx] = 0.0
    wout = W[:, idx].astype(np.float16)
    return dense, np.ascontiguousarray(wout)


# ------------------------------------------------------------ the whole layer


class QuantLayer:
    """Everything the GEMV consumes for one layer, built by the oracle."""

    def __init__(self, fmt, codes, scale, zero, q, idx, wout, N, K):
        self.fmt, self.codes, self.scale, self.zero = fmt, codes, scale, zero
        self.q, self.idx, self.wout, self.N, self.K = q, idx, wout, N, K

    @property
    def n_out(self) -> int:
        return int(len(self.idx))

    @property
    def zero_packed(self) -> np.ndarray:
        """W4 zero points packed two per byte ([SPECTRA] section 3.4)."""
        return pack_zeros_w4(self.zero)

    def w_hat(self) -> np.ndarray:
        if self.fmt in (4, 5):
            return dequant_w4(self.q, self.scale, self.zero)
        return dequant_w2(self.q, self.scale, self.zero)


def quantize_layer(fmt: int, W: np.ndarray, profile=None, ratio: float = 0.0,
                   idx=None) -> QuantLayer:
    """Outlier split (columns ``idx`` if given, else from the profile rule)
    followed by W4 or W2 quantization of the dense residual and packing."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    if idx is not None and len(idx) > 0:
        idx = np.asarray(idx, dtype=np.int32)
        dense, wout = split_outliers(W, idx)
    elif profile is not None and outlier_count(K, ratio) > 0:
        idx = select_outliers(W, profile, ratio)
        dense, wout = split_outliers(W, idx)
    else:
        idx = np.zeros(0, np.int32)
        dense, wout = W, np.zeros((N, 0), np.float16)
    if fmt in (4, 5):   # 5: W4 whose zero points are stored packed (same values)
        q, sc, ze, _ = quantize_w4(dense)
        codes = pack_w4(q)
    elif fmt == 2:
        q, sc, ze = quantize_w2(dense)
        codes = pack_w2(q)
    else:
        raise ValueError("fmt must be 4, 5 or 2")
    return QuantLayer(fmt, codes, sc, ze, q, idx, wout, N, K)


# ------------------------------------------------------------ the product


def background_mask(K: int, idx: np.ndarray) -> np.ndarray:
    m = np.ones(K, dtype=bool)
    m[np.asarray(idx, dtype=np.int64)] = False
    return m


def matvec_ref(w_hat: np.ndarray, x: np.ndarray, idx=None, wout=None):
    """Float64 reference of the fused product ([SPECTRA] 4.1 and 4.2; [OTF]
    "continuous GEMM addition"):

    ``y[m, n] = sum_{k not in outliers} w_hat[n, k] x[m, k]
               + sum_j wout[n, j] x[m, idx[j]]``

    Returns ``(y float64 [M, N], abs_sum float64 [M, N])`` where ``abs_sum`` is
    the same sum over |term|, the scale of the acceptance bound.
    """
    x = np.atleast_2d(np.asarray(x))
    W64 = np.asarray(w_hat, dtype=np.float16).astype(np.float64)
    X64 = x.astype(np.float16).astype(np.float64)
    K = W64.shape[1]
    if idx is not None and len(idx):
        Xb = X64 * background_mask(K, idx)[None, :]
        Xo = X64[:, np.asarray(idx, dtype=np.int64)]
        O64 = np.asarray(wout, dtype=np.float16).astype(np.float64)
        y = Xb @ W64.T + Xo @ O64.T
        a = np.abs(Xb) @ np.abs(W64).T + np.abs(Xo) @ np.abs(O64).T
    else:
        y = X64 @ W64.T
        a = np.abs(X64) @ np.abs(W64).T
    return y, a


# ------------------------------------------------ runtime top-k refinement

REFINE_CHUNK = 1024     # [StrataFlux] 3.2.1: input channels in chunks of 1,024


def topk_chunks(x: np.ndarray, k: int, chunk: int = REFINE_CHUNK) -> np.ndarray:
    """S(x) of [StrataFlux] 3.2.1 "Channel selection": the input channels cut
    into chunks of ``chunk``, and in each chunk the k channels of largest |x_i|
    (all of a chunk shorter than k).  Readings: |x| of the FP16 value, ties go to
    the lower index, each chunk's picks are listed in ascending order, chunks in
    order."""
    x = np.asarray(x, dtype=np.float16).reshape(-1)
    K = x.size
    mag = np.abs(x.astype(np.float64))
    out = []
    for c0 in range(0, K, chunk):
        m = mag[c0:c0 + chunk]
        order = np.lexsort((np.arange(m.size), -m))
        out.append(np.sort(order[:min(k, m.size)]) + c0)
    return np.concatenate(out).astype(np.int32) if out else np.zeros(0, np.int32)


def refinement_w4(W: np.ndarray, w_hat: np.ndarray, idx=None):
    """Refinement columns: the residual R = W - w_hat of the resident layer,
    stored per input channel (R transposed, [K, N]) in the W4 format along N
    ([StrataFlux] 3.2.1: refinement values as integers with their own scale
    factors; DecDEC's 4-bit encoding of the weight residual).  Outlier columns
    ``idx`` are exact already: their residual is 0 (reading).  Returns the W4
    quantization of R^T: (q, scale, zero) with groups of 32 output rows."""
    R = np.asarray(W, dtype=np.float32) - np.asarray(w_hat, dtype=np.float16).astype(np.float32)
    if idx is not None and len(idx):
        R[:, np.asarray(idx, dtype=np.int64)] = 0.0
    q, sc, ze, _ = quantize_w4(np.ascontiguousarray(R.T))
    return q, sc, ze


def refine_ref(y0: np.ndarray, x: np.ndarray, sel: np.ndarray, c_hat: np.ndarray):
    """[StrataFlux] Eq. 2: y' = y0 + sum_{i in S(x)} x_i C[:, i] in float64, with
    C^T = ``c_hat`` [K, N] the dequantized refinement.  Returns (y', abs_sum)
    with abs_sum = |y0| + sum |x_i C[:, i]| (the scale of the acceptance bound)."""
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64).reshape(-1)
    C = np.asarray(c_hat, dtype=np.float16).astype(np.float64)
    y0 = np.asarray(y0, dtype=np.float16).astype(np.float64)
    sel = np.asarray(sel, dtype=np.int64)
    terms = x64[sel][:, None] * C[sel]
    return y0 + terms.sum(axis=0), np.abs(y0) + np.abs(terms).sum(axis=0)


# Acceptance bound per output element: |y_gpu - y_ref| <= REL * sum|w x| + ABS.
TOL_REL = 2e-3
TOL_ABS = 1e-5


def check_tolerance(y_test: np.ndarray, y_ref: np.ndarray, abs_sum: np.ndarray):
    """Returns ``(ok, worst)`` where ``worst`` is max |err| / bound over all
    elements (<= 1 passes)."""
    y_test = np.asarray(y_test, dtype=np.float64).reshape(y_ref.shape)
    bound = TOL_REL * abs_sum + TOL_ABS
    err = np.abs(y_test - y_ref)
    ratio = err / bound
    worst = float(np.max(ratio)) if ratio.size else 0.0
    ok = bool(np.all(np.isfinite(y_test)) and worst <= 1.0)
    return ok, worst


# ------------------------------------------------------------ fidelity metrics


def fidelity(W: np.ndarray, W_hat: np.ndarray):
    """Relative Frobenius error, SNR (dB) and cosine similarity ([SPECTRA]
    section 2.5 criteria; section 2.3 reports them for a Gaussian matrix)."""
    a = np.asarray(W, dtype=np.float64).ravel()
    b = np.asarray(W_hat, dtype=np.float64).ravel()
    e = a - b
    ea, ee, eb = float(a @ a), float(e @ e), float(b @ b)
    rel = np.sqrt(ee / ea)
    snr = 10.0 * np.log10(ea / ee)
    cos = float(a @ b) / np.sqrt(ea * eb)
    return rel, snr, cos
