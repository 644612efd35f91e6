// Host (CPU) half of the library: status/error reporting, the reference
// encoders of the W4 and W2 formats, outlier selection and split, and host
// dequantization.
//
// Build with -ffp-contract=off and without fast-math: every float operation
// here is one IEEE operation in the order written, with round-to-nearest-even,
// so the results are bit-identical to any other implementation that performs
// the same operations in the same order.
//
// Sources: the SPECTRA page ("Compress Any LLM 3x in One Click, Near-Lossless
// in Under 50 MB RAM"), section 3.4 and Appendix A Proposition 2 (W4 grid,
// nibble interleave); the OTF-LLM v4.0 page (pypi otf-llm 4.0.0), sections
// 2-5 (Lloyd-Max codebook, OLS scale/zero, profile-guided outliers, 2-bit
// packing).

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "wq_internal.h"

namespace {

thread_local std::string g_last_error;

// ------------------------------------------------------------------ FP16 bits

// Round to nearest integer, ties to even, for doubles of magnitude below 2^52
// (adding and subtracting 2^52 leaves the rounded value in the default rounding
// mode); larger doubles are already integers.  Avoids nearbyint, whose
// floating-point-environment handling is slow in some C libraries.
inline double round_half_even_d(double v) {
  const double big = 4503599627370496.0;   // 2^52
  const double a = std::fabs(v);
  if (!(a < big)) return v;
  return std::copysign((a + big) - big, v);
}

// IEEE binary16 from binary64, round to nearest, ties to even.  Written from
// the format's definition: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
// bits; subnormals are multiples of 2^-24.
uint16_t f64_to_f16(double v) {
  uint64_t b;
  std::memcpy(&b, &v, 8);
  const uint16_t sign = (uint16_t)((b >> 63) << 15);
  if (std::isnan(v)) return (uint16_t)(sign | 0x7E00u);
  const double a = std::fabs(v);
  // 65520 is half-way between the largest finite FP16 (65504) and 2^16: it and
  // everything above round to infinity.
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  if (a < 0x1p-14) {
    // subnormal (or zero): count of 2^-24 units, rounded to nearest even.  A
    // result of 1024 is the smallest normal, whose bit pattern is the same.
    const double m = round_half_even_d(std::ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)m);
  }
  int e2;
  (void)std::frexp(a, &e2);        // a = f * 2^e2, f in [0.5, 1)
  int e = e2 - 1;                  // a in [2^e, 2^(e+1))
  double m = round_half_even_d(std::ldexp(a, 10 - e));   // in [1024, 2048]
  if (m == 2048.0) {
    m = 1024.0;
    e += 1;
  }
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

uint16_t f32_to_f16(float v) { return f64_to_f16((double)v); }   // float -> double is exact

float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15);
  const uint32_t e = (h >> 10) & 0x1Fu;
  const uint32_t f = h & 0x3FFu;
  double v;
  if (e == 0)
    v = std::ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = std::ldexp((double)(f | 0x400u), (int)e - 25);
  return (float)(sign ? -v : v);
}

// Round to nearest integer, ties to even, in the default rounding mode:
// adding and subtracting 2^23 leaves an integer for |v| < 2^23, and every
// float of larger magnitude is already an integer.  The sign is kept, so
// values in (-0.5, 0) give -0 like any IEEE roundToIntegralTiesToEven.
inline float round_half_even(float v) {
  const float big = 8388608.0f;   // 2^23
  const float a = std::fabs(v);
  if (!(a < big)) return v;
  return std::copysign((a + big) - big, v);
}

// The OTF-LLM codebook {-1.52, -0.45, +0.45, +1.52} at its FP16 values.
const uint16_t kCodebookF16[4] = {0xBE14u, 0xB733u, 0x3733u, 0x3E14u};

}  // namespace

namespace wq {

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return WQ_OK;
}

int check_shape(int64_t N, int64_t K, const char* who) {
  if (N < 1) return fail(WQ_ERR_INVALID_ARG, "%s: N must be >= 1 (got %lld)", who, (long long)N);
  if (K < WQ_GROUP || K % WQ_GROUP)
    return fail(WQ_ERR_UNSUPPORTED, "%s: K must be a positive multiple of 32 (got %lld)", who,
                (long long)K);
  if (K > WQ_MAX_K)
    return fail(WQ_ERR_UNSUPPORTED, "%s: K above %d is not supported (got %lld)", who, WQ_MAX_K,
                (long long)K);
  if (N > (int64_t)1 << 31)
    return fail(WQ_ERR_UNSUPPORTED, "%s: N above 2^31 is not supported", who);
  return WQ_OK;
}

int check_outlier_args(const int32_t* idx, const uint16_t* out_w, int64_t n_out, int64_t K,
                       const char* who) {
  if (n_out < 0 || n_out > K)
    return fail(WQ_ERR_INVALID_ARG, "%s: n_out must be in [0, K] (got %lld)", who,
                (long long)n_out);
  if (n_out > 0 && (!idx || !out_w))
    return fail(WQ_ERR_INVALID_ARG, "%s: out_idx and out_w must be non-NULL when n_out > 0", who);
  return WQ_OK;
}

}  // namespace wq

using wq::fail;

extern "C" {

const char* wq_status_str(int status) {
  switch (status) {
    case WQ_OK: return "ok";
    case WQ_ERR_INVALID_ARG: return "invalid argument";
    case WQ_ERR_UNSUPPORTED: return "unsupported";
    case WQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* wq_last_error(void) { return g_last_error.c_str(); }

const char* wq_version(void) { return "wq 0.1 gfx950"; }

}  // extern "C"

namespace {

// One W4 group of 32 float32 weights (SPECTRA section 3.4, Appendix A): the 16
// code bytes (in-group nibble interleave), the FP16 scale and the FP16 zero.
void quantize_w4_group(const float* w, uint8_t* c, uint16_t* scale, uint16_t* zero) {
  float wmin = w[0], wmax = w[0];
  for (int k = 1; k < WQ_GROUP; ++k) {
    wmin = std::min(wmin, w[k]);
    wmax = std::max(wmax, w[k]);
  }
  float s = (wmax - wmin) / 15.0f;
  if (!(s > 1e-8f)) s = 1e-8f;
  float z = round_half_even(-wmin / s);
  z = std::min(std::max(z, 0.0f), 15.0f);
  uint8_t q[WQ_GROUP];
  for (int k = 0; k < WQ_GROUP; ++k) {
    float t = w[k] / s;
    t = t + z;
    t = round_half_even(t);
    t = std::min(std::max(t, 0.0f), 15.0f);
    q[k] = (uint8_t)t;
  }
  for (int k = 0; k < 16; ++k) c[k] = (uint8_t)((q[k] & 0x0F) | ((q[k + 16] & 0x0F) << 4));
  *scale = f32_to_f16(s);
  *zero = f32_to_f16(z);
}

}  // namespace

extern "C" {

int wq_quantize_w4(const float* W, int64_t N, int64_t K, int32_t group, uint8_t* codes,
                   uint16_t* scales, uint16_t* zeros) {
  if (group != WQ_GROUP) return fail(WQ_ERR_UNSUPPORTED, "wq_quantize_w4: group must be 32");
  if (int r = wq::check_shape(N, K, "wq_quantize_w4")) return r;
  if (!W || !codes || !scales || !zeros)
    return fail(WQ_ERR_INVALID_ARG, "wq_quantize_w4: NULL pointer");
  const int64_t G = K / WQ_GROUP;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < G; ++g)
      quantize_w4_group(W + n * K + g * WQ_GROUP, codes + n * (K / 2) + g * 16,
                        scales + n * G + g, zeros + n * G + g);
  return wq::ok();
}

int wq_quantize_w2(const float* W, int64_t N, int64_t K, int32_t group, uint8_t* codes,
                   uint16_t* scales, uint16_t* zeros) {
  if (group != WQ_GROUP) return fail(WQ_ERR_UNSUPPORTED, "wq_quantize_w2: group must be 32");
  if (int r = wq::check_shape(N, K, "wq_quantize_w2")) return r;
  if (!W || !codes || !scales || !zeros)
    return fail(WQ_ERR_INVALID_ARG, "wq_quantize_w2: NULL pointer");
  double C[4], T[3];
  for (int i = 0; i < 4; ++i) C[i] = (double)f16_to_f32(kCodebookF16[i]);
  for (int i = 0; i < 3; ++i) T[i] = (C[i] + C[i + 1]) / 2.0;   // nearest-centroid thresholds
  const int64_t G = K / WQ_GROUP;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < G; ++g) {
      const float* wf = W + n * K + g * WQ_GROUP;
      double w[WQ_GROUP], d[WQ_GROUP], c[WQ_GROUP], dc[WQ_GROUP];
      uint8_t q[WQ_GROUP];
      double mu = 0.0;
      for (int k = 0; k < WQ_GROUP; ++k) {
        w[k] = (double)wf[k];
        mu = mu + w[k];
      }
      mu = mu / 32.0;
      double ss = 0.0;
      for (int k = 0; k < WQ_GROUP; ++k) {
        d[k] = w[k] - mu;
        ss = ss + d[k] * d[k];
      }
      const double sigma = std::sqrt(ss / 32.0);
      double cs = 0.0;
      for (int k = 0; k < WQ_GROUP; ++k) {
        const double u = sigma > 0.0 ? d[k] / sigma : 0.0;
        q[k] = (uint8_t)((u > T[0]) + (u > T[1]) + (u > T[2]));
        c[k] = C[q[k]];
        cs = cs + c[k];
      }
      const double cbar = cs / 32.0;
      double num = 0.0, den = 0.0;
      for (int k = 0; k < WQ_GROUP; ++k) dc[k] = c[k] - cbar;
      for (int k = 0; k < WQ_GROUP; ++k) num = num + d[k] * dc[k];
      for (int k = 0; k < WQ_GROUP; ++k) den = den + dc[k] * dc[k];
      den = den + 1e-8;
      const double S = num / den;
      const double Z = mu - S * cbar;
      uint8_t* cb = codes + n * (K / 4) + g * 8;
      for (int j = 0; j < 8; ++j)
        cb[j] = (uint8_t)(q[4 * j] | (q[4 * j + 1] << 2) | (q[4 * j + 2] << 4) | (q[4 * j + 3] << 6));
      scales[n * G + g] = f64_to_f16(S);
      zeros[n * G + g] = f64_to_f16(Z);
    }
  }
  return wq::ok();
}

int wq_select_outliers(const float* W, int64_t N, int64_t K, const double* profile, double ratio,
                       int32_t* idx, int64_t idx_cap, int64_t* n_out) {
  if (int r = wq::check_shape(N, K, "wq_select_outliers")) return r;
  if (!W || !profile || !n_out) return fail(WQ_ERR_INVALID_ARG, "wq_select_outliers: NULL pointer");
  if (!(ratio >= 0.0 && ratio <= 1.0))
    return fail(WQ_ERR_INVALID_ARG, "wq_select_outliers: ratio must be in [0, 1]");
  const int64_t n = (int64_t)std::floor(ratio * (double)K);
  if (n > idx_cap || (n > 0 && !idx))
    return fail(WQ_ERR_INVALID_ARG, "wq_select_outliers: idx holds %lld entries, %lld needed",
                (long long)idx_cap, (long long)n);
  std::vector<double> acc((size_t)K, 0.0);
  for (int64_t r = 0; r < N; ++r) {
    const float* row = W + r * K;
    for (int64_t c = 0; c < K; ++c) {
      const double v = (double)row[c];
      acc[c] = acc[c] + v * v;
    }
  }
  std::vector<double> score((size_t)K);
  for (int64_t c = 0; c < K; ++c) score[c] = std::sqrt(acc[c]) * profile[c];
  std::vector<int32_t> order((size_t)K);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return score[a] > score[b]; });
  std::sort(order.begin(), order.begin() + n);
  for (int64_t j = 0; j < n; ++j) idx[j] = order[j];
  *n_out = n;
  return wq::ok();
}

int wq_select_outliers_kurtosis(const float* W, int64_t N, int64_t K, const double* gamma,
                                double r_base, int32_t* idx, int64_t idx_cap, int64_t* n_out,
                                double* ratio, double* kappa) {
  const char* who = "wq_select_outliers_kurtosis";
  if (int r = wq::check_shape(N, K, who)) return r;
  if (!W || !n_out) return fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!(r_base > 0.0 && r_base <= 1.0))
    return fail(WQ_ERR_INVALID_ARG, "%s: r_base must be in (0, 1]", who);
  // saliency S_c = |gamma_c| ||W[:, c]||_2, the column norm summed over rows in order
  std::vector<double> acc((size_t)K, 0.0);
  for (int64_t r = 0; r < N; ++r) {
    const float* row = W + r * K;
    for (int64_t c = 0; c < K; ++c) {
      const double v = (double)row[c];
      acc[c] = acc[c] + v * v;
    }
  }
  std::vector<double> S((size_t)K);
  for (int64_t c = 0; c < K; ++c) S[c] = std::sqrt(acc[c]) * (gamma ? std::fabs(gamma[c]) : 1.0);
  // population kurtosis, every sum left to right; no spread -> 0
  double sum = 0.0;
  for (int64_t c = 0; c < K; ++c) sum = sum + S[c];
  const double mu = sum / (double)K;
  double var = 0.0;
  for (int64_t c = 0; c < K; ++c) {
    const double d = S[c] - mu;
    var = var + d * d;
  }
  var = var / (double)K;
  double kap = 0.0;
  if (var != 0.0) {
    const double sd = std::sqrt(var);
    double m4 = 0.0;
    for (int64_t c = 0; c < K; ++c) {
      const double z = (S[c] - mu) / sd;
      const double z2 = z * z;
      m4 = m4 + z2 * z2;
    }
    kap = m4 / (double)K;
  }
  const double ex = kap - 3.0 > 0.0 ? kap - 3.0 : 0.0;
  double rr = r_base * (1.0 + 0.15 * std::log1p(ex));
  rr = std::min(std::max(rr, 0.005), 0.03);
  const int64_t n = (int64_t)std::floor(rr * (double)K);
  if (n > idx_cap || (n > 0 && !idx))
    return fail(WQ_ERR_INVALID_ARG, "%s: idx holds %lld entries, %lld needed", who,
                (long long)idx_cap, (long long)n);
  std::vector<int32_t> order((size_t)K);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return S[a] > S[b]; });
  std::sort(order.begin(), order.begin() + n);
  for (int64_t j = 0; j < n; ++j) idx[j] = order[j];
  *n_out = n;
  if (ratio) *ratio = rr;
  if (kappa) *kappa = kap;
  return wq::ok();
}

int wq_pack_zeros_w4(const uint16_t* zeros, int64_t N, int64_t K, uint8_t* zeros_packed) {
  if (int r = wq::check_shape(N, K, "wq_pack_zeros_w4")) return r;
  if (!zeros || !zeros_packed) return fail(WQ_ERR_INVALID_ARG, "wq_pack_zeros_w4: NULL pointer");
  const int64_t G = K / WQ_GROUP, Gp = (G + 1) / 2;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < Gp; ++m) {
      uint32_t b = 0;
      for (int64_t h = 0; h < 2 && 2 * m + h < G; ++h) {
        const float z = f16_to_f32(zeros[n * G + 2 * m + h]);
        if (!(z >= 0.f && z <= 15.f && z == (float)(int)z))
          return fail(WQ_ERR_INVALID_ARG,
                      "wq_pack_zeros_w4: zero point of row %lld group %lld is not an integer "
                      "in 0..15", (long long)n, (long long)(2 * m + h));
        b |= (uint32_t)z << (4 * h);
      }
      zeros_packed[n * Gp + m] = (uint8_t)b;
    }
  }
  return wq::ok();
}

int wq_split_outliers(const float* W, int64_t N, int64_t K, const int32_t* idx, int64_t n_out,
                      float* W_dense, uint16_t* W_out) {
  if (int r = wq::check_shape(N, K, "wq_split_outliers")) return r;
  if (!W || !W_dense || (n_out > 0 && (!idx || !W_out)))
    return fail(WQ_ERR_INVALID_ARG, "wq_split_outliers: NULL pointer");
  if (n_out < 0 || n_out > K) return fail(WQ_ERR_INVALID_ARG, "wq_split_outliers: bad n_out");
  for (int64_t j = 0; j < n_out; ++j) {
    if (idx[j] < 0 || idx[j] >= K || (j > 0 && idx[j] <= idx[j - 1]))
      return fail(WQ_ERR_INVALID_ARG,
                  "wq_split_outliers: idx must be strictly increasing within [0, K)");
  }
  for (int64_t r = 0; r < N; ++r) {
    const float* src = W + r * K;
    float* dst = W_dense + r * K;
    for (int64_t j = 0; j < n_out; ++j) W_out[r * n_out + j] = f32_to_f16(src[idx[j]]);
    if (dst != src) std::memcpy(dst, src, sizeof(float) * (size_t)K);
    for (int64_t j = 0; j < n_out; ++j) dst[idx[j]] = 0.0f;
  }
  return wq::ok();
}

int wq_dequant_host(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                    int64_t N, int64_t K, uint16_t* W_hat) {
  if (fmt != WQ_FMT_W4 && fmt != WQ_FMT_W2 && fmt != WQ_FMT_W4P)
    return fail(WQ_ERR_INVALID_ARG,
                "wq_dequant_host: fmt must be WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2");
  if (int r = wq::check_shape(N, K, "wq_dequant_host")) return r;
  if (!codes || !scales || !zeros || !W_hat)
    return fail(WQ_ERR_INVALID_ARG, "wq_dequant_host: NULL pointer");
  const int64_t G = K / WQ_GROUP;
  float C[4];
  for (int i = 0; i < 4; ++i) C[i] = f16_to_f32(kCodebookF16[i]);
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < G; ++g) {
      const float s = f16_to_f32(scales[n * G + g]);
      float z;
      if (fmt == WQ_FMT_W4P) {
        const uint8_t* zp = reinterpret_cast<const uint8_t*>(zeros) + n * ((G + 1) / 2);
        z = (float)((zp[g / 2] >> (4 * (g % 2))) & 0x0F);
      } else {
        z = f16_to_f32(zeros[n * G + g]);
      }
      uint16_t* out = W_hat + n * K + g * WQ_GROUP;
      if (fmt == WQ_FMT_W4 || fmt == WQ_FMT_W4P) {
        const uint8_t* c = codes + n * (K / 2) + g * 16;
        for (int k = 0; k < 16; ++k) {
          const float lo = (float)(c[k] & 0x0F) - z;
          const float hi = (float)(c[k] >> 4) - z;
          out[k] = f32_to_f16(lo * s);
          out[k + 16] = f32_to_f16(hi * s);
        }
      } else {
        const uint8_t* c = codes + n * (K / 4) + g * 8;
        for (int k = 0; k < WQ_GROUP; ++k) {
          const int q = (c[k >> 2] >> (2 * (k & 3))) & 3;
          float w = s * C[q];
          w = w + z;
          out[k] = f32_to_f16(w);
        }
      }
    }
  }
  return wq::ok();
}

int64_t wq_tiled_bytes(int fmt, int64_t N, int64_t K, int64_t n_out) {
  if (fmt != WQ_FMT_W4 && fmt != WQ_FMT_W2 && fmt != WQ_FMT_W4P)
    return fail(WQ_ERR_INVALID_ARG,
                "wq_tiled_bytes: fmt must be WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2");
  if (int r = wq::check_shape(N, K, "wq_tiled_bytes")) return r;
  if (n_out < 0 || n_out > K)
    return fail(WQ_ERR_INVALID_ARG, "wq_tiled_bytes: n_out must be in [0, K]");
  wq::ok();
  return wq::tiled_geometry(fmt, N, K, n_out).total;
}

int wq_tile_host(int fmt, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                 const uint16_t* out_w, int64_t N, int64_t K, int64_t n_out, uint8_t* tiled,
                 int64_t tiled_bytes) {
  const int64_t need = wq_tiled_bytes(fmt, N, K, n_out);
  if (need < 0) return (int)need;
  if (!codes || !scales || !zeros || !tiled || (n_out > 0 && !out_w))
    return fail(WQ_ERR_INVALID_ARG, "wq_tile_host: NULL pointer");
  if (tiled_bytes < need)
    return fail(WQ_ERR_INVALID_ARG, "wq_tile_host: tiled buffer holds %lld bytes, %lld needed",
                (long long)tiled_bytes, (long long)need);
  const wq::TiledGeometry g = wq::tiled_geometry(fmt, N, K, n_out);
  const int64_t row_bytes = fmt == WQ_FMT_W2 ? K / 4 : K / 2;
  const int64_t G = K / WQ_GROUP;
  const int64_t SB = g.slice_bytes;
  std::memset(tiled, 0, (size_t)g.total);
  auto put16 = [](uint8_t* dst, uint16_t v) { std::memcpy(dst, &v, 2); };
  for (int64_t b = 0; b < g.nrb; ++b) {
    for (int64_t s = 0; s < g.nks; ++s) {
      const int64_t tile = b * g.nks + s;
      uint8_t* ct = tiled + g.codes_off + tile * 16 * SB;
      uint8_t* mt = tiled + g.meta_off + tile * g.meta_tile;
      for (int64_t n = 0; n < 16; ++n) {
        const int64_t row = 16 * b + n;
        if (row >= N) break;
        for (int64_t r = 0; r < 4; ++r) {
          const int64_t lane = n + 16 * r;
          for (int64_t u = 0; u < SB / 64; ++u)
            for (int64_t c = 0; c < 16; ++c) {
              const int64_t col = s * SB + 64 * u + 16 * r + c;
              if (col < row_bytes) ct[1024 * u + 16 * lane + c] = codes[row * row_bytes + col];
            }
          if (fmt == WQ_FMT_W4P) {
            const uint8_t* zp = reinterpret_cast<const uint8_t*>(zeros) + row * ((G + 1) / 2);
            for (int64_t i = 0; i < 4; ++i) {
              const int64_t grp = 16 * s + 4 * r + i;
              if (grp < G) put16(mt + 2 * (4 * lane + i), scales[row * G + grp]);
            }
            for (int64_t j = 0; j < 2; ++j) {
              const int64_t m = 8 * s + 2 * r + j;
              if (m < (G + 1) / 2) mt[512 + 2 * lane + j] = zp[m];
            }
          } else {
            for (int64_t i = 0; i < 4; ++i) {
              const int64_t grp = 16 * s + 4 * r + i;
              if (grp >= G) continue;
              put16(mt + 2 * (8 * lane + i), scales[row * G + grp]);
              put16(mt + 2 * (8 * lane + 4 + i), zeros[row * G + grp]);
            }
          }
        }
      }
    }
    for (int64_t c = 0; c < g.nch; ++c) {
      uint8_t* ot = tiled + g.slab_off + (b * g.nch + c) * 256;
      for (int64_t n = 0; n < 16; ++n) {
        const int64_t row = 16 * b + n;
        if (row >= N) break;
        for (int64_t i = 0; i < 8; ++i) {
          const int64_t j = 8 * c + i;
          if (j < n_out) put16(ot + 2 * (8 * n + i), out_w[row * n_out + j]);
        }
      }
    }
  }
  return wq::ok();
}

int wq_refinement_w4(int fmt, const float* W, const uint8_t* codes, const uint16_t* scales,
                     const uint16_t* zeros, int64_t N, int64_t K, const int32_t* out_idx,
                     int64_t n_out, uint8_t* rcodes, uint16_t* rscales, uint16_t* rzeros) {
  const char* who = "wq_refinement_w4";
  if (fmt != WQ_FMT_W4 && fmt != WQ_FMT_W2 && fmt != WQ_FMT_W4P)
    return fail(WQ_ERR_INVALID_ARG, "%s: fmt must be WQ_FMT_W4, WQ_FMT_W4P or WQ_FMT_W2", who);
  if (int r = wq::check_shape(N, K, who)) return r;
  if (N % WQ_GROUP != 0 || N > WQ_MAX_K)
    return fail(WQ_ERR_UNSUPPORTED, "%s: N must be a multiple of 32 up to %d", who, WQ_MAX_K);
  if (n_out < 0 || n_out > K)
    return fail(WQ_ERR_INVALID_ARG, "%s: n_out must be in [0, K] (got %lld)", who,
                (long long)n_out);
  if (!W || !codes || !scales || !zeros || !rcodes || !rscales || !rzeros ||
      (n_out > 0 && !out_idx))
    return fail(WQ_ERR_INVALID_ARG, "%s: NULL pointer", who);
  for (int64_t j = 0; j < n_out; ++j)
    if (out_idx[j] < 0 || out_idx[j] >= K || (j > 0 && out_idx[j] <= out_idx[j - 1]))
      return fail(WQ_ERR_INVALID_ARG, "%s: out_idx must be strictly increasing in [0, K)", who);
  const int64_t G = K / WQ_GROUP, Gn = N / WQ_GROUP;
  const int64_t row_bytes = fmt == WQ_FMT_W2 ? K / 4 : K / 2;
  const int64_t zrow = fmt == WQ_FMT_W4P ? (G + 1) / 2 : 2 * G;   // bytes of zero points per row
  std::vector<uint8_t> outlier(K, 0);
  for (int64_t j = 0; j < n_out; ++j) outlier[out_idx[j]] = 1;
  // 32 output rows at a time: their dequantized weights, then R^T of the block
  // ([K][32]: one refinement group per input channel), quantized group by group
  std::vector<uint16_t> what((size_t)WQ_GROUP * K);
  std::vector<float> rt((size_t)K * WQ_GROUP);
  for (int64_t gn = 0; gn < Gn; ++gn) {
    const int64_t n0 = gn * WQ_GROUP;
    const uint16_t* zrows =
        reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(zeros) + n0 * zrow);
    if (int r = wq_dequant_host(fmt, codes + n0 * row_bytes, scales + n0 * G, zrows, WQ_GROUP, K,
                                what.data()))
      return r;
    for (int64_t r = 0; r < WQ_GROUP; ++r)
      for (int64_t k = 0; k < K; ++k)
        rt[k * WQ_GROUP + r] =
            outlier[k] ? 0.0f : W[(n0 + r) * K + k] - f16_to_f32(what[r * K + k]);
    for (int64_t k = 0; k < K; ++k)
      quantize_w4_group(&rt[k * WQ_GROUP], rcodes + k * (N / 2) + gn * 16, rscales + k * Gn + gn,
                        rzeros + k * Gn + gn);
  }
  return wq::ok();
}

}  // extern "C"
