// Drives every host entry point of the library's C ABI (the encoders in
// wq_host.cpp) on seeded inputs of several shapes, with every output buffer
// allocated at exactly the size the header states, plus the documented error
// paths.  Built with AddressSanitizer and UndefinedBehaviorSanitizer by the
// CPU test suite: any out-of-bounds access, use of uninitialised or freed
// memory, signed overflow or misaligned access aborts the run.  Checks made
// here are structural (return codes, counts, orderings, round trips); the
// values themselves are pinned against the oracle by the other host tests.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "wq.h"

namespace {

int g_fail = 0;

#define CHECK(cond)                                                             \
  do {                                                                          \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                                 \
    }                                                                           \
  } while (0)

// splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014): seeded uniform bits for the test weights.
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return (next() >> 11) * (1.0 / 9007199254740992.0); }
  float weight() {   // a sum of uniforms: bell-shaped, mean 0
    double a = 0;
    for (int i = 0; i < 4; ++i) a += uniform() - 0.5;
    return (float)(0.02 * a);
  }
};

float h2f(uint16_t h) {
  const uint32_t s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0) v = std::ldexp((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp((float)(m | 1024), (int)e - 25);
  return s ? -v : v;
}

void run_shape(int64_t N, int64_t K, double ratio, uint64_t seed) {
  Rng rng{seed};
  const int64_t G = K / 32;
  std::vector<float> W((size_t)(N * K));
  for (auto& w : W) w = rng.weight();
  for (int64_t n = 0; n < N; ++n) W[(size_t)(n * K + (K / 3))] *= 40.0f;   // one spiked channel
  std::vector<double> profile((size_t)K);
  for (auto& p : profile) p = 0.5 + rng.uniform();

  // outlier selection, profile-guided and kurtosis-adaptive
  const int64_t cap = (int64_t)std::floor(ratio * (double)K);
  std::vector<int32_t> idx((size_t)(cap > 0 ? cap : 1));
  int64_t n_out = -1;
  CHECK(wq_select_outliers(W.data(), N, K, profile.data(), ratio, idx.data(), cap, &n_out) == 0);
  CHECK(n_out == cap);
  for (int64_t j = 1; j < n_out; ++j) CHECK(idx[(size_t)j - 1] < idx[(size_t)j]);
  const int64_t kcap = (int64_t)std::floor(0.03 * (double)K);
  std::vector<int32_t> kidx((size_t)(kcap > 0 ? kcap : 1));
  int64_t kn = -1;
  double r = 0, kappa = 0;
  CHECK(wq_select_outliers_kurtosis(W.data(), N, K, nullptr, 0.01, kidx.data(), kcap, &kn, &r,
                                    &kappa) == 0);
  CHECK(kn >= 0 && kn <= kcap && r >= 0.005 && r <= 0.03);
  for (int64_t j = 1; j < kn; ++j) CHECK(kidx[(size_t)j - 1] < kidx[(size_t)j]);

  // split: dense residual (in place as well) and the FP16 slab
  std::vector<float> dense((size_t)(N * K));
  std::vector<uint16_t> wout((size_t)(N * (n_out > 0 ? n_out : 1)));
  CHECK(wq_split_outliers(W.data(), N, K, n_out ? idx.data() : nullptr, n_out, dense.data(),
                          wout.data()) == 0);
  for (int64_t j = 0; j < n_out; ++j)
    for (int64_t n = 0; n < N; ++n) CHECK(dense[(size_t)(n * K + idx[(size_t)j])] == 0.0f);
  std::vector<float> inplace(W);
  CHECK(wq_split_outliers(inplace.data(), N, K, n_out ? idx.data() : nullptr, n_out,
                          inplace.data(), wout.data()) == 0);
  CHECK(std::memcmp(inplace.data(), dense.data(), dense.size() * sizeof(float)) == 0);

  for (int fmt : {WQ_FMT_W4, WQ_FMT_W2, WQ_FMT_W4P}) {
    const int64_t row_bytes = fmt == WQ_FMT_W2 ? K / 4 : K / 2;
    std::vector<uint8_t> codes((size_t)(N * row_bytes));
    std::vector<uint16_t> scales((size_t)(N * G)), zeros((size_t)(N * G));
    if (fmt == WQ_FMT_W2)
      CHECK(wq_quantize_w2(dense.data(), N, K, 32, codes.data(), scales.data(), zeros.data()) == 0);
    else
      CHECK(wq_quantize_w4(dense.data(), N, K, 32, codes.data(), scales.data(), zeros.data()) == 0);
    const uint16_t* zarg = zeros.data();
    std::vector<uint8_t> zp((size_t)(N * ((G + 1) / 2)));
    if (fmt == WQ_FMT_W4P) {
      CHECK(wq_pack_zeros_w4(zeros.data(), N, K, zp.data()) == 0);
      for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < G; ++g) {
          const int v = (zp[(size_t)(n * ((G + 1) / 2) + g / 2)] >> (4 * (g & 1))) & 15;
          CHECK((float)v == h2f(zeros[(size_t)(n * G + g)]));
        }
      zarg = reinterpret_cast<const uint16_t*>(zp.data());
    }
    std::vector<uint16_t> what((size_t)(N * K));
    CHECK(wq_dequant_host(fmt, codes.data(), scales.data(), zarg, N, K, what.data()) == 0);
    for (int64_t i = 0; i < N * K; ++i) CHECK(std::isfinite(h2f(what[(size_t)i])));

    // tiled layout into a buffer of exactly the stated size
    const int64_t tb = wq_tiled_bytes(fmt, N, K, n_out);
    CHECK(tb > 0);
    std::vector<uint8_t> tiled((size_t)tb);
    CHECK(wq_tile_host(fmt, codes.data(), scales.data(), zarg, n_out ? wout.data() : nullptr, N, K,
                       n_out, tiled.data(), tb) == 0);
    CHECK(wq_tile_host(fmt, codes.data(), scales.data(), zarg, n_out ? wout.data() : nullptr, N, K,
                       n_out, tiled.data(), tb - 1) < 0);

    // refinement columns (N a multiple of 32)
    if (N % 32 == 0) {
      std::vector<uint8_t> rc((size_t)(K * (N / 2)));
      std::vector<uint16_t> rs((size_t)(K * (N / 32))), rz((size_t)(K * (N / 32)));
      CHECK(wq_refinement_w4(fmt, W.data(), codes.data(), scales.data(), zarg, N, K,
                             n_out ? idx.data() : nullptr, n_out, rc.data(), rs.data(),
                             rz.data()) == 0);
      for (int64_t j = 0; j < n_out; ++j)      // outlier channels: an all-zero residual
        for (int64_t m = 0; m < N / 2; ++m) CHECK(rc[(size_t)(idx[(size_t)j] * (N / 2) + m)] == 0);
    } else {
      std::vector<uint8_t> rc(16);
      std::vector<uint16_t> rs(16), rz(16);
      CHECK(wq_refinement_w4(fmt, W.data(), codes.data(), scales.data(), zarg, N, K, nullptr, 0,
                             rc.data(), rs.data(), rz.data()) == WQ_ERR_UNSUPPORTED);
    }
  }
}

void error_paths() {
  std::vector<float> W(64 * 64, 0.0f);
  std::vector<uint8_t> codes(64 * 32);
  std::vector<uint16_t> s(64 * 2), z(64 * 2), out(64 * 64);
  std::vector<int32_t> idx(8);
  int64_t n = 0;
  CHECK(wq_quantize_w4(W.data(), 64, 40, 32, codes.data(), s.data(), z.data()) == WQ_ERR_UNSUPPORTED);
  CHECK(wq_quantize_w4(W.data(), 64, 64, 16, codes.data(), s.data(), z.data()) == WQ_ERR_UNSUPPORTED);
  CHECK(wq_quantize_w4(nullptr, 64, 64, 32, codes.data(), s.data(), z.data()) == WQ_ERR_INVALID_ARG);
  CHECK(wq_quantize_w2(W.data(), 0, 64, 32, codes.data(), s.data(), z.data()) == WQ_ERR_INVALID_ARG);
  CHECK(std::strlen(wq_last_error()) > 0);
  CHECK(wq_select_outliers(W.data(), 64, 64, nullptr, 0.1, idx.data(), 8, &n) < 0);
  std::vector<double> prof(64, 1.0);
  CHECK(wq_select_outliers(W.data(), 64, 64, prof.data(), 1.5, idx.data(), 8, &n) == WQ_ERR_INVALID_ARG);
  CHECK(wq_select_outliers(W.data(), 64, 64, prof.data(), 0.5, idx.data(), 8, &n) == WQ_ERR_INVALID_ARG);
  CHECK(wq_select_outliers_kurtosis(W.data(), 64, 64, nullptr, 0.0, idx.data(), 8, &n, nullptr,
                                    nullptr) == WQ_ERR_INVALID_ARG);
  CHECK(wq_select_outliers_kurtosis(W.data(), 64, 64, nullptr, 0.01, idx.data(), 8, &n, nullptr,
                                    nullptr) == 0);   // all saliencies equal: kappa 0
  const int32_t unsorted[3] = {5, 3, 9}, outside[2] = {1, 64};
  CHECK(wq_split_outliers(W.data(), 64, 64, unsorted, 3, W.data(), out.data()) == WQ_ERR_INVALID_ARG);
  CHECK(wq_split_outliers(W.data(), 64, 64, outside, 2, W.data(), out.data()) == WQ_ERR_INVALID_ARG);
  std::vector<uint16_t> bad_z(64 * 2, 0x4C00u);   // 16.0: not a 4-bit zero point
  std::vector<uint8_t> zp(64);
  CHECK(wq_pack_zeros_w4(bad_z.data(), 64, 64, zp.data()) == WQ_ERR_INVALID_ARG);
  CHECK(wq_dequant_host(3, codes.data(), s.data(), z.data(), 64, 64, out.data()) < 0);
  CHECK(wq_tiled_bytes(3, 64, 64, 0) < 0 && wq_tiled_bytes(WQ_FMT_W4, 64, 64, 65) < 0);
  std::vector<uint8_t> rc(64 * 32);
  std::vector<uint16_t> rs(64 * 2), rz(64 * 2);
  CHECK(wq_refinement_w4(WQ_FMT_W4, W.data(), codes.data(), s.data(), z.data(), 64, 64, outside,
                         2, rc.data(), rs.data(), rz.data()) == WQ_ERR_INVALID_ARG);
  CHECK(wq_refinement_w4(WQ_FMT_W4, W.data(), codes.data(), s.data(), z.data(), 64, 64, unsorted,
                         3, rc.data(), rs.data(), rz.data()) == WQ_ERR_INVALID_ARG);
  CHECK(std::strcmp(wq_status_str(WQ_OK), "ok") == 0);
}

}  // namespace

int main() {
  const struct { int64_t N, K; double ratio; } shapes[] = {
      {1, 32, 0.0}, {17, 96, 0.05}, {48, 544, 0.035}, {33, 4128, 0.035}, {64, 1024, 0.2},
      {96, 2048, 0.0}, {160, 4096, 0.035},
  };
  uint64_t seed = 1;
  for (const auto& sh : shapes) run_shape(sh.N, sh.K, sh.ratio, seed++);
  error_paths();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host entry points: all checks passed under the sanitizers\n");
  return 0;
}
