// Runs the C++ oracle (oracle/onebit_ref.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer: ragged sizes, every worker count from 1 to 9,
// special and extreme values, and sums of squares that carry through the top
// limbs of the exact accumulator.  Every buffer has exactly its stated size,
// so an access past it is reported.  Checks a few invariants of each step and
// exits non-zero on a failure; prints "ok" otherwise.
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

extern "C" {
double ref_sum_of_squares(const float *x, int64_t n);
float ref_scale(const float *x, int64_t n);
void ref_pack_signs(const float *x, int64_t n, uint64_t *words);
int ref_compression_step(int64_t n, int32_t W, const float *g, double beta1, double lr, double eps,
                         float *p, float *m, const float *v, float *err_s, float *err_w,
                         uint64_t *packed_w, float *scale_w, uint64_t *packed_s, float *scale_s);
int ref_warmup_step(int64_t n, int32_t W, const float *g, double beta1, double beta2, double lr, double eps,
                    float *p, float *m, float *v);
int ref_cltk_step(int64_t n, int32_t W, int64_t step, int64_t k, const float *g, float *memory,
                  int64_t *index, float *values, float *average);
}

static int failures = 0;

static void expect(bool ok, const char *what, long long a, long long b) {
  if (!ok) {
    std::printf("FAIL %s (%lld, %lld)\n", what, a, b);
    ++failures;
  }
}

int main() {
  std::mt19937 rng(7);
  std::normal_distribution<float> normal(0.0f, 1e-3f);
  const int64_t sizes[] = {1, 2, 63, 64, 65, 1000, 4097};
  for (int64_t n : sizes) {
    const int64_t nw = (n + 63) / 64;
    for (int32_t W = 1; W <= 9; ++W) {
      std::vector<float> g(static_cast<size_t>(W * n)), p(n), m(n, 0.0f), v(n), es(n, 0.0f),
          ew(static_cast<size_t>(W * n), 0.0f), sw(W), ss(1);
      std::vector<uint64_t> pw(static_cast<size_t>(W * nw)), ps(nw);
      for (int64_t i = 0; i < n; ++i) {
        p[i] = normal(rng) * 20.0f;
        v[i] = normal(rng) * normal(rng) + 1e-12f;
      }
      for (int step = 0; step < 2; ++step) {
        for (size_t i = 0; i < g.size(); ++i) g[i] = normal(rng);
        g[0] = -0.0f;
        if (g.size() > 3) g[3] = 1e-42f;   // subnormal
        if (g.size() > 5) g[5] = 1e30f;
        const int st = ref_compression_step(n, W, g.data(), 0.9, 1e-4, 1e-8, p.data(), m.data(), v.data(),
                                            es.data(), ew.data(), pw.data(), sw.data(), ps.data(), ss.data());
        expect(st == 0, "step status", n, W);
        const int tail = static_cast<int>(n % 64);
        if (tail != 0) {   // bits past the tensor's end are 0
          const uint64_t past = ~((1ull << tail) - 1);
          for (int32_t w = 0; w < W; ++w) expect((pw[w * nw + nw - 1] & past) == 0, "worker padding bits", n, w);
          expect((ps[nw - 1] & past) == 0, "server padding bits", n, W);
        }
        for (int64_t i = 0; i < n; ++i) {   // the momentum is the server's reconstruction
          const bool bit = (ps[i / 64] >> (i % 64)) & 1u;
          expect(m[i] == (bit ? ss[0] : -ss[0]), "momentum", n, i);
        }
      }
    }
  }
  // the warmup step and the CLT-k exchange on the same sizes, every k from 1 to n for small n
  for (int64_t n : sizes) {
    for (int32_t W = 1; W <= 9; W += 4) {
      std::vector<float> g(static_cast<size_t>(W * n)), p(n, 0.5f), m(n, 0.0f), v(n, 0.0f),
          mem(static_cast<size_t>(W * n), 0.0f);
      for (size_t i = 0; i < g.size(); ++i) g[i] = (i % 5 == 0) ? 0.0f : normal(rng);   // ties at 0
      expect(ref_warmup_step(n, W, g.data(), 0.9, 0.999, 1e-3, 1e-8, p.data(), m.data(), v.data()) == 0,
             "warmup status", n, W);
      for (int64_t k = 1; k <= n; k += (n < 70 ? 1 : n / 7)) {
        std::vector<int64_t> index(k);
        std::vector<float> values(static_cast<size_t>(W * k)), average(k);
        expect(ref_cltk_step(n, W, k, k, g.data(), mem.data(), index.data(), values.data(), average.data()) == 0,
               "cltk status", n, k);
        for (int64_t j = 1; j < k; ++j) expect(index[j - 1] < index[j], "cltk index ascending", n, j);
      }
    }
  }
  // sums of squares at the ends of the fp32 range; 2^16 copies of FLT_MAX carry
  // into the top limbs (FLT_MAX^2 has 48 significant bits: every sum is exact)
  const int64_t big = 1 << 16;
  std::vector<float> top(big, FLT_MAX), tiny(big, 1e-45f);
  const double fm = static_cast<double>(FLT_MAX);
  expect(ref_sum_of_squares(top.data(), big) == static_cast<double>(big) * (fm * fm), "FLT_MAX sum", big, 0);
  expect(ref_scale(top.data(), big) == FLT_MAX, "FLT_MAX scale", big, 0);
  const double dm = std::ldexp(1.0, -149);
  expect(ref_sum_of_squares(tiny.data(), big) == static_cast<double>(big) * (dm * dm), "denorm sum", big, 0);
  std::vector<uint64_t> words(1);
  const float signs[3] = {-0.0f, NAN, -1.0f};
  ref_pack_signs(signs, 3, words.data());
  expect(words[0] == 1u, "pack of -0, NaN, -1", static_cast<long long>(words[0]), 1);
  if (failures == 0) std::printf("ok\n");
  return failures == 0 ? 0 : 1;
}
