// Plain, single-threaded C++ oracle of one compression-phase step of 1-bit
// Adam, of one warmup-phase (uncompressed Adam) step, and of one exchange of
// ScaleCom's cyclic local top-k codec, for one tensor.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the
// build entry module and the CPU-baseline leg of the benchmark load this
// library.  It shares no code with the HIP library (no header, no helper, no
// table) and the HIP library never loads it.
//
// Source pages: the nubint.ai review of "1-bit Adam: Communication Efficient
// Large-Scale Training with Adam's Convergence Speed" (Tang, Gan et al.).  In
// the compression phase, Adam's variance is frozen and used as a fixed
// preconditioner (Abstract; Proposed method, bullet 2), and training runs as
// momentum SGD whose momentum is sent with error-compensated 1-bit
// compression (One-line summary; Proposed method, bullets 1 and 3) through a
// collective (bullet 4), here a local average of the W workers' messages
// followed by a server-side re-compression with its own error buffer.
//
// The pages give no formulas.  The readings taken (the same as the numpy
// oracle's R1-R9):
//   scale     s = fp32( sqrt64( fl64(exact sum of x_i^2) / n ) )       (R1)
//   sign bit  x >= 0 gives 1 (also for -0); NaN gives 0                (R2)
//   layout    uint64 words, bit k of word j is element 64 j + k;
//             bits past the tensor's end are 0                         (R3)
//   one scale per (worker, tensor), one for the server                 (R4)
//   momentum  m_w = c1*m + c2*g_w, c1 = fp32(beta1),
//             c2 = fp32(1 - beta1) with the complement in double      (R5)
//   average   ascending fp32 sum over workers from +0, then / W        (R6)
//   momentum after the step: the server's reconstruction               (R7)
//   update    p - lr*(m/(sqrt(v)+eps)), fp32, correctly rounded       (R8)
//   a NaN or Inf anywhere in a tensor makes its scale NaN              (R9)
//   partitioned server: one scale per chunk of whole 8192-element blocks (R11)
//   1-bit LAMB's layer-wise trust ratio on the update                  (R14)
//   warmup    Adam on the R6 average of the gradients, v with
//             b2 = fp32(beta2), cb2 = fp32(1 - beta2), no bias correction (R10)
// Every fp32 product and sum below is its own statement and the file is
// compiled with -ffp-contract=off, so each rounds once.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// exact sum of squares of fp32 values (R1)
//
// |x| = M * 2^(k - 149) with M < 2^24 an integer and 0 <= k <= 253
// (normal: M = 2^23 + fraction, k = biased exponent - 1; subnormal: M =
// fraction, k = 0).  So x^2 = M^2 * 2^(2k - 298) with M^2 < 2^48, and
// 2^298 * sum x^2 = sum over k of B_k * 2^(2k), B_k = sum of M^2 over the
// elements with exponent index k (below 2^88 for up to 2^40 terms: exact in
// 128 bits).  The total is an integer below 2^(506 + 88): ten 64-bit limbs
// hold it exactly.
// ---------------------------------------------------------------------------
constexpr int kLimbs = 10;

struct BigSum {
  uint64_t limb[kLimbs] = {};

  // += v * 2^shift
  void add(uint64_t v, int shift) {
    int i = shift / 64;
    const int b = shift % 64;
    unsigned __int128 part = static_cast<unsigned __int128>(v) << b;   // < 2^127
    unsigned __int128 carry = 0;
    while ((part != 0 || carry != 0) && i < kLimbs) {   // the total stays below 2^640
      const unsigned __int128 t = static_cast<unsigned __int128>(limb[i]) +
                                  static_cast<uint64_t>(part) + carry;
      limb[i] = static_cast<uint64_t>(t);
      carry = t >> 64;
      part >>= 64;
      ++i;
    }
  }

  int top_bit() const {   // index of the highest set bit, -1 for zero
    for (int i = kLimbs - 1; i >= 0; --i)
      if (limb[i] != 0) return 64 * i + 63 - __builtin_clzll(limb[i]);
    return -1;
  }

  bool bit(int pos) const { return pos >= 0 && ((limb[pos / 64] >> (pos % 64)) & 1u); }

  bool any_below(int pos) const {   // any set bit at an index < pos
    for (int i = 0; i < kLimbs && 64 * i < pos; ++i) {
      const int hi = pos - 64 * i;   // bits [0, hi) of this limb count
      const uint64_t mask = hi >= 64 ? ~0ull : ((1ull << hi) - 1);
      if (limb[i] & mask) return true;
    }
    return false;
  }

  // this * 2^-298 rounded once to the nearest double, ties to even
  double to_double() const {
    const int h = top_bit();
    if (h < 0) return 0.0;
    uint64_t sig = 0;   // the 53 bits [h-52, h], or all of them when h <= 52
    const int lo = h >= 52 ? h - 52 : 0;
    for (int pos = h; pos >= lo; --pos) sig = (sig << 1) | (bit(pos) ? 1u : 0u);
    if (h > 52) {
      const bool half = bit(lo - 1);
      const bool sticky = any_below(lo - 1);
      if (half && (sticky || (sig & 1u))) sig += 1;   // may reach 2^53: still exact below
    }
    return std::ldexp(static_cast<double>(sig), lo - 298);
  }
};

double exact_sum_of_squares(const float *x, int64_t n) {
  unsigned __int128 bucket[254] = {};   // B_k
  for (int64_t i = 0; i < n; ++i) {
    if (!std::isfinite(x[i])) return std::nan("");
    uint32_t u;
    std::memcpy(&u, &x[i], 4);
    const uint32_t biased = (u >> 23) & 0xFFu;
    const uint32_t frac = u & 0x7FFFFFu;
    const uint64_t M = biased > 0 ? (frac | 0x800000u) : frac;
    const int k = biased > 0 ? static_cast<int>(biased) - 1 : 0;
    bucket[k] += M * M;
  }
  BigSum acc;
  for (int k = 0; k < 254; ++k) {
    acc.add(static_cast<uint64_t>(bucket[k]), 2 * k);
    acc.add(static_cast<uint64_t>(bucket[k] >> 64), 2 * k + 64);
  }
  return acc.to_double();
}

float onebit_scale(const float *x, int64_t n) {
  const double S = exact_sum_of_squares(x, n);
  const double q = S / static_cast<double>(n);
  return static_cast<float>(std::sqrt(q));
}

// gradient element i of a row-major array: fp32, or a bf16 bit pattern
// widened exactly (bf16 is the upper half of the fp32 with the same value)
float gradient(const void *g, int32_t bf16, size_t i) {
  if (!bf16) return static_cast<const float *>(g)[i];
  const uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t *>(g)[i]) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

bool sign_bit(float x) { return x >= 0.0f; }   // R2

void pack_signs(const float *x, int64_t n, uint64_t *words) {
  const int64_t nw = (n + 63) / 64;
  for (int64_t j = 0; j < nw; ++j) words[j] = 0;
  for (int64_t i = 0; i < n; ++i) words[i / 64] |= static_cast<uint64_t>(sign_bit(x[i])) << (i % 64);
}

bool unpacked_bit(const uint64_t *words, int64_t i) { return (words[i / 64] >> (i % 64)) & 1u; }

// decompress of one element of a 1-bit message
float decompressed(const uint64_t *words, float s, int64_t i) { return unpacked_bit(words, i) ? s : -s; }

}  // namespace

extern "C" {

double ref_sum_of_squares(const float *x, int64_t n) { return exact_sum_of_squares(x, n); }

float ref_scale(const float *x, int64_t n) { return onebit_scale(x, n); }

void ref_pack_signs(const float *x, int64_t n, uint64_t *words) { pack_signs(x, n, words); }

// One compression-phase step of one tensor of n elements with W workers, with
// the server partitioned into C chunks (R11: chunk j covers [j*S, min((j+1)*S,
// n)), S = 8192*ceil(ceil(n/8192)/C), each with its own scale; C = 1 is one
// scale per tensor) and, when trust != 0, the update scaled by the layer-wise
// trust ratio of 1-bit LAMB (R14: u = m/(sqrt(v)+eps), plus wd*p when wd > 0;
// r = fp32(sqrt(fl64(sum p^2)) / sqrt(fl64(sum u^2))), 1 when a sum is 0;
// p - lr*(r*u)).
//   g        [W] rows of n gradients, row w at g + w*ldg elements: fp32, or
//            bf16 bit patterns (uint16) when g_bf16 != 0 (widened exactly: the
//            bf16 bits are the upper half of the fp32 with the same value)
//   p, m     [n] parameters and the shared momentum, read and overwritten
//   v        [n] frozen variance
//   err_s    [n] server error, read and overwritten
//   err_w    [W] rows of n worker errors (row w at err_w + w*lde), read and
//            overwritten
//   packed_w [W] rows of ceil(n/64) words (row w at packed_w + w*ldp) and
//            scale_w[w*lds]: the worker messages (written)
//   packed_s [ceil(n/64)] and scale_s [chunks]: the server message (written)
// The strides let a caller run the step in place on one tensor of a padded
// flat list whose per-worker rows are N elements long.
// Returns 0, or 1 for a bad argument (n < 1, W < 1, C < 1, a null pointer, a
// stride shorter than a row).
int ref_compression_step_strided(int64_t n, int32_t W, const void *g, int32_t g_bf16, int64_t ldg,
                                 double beta1, double lr, double eps, int32_t chunks, int32_t trust, double wd,
                                 float *p, float *m, const float *v, float *err_s, float *err_w, int64_t lde,
                                 uint64_t *packed_w, int64_t ldp, float *scale_w, int64_t lds,
                                 uint64_t *packed_s, float *scale_s) {
  if (n < 1 || W < 1 || chunks < 1 || !g || !p || !m || !v || !err_s || !err_w || !packed_w || !scale_w ||
      !packed_s || !scale_s)
    return 1;
  if (ldg < n || lde < n || ldp < (n + 63) / 64 || lds < 1) return 1;
  const float c1 = static_cast<float>(beta1);          // R5
  const float c2 = static_cast<float>(1.0 - beta1);
  std::vector<float> x(static_cast<size_t>(n));

  // workers, each on its own: momentum, error feedback, 1-bit message, new error
  for (int32_t w = 0; w < W; ++w) {
    float *ew = err_w + static_cast<size_t>(w) * lde;
    uint64_t *words = packed_w + static_cast<size_t>(w) * ldp;
    for (int64_t i = 0; i < n; ++i) {
      const float gi = gradient(g, g_bf16, static_cast<size_t>(w) * ldg + i);
      const float a = c1 * m[i];
      const float b = c2 * gi;
      const float mw = a + b;
      x[i] = mw + ew[i];
    }
    const float s = onebit_scale(x.data(), n);
    pack_signs(x.data(), n, words);
    scale_w[static_cast<size_t>(w) * lds] = s;
    for (int64_t i = 0; i < n; ++i) ew[i] = x[i] - decompressed(words, s, i);   // e = x - C(x)
  }

  // server: average of the decompressed messages, plus its own error
  const float wf = static_cast<float>(W);
  for (int64_t i = 0; i < n; ++i) {
    float acc = 0.0f;
    for (int32_t w = 0; w < W; ++w)
      acc = acc + decompressed(packed_w + static_cast<size_t>(w) * ldp, scale_w[static_cast<size_t>(w) * lds], i);
    const float y = acc / wf;
    x[i] = y + err_s[i];
  }
  // the server's message: signs of every element, one scale per chunk
  const int64_t blocks = (n + 8191) / 8192;
  const int64_t chunk = 8192 * ((blocks + chunks - 1) / chunks);
  for (int64_t lo = 0; lo < n; lo += chunk) {
    const int64_t hi = lo + chunk < n ? lo + chunk : n;
    scale_s[lo / chunk] = onebit_scale(x.data() + lo, hi - lo);
  }
  pack_signs(x.data(), n, packed_s);

  // server error and momentum = the server's reconstruction
  std::vector<float> u(static_cast<size_t>(n));
  const float eps32 = static_cast<float>(eps);
  const float wd32 = static_cast<float>(wd);
  for (int64_t i = 0; i < n; ++i) {
    const float mhat = decompressed(packed_s, scale_s[i / chunk], i);
    err_s[i] = x[i] - mhat;
    m[i] = mhat;
    const float d = std::sqrt(v[i]) + eps32;
    u[i] = mhat / d;
    if (trust && wd > 0.0) {
      const float t = wd32 * p[i];
      u[i] = u[i] + t;
    }
  }
  // preconditioned update, scaled by the trust ratio when asked
  const float lr32 = static_cast<float>(lr);
  float r = 1.0f;
  if (trust) {
    const double sp = exact_sum_of_squares(p, n);
    const double su = exact_sum_of_squares(u.data(), n);
    r = (sp == 0.0 || su == 0.0) ? 1.0f : static_cast<float>(std::sqrt(sp) / std::sqrt(su));
  }
  for (int64_t i = 0; i < n; ++i) {
    const float ru = trust ? r * u[i] : u[i];
    const float step = lr32 * ru;
    p[i] = p[i] - step;
  }
  return 0;
}

// The same step on contiguous [W][n] gradients (fp32), errors and messages.
int ref_compression_step_opts(int64_t n, int32_t W, const float *g, double beta1, double lr, double eps,
                              int32_t chunks, int32_t trust, double wd, float *p, float *m, const float *v,
                              float *err_s, float *err_w, uint64_t *packed_w, float *scale_w,
                              uint64_t *packed_s, float *scale_s) {
  return ref_compression_step_strided(n, W, g, 0, n, beta1, lr, eps, chunks, trust, wd, p, m, v, err_s, err_w,
                                      n, packed_w, (n + 63) / 64, scale_w, 1, packed_s, scale_s);
}

// The step with one server scale per tensor and the plain update.
int ref_compression_step(int64_t n, int32_t W, const float *g, double beta1, double lr, double eps,
                         float *p, float *m, const float *v, float *err_s, float *err_w,
                         uint64_t *packed_w, float *scale_w, uint64_t *packed_s, float *scale_s) {
  return ref_compression_step_opts(n, W, g, beta1, lr, eps, 1, 0, 0.0, p, m, v, err_s, err_w, packed_w,
                                   scale_w, packed_s, scale_s);
}

// One warmup-phase step of one tensor: full-precision Adam on the workers'
// average gradient (the review's Proposed method, bullet 1: Adam for about the
// first 20% of steps), no bias correction (R10):
//   gbar = (ascending fp32 sum over w of g_w, from +0) / W
//   m = c1*m + c2*gbar;  v = b2*v + cb2*(gbar*gbar);  p = p - lr*(m/(sqrt(v)+eps))
// with c1, c2 as in R5 and b2 = fp32(beta2), cb2 = fp32(1 - beta2) (complement
// in double).  g [W][n] fp32; p, m, v [n] read and overwritten.  Returns 0, or
// 1 for a bad argument.
int ref_warmup_step(int64_t n, int32_t W, const float *g, double beta1, double beta2, double lr, double eps,
                    float *p, float *m, float *v) {
  if (n < 1 || W < 1 || !g || !p || !m || !v) return 1;
  const float c1 = static_cast<float>(beta1);
  const float c2 = static_cast<float>(1.0 - beta1);
  const float b2 = static_cast<float>(beta2);
  const float cb2 = static_cast<float>(1.0 - beta2);
  const float wf = static_cast<float>(W);
  const float lr32 = static_cast<float>(lr);
  const float eps32 = static_cast<float>(eps);
  for (int64_t i = 0; i < n; ++i) {
    float acc = 0.0f;
    for (int32_t w = 0; w < W; ++w) acc = acc + g[static_cast<size_t>(w) * n + i];
    const float gbar = acc / wf;
    const float m1 = c1 * m[i];
    const float m2 = c2 * gbar;
    m[i] = m1 + m2;
    const float v1 = b2 * v[i];
    const float sq = gbar * gbar;
    const float v2 = cb2 * sq;
    v[i] = v1 + v2;
    const float d = std::sqrt(v[i]) + eps32;
    const float u = m[i] / d;
    const float step = lr32 * u;
    p[i] = p[i] - step;
  }
  return 0;
}

// One exchange of the cyclic local top-k codec of the ScaleCom review (Proposed
// method: a leader chosen cyclically picks the top-k indices, which every
// worker then uses) with plain error feedback (R15): x_w = mem_w + g_w (fp32);
// the leader is worker step mod W; the index set is the k positions of largest
// |x_leader|, ties to the lower position, listed in ascending order; worker w
// sends x_w there and keeps x_w with those positions zeroed as its memory; the
// server averages the W messages (ascending fp32 sum from +0, then / W).
//   g [W][n] fp32; memory [W][n] read and overwritten; index [k] (positions
//   within the tensor), values [W][k] and average [k] written.
// Returns 0, or 1 for a bad argument (k outside [1, n]).
int ref_cltk_step(int64_t n, int32_t W, int64_t step, int64_t k, const float *g, float *memory,
                  int64_t *index, float *values, float *average) {
  if (n < 1 || W < 1 || k < 1 || k > n || step < 0 || !g || !memory || !index || !values || !average) return 1;
  std::vector<float> x(static_cast<size_t>(W) * n);
  for (size_t i = 0; i < x.size(); ++i) x[i] = memory[i] + g[i];
  const float *lead = x.data() + static_cast<size_t>(step % W) * n;
  // the k first positions in the order (|x_leader| descending, position ascending)
  std::vector<int64_t> order(static_cast<size_t>(n));
  std::iota(order.begin(), order.end(), int64_t{0});
  auto before = [&](int64_t a, int64_t b) {
    const float ka = std::fabs(lead[a]), kb = std::fabs(lead[b]);
    return ka > kb || (ka == kb && a < b);
  };
  std::nth_element(order.begin(), order.begin() + (k - 1), order.end(), before);
  std::sort(order.begin(), order.begin() + k);   // ascending positions
  const float wf = static_cast<float>(W);
  for (int64_t j = 0; j < k; ++j) {
    const int64_t i = order[j];
    index[j] = i;
    float acc = 0.0f;
    for (int32_t w = 0; w < W; ++w) {
      const float xv = x[static_cast<size_t>(w) * n + i];
      values[static_cast<size_t>(w) * k + j] = xv;
      acc = acc + xv;
    }
    average[j] = acc / wf;
  }
  for (size_t i = 0; i < x.size(); ++i) memory[i] = x[i];
  for (int64_t j = 0; j < k; ++j)
    for (int32_t w = 0; w < W; ++w) memory[static_cast<size_t>(w) * n + order[j]] = 0.0f;
  return 0;
}

}  // extern "C"
