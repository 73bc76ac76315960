// HIP kernels (gfx950) of the 1-bit Adam compression-phase step.
//
// Method: the nubint.ai review of "1-bit Adam: Communication Efficient
// Large-Scale Training with Adam's Convergence Speed" — error-compensated
// 1-bit compression of the momentum (Proposed method, bullet 3), exchanged
// between workers (bullet 4), applied as momentum SGD preconditioned by the
// variance frozen after warmup (Abstract; bullet 2).
//
// Every kernel streams HBM: per element it does a handful of fp32 operations
// and, for the scales, an exact fp64 square with a compensated (two-sum)
// accumulation.  Nothing here is a dense contraction, so there is no MFMA.
//
// Element mapping.  A workgroup of 4 wavefronts handles one tile of up to
// 8192 elements of one tensor; wavefront v owns elements [2048 v, 2048 v +
// 2048) of the tile and lane l owns element 64 c + l of that range for
// c = 0..31.  Every load and store of one c is a contiguous 256-byte wave
// access, and __ballot over one c is directly the packed sign word (bit l =
// element 64 c + l), so packing costs one compare per element.
//
// Floating point.  fp32 products and sums are written as separate operations
// and the file is compiled without contraction, so each rounds once, as the
// method's readings require; fp32 sqrt and division are correctly rounded.
#include "internal.h"

#pragma clang fp contract(off)

namespace ob {
namespace {

template <typename G>
__device__ __forceinline__ float grad_value(const G *p);

template <>
__device__ __forceinline__ float grad_value<float>(const float *p) { return *p; }

// bf16 bits are the upper half of the fp32 with the same value: exact widening.
template <>
__device__ __forceinline__ float grad_value<uint16_t>(const uint16_t *p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

// x^2 of an fp32 value is exact in fp64 (48 significant bits); add it to the
// (hi, lo) pair with Knuth's two-sum, so hi + lo carries the running sum
// with a relative error of order 1e-30 rather than 1e-16.
__device__ __forceinline__ void dd_accumulate(double &hi, double &lo, float x) {
  const double xd = static_cast<double>(x);
  const double q = xd * xd;
  const double s = hi + q;
  const double bp = s - hi;
  lo += (hi - (s - bp)) + (q - bp);
  hi = s;
}

// (hi, lo) += (bhi, blo), renormalised.
__device__ __forceinline__ void dd_add(double &hi, double &lo, double bhi, double blo) {
  const double s = hi + bhi;
  const double bp = s - hi;
  double e = (hi - (s - bp)) + (bhi - bp);
  e = e + (lo + blo);
  const double h = s + e;
  lo = e - (h - s);
  hi = h;
}

__device__ __forceinline__ void dd_wave_reduce(double &hi, double &lo) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const double oh = __shfl_xor(hi, d);
    const double ol = __shfl_xor(lo, d);
    dd_add(hi, lo, oh, ol);
  }
}

// Sum the four wavefronts' pairs in a fixed order and store one partial.
// red is a [kWaves] LDS slot owned by this call; the caller alternates two
// slots so one barrier per call suffices.
__device__ __forceinline__ void dd_block_store(double hi, double lo, double2 *red, double2 *out) {
  dd_wave_reduce(hi, lo);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = make_double2(hi, lo);
  __syncthreads();
  if (threadIdx.x == 0) {
    double h = red[0].x, l = red[0].y;
#pragma unroll
    for (int v = 1; v < kWaves; ++v) dd_add(h, l, red[v].x, red[v].y);
    *out = make_double2(h, l);
  }
}

struct Lanes {
  int lane;     // 0..63
  int sub0;     // first element of this wavefront within the tile
  int64_t base; // flat index of that element
  int nwords;   // sign words of this wavefront that fall inside the tile
};

template <bool kFull>
__device__ __forceinline__ Lanes lanes_of(const Tile &tl) {
  Lanes r;
  r.lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  r.sub0 = wave * kSub;
  r.base = tl.start + r.sub0;
  if (kFull) {
    r.nwords = kPerLane;
  } else {
    const int rem = tl.len - r.sub0;
    r.nwords = rem <= 0 ? 0 : (rem >= kSub ? kPerLane : (rem + 63) / 64);
  }
  return r;
}

template <bool kFull>
__device__ __forceinline__ bool in_tile(const Tile &tl, const Lanes &ln, int c) {
  return kFull || (ln.sub0 + 64 * c + ln.lane < tl.len);
}

// ---------------------------------------------------------------------------
// worker pass 1: x = (c1*m + c2*g) + e, sign words, per-tile sum of x^2
// ---------------------------------------------------------------------------
template <typename G, bool kFull>
__device__ __forceinline__ void worker_pass1_tile(const Tile &tl, const G *__restrict__ grads,
                                                  const float *__restrict__ m,
                                                  const float *__restrict__ err_w,
                                                  uint64_t *__restrict__ packed_w,
                                                  double2 *__restrict__ partials, int64_t N,
                                                  int64_t Nw, int num_tiles, int w0, int w1,
                                                  float c1, float c2, double2 *red) {
  const Lanes ln = lanes_of<kFull>(tl);
  float mr[kPerLane];
#pragma unroll
  for (int c = 0; c < kPerLane; ++c)
    mr[c] = in_tile<kFull>(tl, ln, c) ? m[ln.base + 64 * c + ln.lane] : 0.0f;

  for (int w = w0; w < w1; ++w) {
    const G *gw = grads + static_cast<size_t>(w) * N + ln.base + ln.lane;
    const float *ew = err_w + static_cast<size_t>(w) * N + ln.base + ln.lane;
    float gv[kPerLane], ev[kPerLane];
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const bool ok = in_tile<kFull>(tl, ln, c);
      gv[c] = ok ? grad_value(gw + 64 * c) : 0.0f;
      ev[c] = ok ? ew[64 * c] : 0.0f;
    }
    double hi = 0.0, lo = 0.0;
    uint64_t word = 0;
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const float mw = c1 * mr[c] + c2 * gv[c];
      const float x = mw + ev[c];
      const uint64_t bal = __ballot(in_tile<kFull>(tl, ln, c) && x >= 0.0f);
      if (ln.lane == c) word = bal;
      dd_accumulate(hi, lo, x);  // lanes outside the tile hold x = 0 and add nothing
    }
    if (ln.lane < ln.nwords)
      packed_w[static_cast<size_t>(w) * Nw + (ln.base >> 6) + ln.lane] = word;
    dd_block_store(hi, lo, red + (w & 1) * kWaves,
                   partials + static_cast<size_t>(w) * num_tiles + blockIdx.x);
  }
}

template <typename G>
__global__ __launch_bounds__(kBlock) void worker_pass1(Geometry g, const G *__restrict__ grads,
                                                       const float *__restrict__ m,
                                                       const float *__restrict__ err_w,
                                                       uint64_t *__restrict__ packed_w,
                                                       double2 *__restrict__ partials, int w0,
                                                       int w1, float c1, float c2) {
  __shared__ double2 red[2 * kWaves];
  const Tile tl = g.tiles[blockIdx.x];
  if (tl.len == kTile)
    worker_pass1_tile<G, true>(tl, grads, m, err_w, packed_w, partials, g.N, g.Nw, g.num_tiles,
                               w0, w1, c1, c2, red);
  else
    worker_pass1_tile<G, false>(tl, grads, m, err_w, packed_w, partials, g.N, g.Nw, g.num_tiles,
                                w0, w1, c1, c2, red);
}

// ---------------------------------------------------------------------------
// worker pass 2: recompute x, store e = x - s*sign(x)
// ---------------------------------------------------------------------------
template <typename G, bool kFull>
__device__ __forceinline__ void worker_pass2_tile(const Tile &tl, const G *__restrict__ grads,
                                                  const float *__restrict__ m,
                                                  float *__restrict__ err_w,
                                                  const float *__restrict__ scale_w, int64_t N,
                                                  int T, int w0, int w1, float c1, float c2) {
  const Lanes ln = lanes_of<kFull>(tl);
  float mr[kPerLane];
#pragma unroll
  for (int c = 0; c < kPerLane; ++c)
    mr[c] = in_tile<kFull>(tl, ln, c) ? m[ln.base + 64 * c + ln.lane] : 0.0f;

  for (int w = w0; w < w1; ++w) {
    const float s = scale_w[static_cast<size_t>(w) * T + tl.tensor];
    const G *gw = grads + static_cast<size_t>(w) * N + ln.base + ln.lane;
    float *ew = err_w + static_cast<size_t>(w) * N + ln.base + ln.lane;
    float gv[kPerLane], ev[kPerLane];
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const bool ok = in_tile<kFull>(tl, ln, c);
      gv[c] = ok ? grad_value(gw + 64 * c) : 0.0f;
      ev[c] = ok ? ew[64 * c] : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const float mw = c1 * mr[c] + c2 * gv[c];
      const float x = mw + ev[c];
      const float e = x >= 0.0f ? x - s : x + s;
      if (in_tile<kFull>(tl, ln, c)) ew[64 * c] = e;
    }
  }
}

template <typename G>
__global__ __launch_bounds__(kBlock) void worker_pass2(Geometry g, const G *__restrict__ grads,
                                                       const float *__restrict__ m,
                                                       float *__restrict__ err_w,
                                                       const float *__restrict__ scale_w, int w0,
                                                       int w1, float c1, float c2) {
  const Tile tl = g.tiles[blockIdx.x];
  if (tl.len == kTile)
    worker_pass2_tile<G, true>(tl, grads, m, err_w, scale_w, g.N, g.T, w0, w1, c1, c2);
  else
    worker_pass2_tile<G, false>(tl, grads, m, err_w, scale_w, g.N, g.T, w0, w1, c1, c2);
}

// ---------------------------------------------------------------------------
// scale finalize: one wavefront per (row, tensor)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void scale_finalize(Geometry g,
                                                         const double2 *__restrict__ partials,
                                                         int row0, int nrows,
                                                         float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (id >= static_cast<int64_t>(nrows) * g.T) return;  // whole wavefront leaves together
  const int r = static_cast<int>(id / g.T);
  const int t = static_cast<int>(id % g.T);
  const double2 *row = partials + static_cast<size_t>(row0 + r) * g.num_tiles;
  double hi = 0.0, lo = 0.0;
  for (int i = g.tile_begin[t] + lane; i < g.tile_begin[t + 1]; i += 64) {
    const double2 p = row[i];
    dd_add(hi, lo, p.x, p.y);
  }
  dd_wave_reduce(hi, lo);
  if (lane == 0) {
    const double S = hi + lo;                          // fl64 of the sum of squares
    const double q = S / static_cast<double>(g.numel[t]);
    out[static_cast<size_t>(r) * g.T + t] = static_cast<float>(__builtin_sqrt(q));
  }
}

// ---------------------------------------------------------------------------
// server: y = (ascending sum of +-s_w) / W, z = y + e_s
//   kMode 0: per-tile sum of z^2
//   kMode 1: sign words of z, e_s = z - s_s*sign(z)
//   kMode 2: kMode 1 plus m = s_s*sign(z) and the frozen-variance update
// ---------------------------------------------------------------------------
template <bool kFull, int kMode>
__device__ __forceinline__ void server_tile(const Tile &tl, const Geometry &g,
                                            const uint64_t *__restrict__ packed_w,
                                            const float *__restrict__ scale_w,
                                            float *__restrict__ err_s,
                                            double2 *__restrict__ partials,
                                            const float *__restrict__ scale_s,
                                            uint64_t *__restrict__ packed_s,
                                            const float *__restrict__ v, float *__restrict__ m,
                                            float *__restrict__ params, float lr, float eps,
                                            double2 *red) {
  const Lanes ln = lanes_of<kFull>(tl);
  float acc[kPerLane];
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) acc[c] = 0.0f;
  const uint64_t *pw = packed_w + (ln.base >> 6);
  for (int w = 0; w < g.W; ++w) {
    const float s = scale_w[static_cast<size_t>(w) * g.T + tl.tensor];
    const uint64_t *row = pw + static_cast<size_t>(w) * g.Nw;
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const uint64_t word = (kFull || c < ln.nwords) ? row[c] : 0ull;
      const bool bit = (word >> ln.lane) & 1ull;
      acc[c] = acc[c] + (bit ? s : -s);
    }
  }
  const float wf = static_cast<float>(g.W);
  float *es = err_s + ln.base + ln.lane;
  float z[kPerLane];
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    const bool ok = in_tile<kFull>(tl, ln, c);
    const float e_old = ok ? es[64 * c] : 0.0f;
    z[c] = ok ? acc[c] / wf + e_old : 0.0f;
  }
  if (kMode == 0) {
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) dd_accumulate(hi, lo, z[c]);
    dd_block_store(hi, lo, red, partials + static_cast<size_t>(g.W) * g.num_tiles + blockIdx.x);
    return;
  }
  const float ss = scale_s[tl.tensor];
  uint64_t word = 0;
  float vv[kPerLane], pv[kPerLane];
  if (kMode == 2) {
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const bool ok = in_tile<kFull>(tl, ln, c);
      vv[c] = ok ? v[ln.base + 64 * c + ln.lane] : 0.0f;
      pv[c] = ok ? params[ln.base + 64 * c + ln.lane] : 0.0f;
    }
  }
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    const bool ok = in_tile<kFull>(tl, ln, c);
    const bool bit = z[c] >= 0.0f;
    const uint64_t bal = __ballot(ok && bit);
    if (ln.lane == c) word = bal;
    if (ok) {
      es[64 * c] = bit ? z[c] - ss : z[c] + ss;
      if (kMode == 2) {
        const float mv = bit ? ss : -ss;
        const float d = __builtin_sqrtf(vv[c]) + eps;
        const float u = mv / d;
        m[ln.base + 64 * c + ln.lane] = mv;
        params[ln.base + 64 * c + ln.lane] = pv[c] - lr * u;
      }
    }
  }
  if (ln.lane < ln.nwords) packed_s[(ln.base >> 6) + ln.lane] = word;
}

template <int kMode>
__global__ __launch_bounds__(kBlock) void server_kernel(
    Geometry g, const uint64_t *__restrict__ packed_w, const float *__restrict__ scale_w,
    float *__restrict__ err_s, double2 *__restrict__ partials, const float *__restrict__ scale_s,
    uint64_t *__restrict__ packed_s, const float *__restrict__ v, float *__restrict__ m,
    float *__restrict__ params, float lr, float eps) {
  __shared__ double2 red[kWaves];
  const Tile tl = g.tiles[blockIdx.x];
  if (tl.len == kTile)
    server_tile<true, kMode>(tl, g, packed_w, scale_w, err_s, partials, scale_s, packed_s, v, m,
                             params, lr, eps, red);
  else
    server_tile<false, kMode>(tl, g, packed_w, scale_w, err_s, partials, scale_s, packed_s, v, m,
                              params, lr, eps, red);
}

// ---------------------------------------------------------------------------
// update from a server message: m = s_s*sign, p -= lr * m / (sqrt(v) + eps)
// ---------------------------------------------------------------------------
template <bool kFull>
__device__ __forceinline__ void apply_tile(const Tile &tl, const uint64_t *__restrict__ packed_s,
                                           const float *__restrict__ scale_s,
                                           const float *__restrict__ v, float *__restrict__ m,
                                           float *__restrict__ params, float lr, float eps) {
  const Lanes ln = lanes_of<kFull>(tl);
  const float ss = scale_s[tl.tensor];
  const uint64_t *ps = packed_s + (ln.base >> 6);
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    if (!in_tile<kFull>(tl, ln, c)) continue;
    const uint64_t word = ps[c];
    const bool bit = (word >> ln.lane) & 1ull;
    const int64_t i = ln.base + 64 * c + ln.lane;
    const float mv = bit ? ss : -ss;
    const float d = __builtin_sqrtf(v[i]) + eps;
    const float u = mv / d;
    m[i] = mv;
    params[i] = params[i] - lr * u;
  }
}

__global__ __launch_bounds__(kBlock) void apply_update(Geometry g,
                                                       const uint64_t *__restrict__ packed_s,
                                                       const float *__restrict__ scale_s,
                                                       const float *__restrict__ v,
                                                       float *__restrict__ m,
                                                       float *__restrict__ params, float lr,
                                                       float eps) {
  const Tile tl = g.tiles[blockIdx.x];
  if (tl.len == kTile)
    apply_tile<true>(tl, packed_s, scale_s, v, m, params, lr, eps);
  else
    apply_tile<false>(tl, packed_s, scale_s, v, m, params, lr, eps);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
void launch_worker_pass1(const Geometry &g, bool bf16, int w0, int w1, const void *grads,
                         const float *m, const float *err_w, uint64_t *packed_w,
                         double2 *partials, float c1, float c2, hipStream_t s) {
  const dim3 grid(g.num_tiles), block(kBlock);
  if (bf16)
    hipLaunchKernelGGL(worker_pass1<uint16_t>, grid, block, 0, s, g,
                       static_cast<const uint16_t *>(grads), m, err_w, packed_w, partials, w0, w1,
                       c1, c2);
  else
    hipLaunchKernelGGL(worker_pass1<float>, grid, block, 0, s, g,
                       static_cast<const float *>(grads), m, err_w, packed_w, partials, w0, w1, c1,
                       c2);
}

void launch_scale_finalize(const Geometry &g, const double2 *partials, int row0, int nrows,
                           float *out, hipStream_t s) {
  const int64_t waves = static_cast<int64_t>(nrows) * g.T;
  const dim3 grid(static_cast<unsigned>((waves + kWaves - 1) / kWaves)), block(kBlock);
  hipLaunchKernelGGL(scale_finalize, grid, block, 0, s, g, partials, row0, nrows, out);
}

void launch_worker_pass2(const Geometry &g, bool bf16, int w0, int w1, const void *grads,
                         const float *m, float *err_w, const float *scale_w, float c1, float c2,
                         hipStream_t s) {
  const dim3 grid(g.num_tiles), block(kBlock);
  if (bf16)
    hipLaunchKernelGGL(worker_pass2<uint16_t>, grid, block, 0, s, g,
                       static_cast<const uint16_t *>(grads), m, err_w, scale_w, w0, w1, c1, c2);
  else
    hipLaunchKernelGGL(worker_pass2<float>, grid, block, 0, s, g,
                       static_cast<const float *>(grads), m, err_w, scale_w, w0, w1, c1, c2);
}

void launch_server_pass1(const Geometry &g, const uint64_t *packed_w, const float *scale_w,
                         const float *err_s, double2 *partials, hipStream_t s) {
  hipLaunchKernelGGL(server_kernel<0>, dim3(g.num_tiles), dim3(kBlock), 0, s, g, packed_w,
                     scale_w, const_cast<float *>(err_s), partials, nullptr, nullptr, nullptr,
                     nullptr, nullptr, 0.0f, 0.0f);
}

void launch_server_pass2(const Geometry &g, bool update, const uint64_t *packed_w,
                         const float *scale_w, float *err_s, const float *scale_s,
                         uint64_t *packed_s, const float *v, float *m, float *params, float lr,
                         float eps, hipStream_t s) {
  if (update)
    hipLaunchKernelGGL(server_kernel<2>, dim3(g.num_tiles), dim3(kBlock), 0, s, g, packed_w,
                       scale_w, err_s, nullptr, scale_s, packed_s, v, m, params, lr, eps);
  else
    hipLaunchKernelGGL(server_kernel<1>, dim3(g.num_tiles), dim3(kBlock), 0, s, g, packed_w,
                       scale_w, err_s, nullptr, scale_s, packed_s, nullptr, nullptr, nullptr, 0.0f,
                       0.0f);
}

void launch_apply_update(const Geometry &g, const uint64_t *packed_s, const float *scale_s,
                         const float *v, float *m, float *params, float lr, float eps,
                         hipStream_t s) {
  hipLaunchKernelGGL(apply_update, dim3(g.num_tiles), dim3(kBlock), 0, s, g, packed_s, scale_s, v,
                     m, params, lr, eps);
}

}  // namespace ob
