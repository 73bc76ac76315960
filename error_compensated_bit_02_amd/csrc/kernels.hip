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
// kTile elements of one tensor; wavefront v owns elements [v kSub, (v+1) kSub)
// of the tile and lane l owns element 64 c + l of that range for
// c < kPerLane.  Every load and store of one c is a contiguous 256-byte
// wavefront access, and __ballot over one c is directly the packed sign word
// (bit l = element 64 c + l), so packing costs one compare per element.
// Sums of squares are reduced per wavefront, parked in LDS, folded per tile
// in a fixed order (two barriers per tile, none per worker) and per tensor by
// scale_finalize.  Several passes take their tile in chunks of 1024 elements
// instead, one workgroup per chunk (lane l of wavefront v owning element
// 256 v + 64 c + l of the chunk): the parameter update, the warmup step, the
// residual worker pass and, with fp32 gradients, the strict form's pass 2
// (one workgroup per (chunk, worker), one partial sum per chunk).  On MI355X
// a read-modify-write stream runs faster in such 4 KB workgroups; the
// read-mostly strict pass 1 keeps the tiles.
//
// Two forms of the state between steps:
//   strict    err_w / err_s hold the errors and m the momentum (two passes
//             per phase: the error needs the whole-tensor scale);
//   residual  err_w / err_s hold the values that were compressed (x, z) and
//             the scales of that step; the error x - s*sign(x) is formed,
//             exactly as the strict form stores it, when the next step reads
//             it, and the momentum is the server message (+-s_s per sign bit),
//             which it equals exactly.  One pass per phase.
//
// Floating point.  fp32 products and sums are written as separate operations
// and the file is compiled without contraction, so each rounds once; fp32
// sqrt and division are correctly rounded.
#include "internal.h"
#include "worker_runs.h"

#include <mutex>

#pragma clang fp contract(off)

namespace ob {
namespace {

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
// A gradient element.  Every pass reads each gradient row once, so the loads
// are non-temporal: kept out of the caches, they leave them to the rows that
// are read again (the momentum shared by the workers, the rows written back
// in place).  The frozen variance v, read once by the update, is loaded the
// same way (the update 3-4% faster).  Measured on MI355X, bit-identical: the residual worker pass
// 3.1-3.3% faster at BERT-Large and BERT-base, the strict pass 2 up to 9%,
// the warmup step 1.4-5.3%; non-temporal loads of the x rows as well, which
// are read and written back, were neutral or slower.
template <typename G>
__device__ __forceinline__ float grad_value(const G *p);

template <>
__device__ __forceinline__ float grad_value<float>(const float *p) { return __builtin_nontemporal_load(p); }

// bf16 bits are the upper half of the fp32 with the same value: exact widening.
template <>
__device__ __forceinline__ float grad_value<uint16_t>(const uint16_t *p) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_nontemporal_load(p)) << 16);
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

// Per-tile partial sums: each wavefront parks its reduced pair for row r in
// red[r % kFlushRows][wave]; every kFlushRows rows (and after the last) the
// workgroup folds the four wavefronts' pairs in a fixed order and stores one
// partial per (row, tile).  Two barriers per flush, none per row otherwise.
constexpr int kFlushRows = 32;

struct PartialSink {
  double2 (*red)[kWaves];
  double2 *partials;   // row-major [rows][num_tiles]
  int num_tiles;
  int tile;            // column of this workgroup's tile
};

__device__ __forceinline__ void park_partial(const PartialSink &ps, int slot, int wave, double hi,
                                             double lo) {
  dd_wave_reduce(hi, lo);
  if ((threadIdx.x & 63) == 0) ps.red[slot][wave] = make_double2(hi, lo);
}

// Rows [row0, row0 + nrows) parked in slots [0, nrows); workgroup-uniform call.
__device__ __forceinline__ void flush_partials(const PartialSink &ps, int row0, int nrows) {
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < nrows) {
    const int r = threadIdx.x;
    double h = ps.red[r][0].x, l = ps.red[r][0].y;
#pragma unroll
    for (int v = 1; v < kWaves; ++v) dd_add(h, l, ps.red[r][v].x, ps.red[r][v].y);
    ps.partials[static_cast<size_t>(row0 + r) * ps.num_tiles + ps.tile] = make_double2(h, l);
  }
  __syncthreads();
}

// x - s*sign(x) with sign(x) = +1 for x >= 0: the error left by a 1-bit code.
__device__ __forceinline__ float onebit_error(float x, float s) { return x >= 0.0f ? x - s : x + s; }

struct Lanes {
  int lane;      // 0..63
  int wave;      // 0..kWaves-1 (wavefront-uniform)
  int sub0;      // first element of this wavefront within the tile
  int64_t base;  // flat index of that element
  int nwords;    // sign words of this wavefront that fall inside the tile
};

template <bool kFull>
__device__ __forceinline__ Lanes lanes_of(const Tile &tl) {
  Lanes r;
  r.lane = threadIdx.x & 63;
  r.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  r.sub0 = r.wave * kSub;
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

// Sign words of one packed row for this wavefront: lane j < nwords holds word
// j (one coalesced load); word c is broadcast from lane c by readlane.
template <bool kFull>
__device__ __forceinline__ uint64_t load_words(const uint64_t *row, const Lanes &ln) {
  return (kFull ? ln.lane < kPerLane : ln.lane < ln.nwords) ? row[ln.lane] : 0ull;
}

// +-s for this lane's element 64 c + lane, from the words held by load_words.
// Word c, broadcast to scalar registers, is a lane mask (bit l <-> lane l), so
// the choice between s and -s is one v_cndmask with the word as its mask.
__device__ __forceinline__ float signed_scale(uint64_t words, int c, float s) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(words)), c);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(words >> 32)), c);
  const uint64_t word = (static_cast<uint64_t>(hi) << 32) | lo;
  return __builtin_amdgcn_inverse_ballot_w64(word) ? s : -s;
}

// ---------------------------------------------------------------------------
// worker kernels
//   kPass1       strict: x = (c1*m + c2*g) + e; signs; sum of x^2
//   kPass2       strict: recompute x; e = x - s*sign(x)
//   kResidFirst  residual, first step: as kPass1 from stored e and m, and x is stored
//   kResid       residual: e = x_prev - s_prev*sign(x_prev), m = previous server
//                message; then as kResidFirst
//   kPass2Chunk  kPass2 in chunks
// The strict pass 1 runs in tiles (worker_kernel), a group of workers per
// workgroup sharing one load of m; pass 2 too with bf16 gradients.  The
// other modes run in chunks (worker_chunk_kernel), one worker per workgroup:
// kResid worker-major, the modes that read m worker-fastest, so that a
// chunk's W workgroups run together and all but the first read m from cache
// (measured on MI355X: the first residual step 7.87 -> 5.92 ms at BERT-Large;
// chunked pass 2 with fp32 gradients 1.6-4.4% off the strict step, the
// chunked pass 1 and, with bf16 gradients, pass 2 slower than in tiles).
// ---------------------------------------------------------------------------
enum { kPass1 = 0, kPass2 = 1, kResidFirst = 2, kResid = 3, kPass2Chunk = 4 };

template <int kMode, typename G, bool kFull>
__device__ __forceinline__ void worker_tile(const Tile &tl, const Geometry &g, const WorkerArgs &a,
                                            int w_lo, int w_hi, const PartialSink &sink) {
  static_assert(kMode == kPass1 || kMode == kPass2, "the tiled worker pass is the strict form's");
  const Lanes ln = lanes_of<kFull>(tl);
  const int t = tl.tensor;
  float mr[kPerLane];
#pragma unroll
  for (int c = 0; c < kPerLane; ++c)
    mr[c] = in_tile<kFull>(tl, ln, c) ? a.m[ln.base + 64 * c + ln.lane] : 0.0f;

  const G *grads = static_cast<const G *>(a.grads) + ln.base + ln.lane;
  float gv[kPerLane], ev[kPerLane];
  auto load = [&](int w, float *gdst, float *edst) {
    const G *gw = grads + static_cast<size_t>(w) * g.N;
    const float *ew = a.err_w + static_cast<size_t>(w) * g.N + ln.base + ln.lane;
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const bool ok = in_tile<kFull>(tl, ln, c);
      gdst[c] = ok ? grad_value(gw + 64 * c) : 0.0f;
      edst[c] = ok ? ew[64 * c] : 0.0f;
    }
  };
  for (int w = w_lo; w < w_hi; ++w) {
    load(w, gv, ev);
    if (kMode == kPass2) {
      float *ew = a.err_w + static_cast<size_t>(w) * g.N + ln.base + ln.lane;
      const float s = a.scale_w[static_cast<size_t>(w) * g.T + t];   // this step's scale
#pragma unroll
      for (int c = 0; c < kPerLane; ++c) {
        const float mw = a.c1 * mr[c] + a.c2 * gv[c];
        const float x = mw + ev[c];
        if (in_tile<kFull>(tl, ln, c)) ew[64 * c] = onebit_error(x, s);
      }
      continue;
    }
    double hi = 0.0, lo = 0.0;
    LaneWords word;
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const bool ok = in_tile<kFull>(tl, ln, c);
      const float mw = a.c1 * mr[c] + a.c2 * gv[c];
      const float x = ok ? mw + ev[c] : 0.0f;
      const uint64_t bal = __ballot(ok && x >= 0.0f);
      word.put(bal, c);
      dd_accumulate(hi, lo, x);  // lanes outside the tile hold x = 0 and add nothing
    }
    // Non-temporal: the sign words are read only by the server pass.  Cached,
    // one 256-byte row piece per worker beside the other rows slowed a tiled
    // worker pass by ~7% at W = 64 (measured; no effect at W = 8).
    if (ln.lane < ln.nwords)
      __builtin_nontemporal_store(word.get(), &a.packed_w[static_cast<size_t>(w) * g.Nw + (ln.base >> 6) + ln.lane]);
    const int slot = (w - w_lo) % kFlushRows;
    park_partial(sink, slot, ln.wave, hi, lo);
    if (slot == kFlushRows - 1 || w == w_hi - 1) flush_partials(sink, w - slot, slot + 1);
  }
}

// Workgroup b handles tile b % num_tiles for the worker group b / num_tiles
// (workers [w0 + grp*wgroup, ...)): group-major, so the workgroups resident at
// one time stream a few workers' rows through contiguous memory.
template <typename G, int kMode>
__global__ __launch_bounds__(kBlock) void worker_kernel(Geometry g, WorkerArgs a) {
  __shared__ double2 red[kFlushRows][kWaves];
  const int tile = static_cast<int>(blockIdx.x % static_cast<unsigned>(g.num_tiles));
  const int grp = static_cast<int>(blockIdx.x / static_cast<unsigned>(g.num_tiles));
  const int w_lo = a.w0 + grp * a.wgroup;
  const int w_hi = min(a.w1, w_lo + a.wgroup);
  const PartialSink sink{red, a.partials, g.num_tiles, tile};
  const Tile tl = g.tiles[tile];
  if (tl.len == kTile)
    worker_tile<kMode, G, true>(tl, g, a, w_lo, w_hi, sink);
  else
    worker_tile<kMode, G, false>(tl, g, a, w_lo, w_hi, sink);
}

// ---------------------------------------------------------------------------
// residual worker pass, one workgroup per (chunk, worker)
//
// The residual form reads no fp32 momentum (it is the previous server
// message, 1/8 byte per element), so a workgroup can take one worker's row of
// one chunk of kChunk elements at little cost.  Chunks are consecutive
// blockIdx.x, workers blockIdx.y: the workgroups resident at one time stream
// one worker's row through a short window of memory, and consecutive 4 KB
// pieces of it go to consecutive XCDs (workgroups are dispatched to the XCDs
// in turn).  Sums of squares go to one partial per (worker, chunk).
//
// On MI355X this shape beat a tiled pass that loops over the workers of each
// 8192-element tile with fp32 gradients at 8, 32 and 64 workers, and it
// varies far less between processes: at a BERT-Large-sized list with 8
// workers 5.4-5.6 ms against 5.8-6.3 ms in fresh processes, at a
// BERT-base-sized list with 64 workers 13.9-14.1 ms against 15.2-16.7 ms.
// With bf16 gradients (GPT-1.3B-sized list) it took 19.2-19.3 ms against
// 19.1-21.3 ms for the tiled pass.
// ---------------------------------------------------------------------------
constexpr int kChunkSub = kChunk / kWaves;   // elements per wavefront
constexpr int kChunkPerLane = kChunkSub / 64;

template <int kMode, typename G, bool kFull>
__device__ __forceinline__ void worker_chunk(const Tile &tl, int tile, int q, int w, const Geometry &g,
                                             const WorkerArgs &a, double2 *red) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub0 = q * kChunk + wave * kChunkSub;   // first element of this wavefront in the tile
  const int64_t base = tl.start + sub0;
  const int rem = tl.len - sub0;
  const int nwords = kFull ? kChunkPerLane
                           : (rem <= 0 ? 0 : (rem >= kChunkSub ? kChunkPerLane : (rem + 63) / 64));
  auto ok = [&](int c) { return kFull || sub0 + 64 * c + lane < tl.len; };
  const int t = tl.tensor;
  float mr[kChunkPerLane];
  if (kMode == kResid) {
    const float ss = a.scale_s[g.tile_piece[tile]];
    const uint64_t words = lane < nwords ? a.packed_s[(base >> 6) + lane] : 0ull;
#pragma unroll
    for (int c = 0; c < kChunkPerLane; ++c) mr[c] = ok(c) ? signed_scale(words, c, ss) : 0.0f;
  } else {
#pragma unroll
    for (int c = 0; c < kChunkPerLane; ++c) mr[c] = ok(c) ? a.m[base + 64 * c + lane] : 0.0f;
  }
  const size_t row = static_cast<size_t>(w) * g.N + base + lane;
  const G *gw = static_cast<const G *>(a.grads) + row;
  float *ew = a.err_w + row;
  float gv[kChunkPerLane], ev[kChunkPerLane];
#pragma unroll
  for (int c = 0; c < kChunkPerLane; ++c) {
    gv[c] = ok(c) ? grad_value(gw + 64 * c) : 0.0f;
    ev[c] = ok(c) ? ew[64 * c] : 0.0f;
  }
  // kResid: the previous step's scale; kPass2Chunk: this step's
  const float s = (kMode == kResid || kMode == kPass2Chunk) ? a.scale_w[static_cast<size_t>(w) * g.T + t] : 0.0f;
  if (kMode == kPass2Chunk) {
#pragma unroll
    for (int c = 0; c < kChunkPerLane; ++c) {
      const float mw = a.c1 * mr[c] + a.c2 * gv[c];
      const float x = mw + ev[c];
      if (ok(c)) ew[64 * c] = onebit_error(x, s);
    }
    return;
  }
  double hi = 0.0, lo = 0.0;
  LaneWords word;
#pragma unroll
  for (int c = 0; c < kChunkPerLane; ++c) {
    const float e = (kMode == kResid) ? onebit_error(ev[c], s) : ev[c];
    const float mw = a.c1 * mr[c] + a.c2 * gv[c];
    const float x = ok(c) ? mw + e : 0.0f;
    const uint64_t bal = __ballot(ok(c) && x >= 0.0f);
    word.put(bal, c);
    dd_accumulate(hi, lo, x);   // lanes outside the tile hold x = 0 and add nothing
    if (ok(c)) ew[64 * c] = x;
  }
  // non-temporal: the sign words are read only by the server pass
  if (lane < nwords)
    __builtin_nontemporal_store(word.get(), &a.packed_w[static_cast<size_t>(w) * g.Nw + (base >> 6) + lane]);
  dd_wave_reduce(hi, lo);
  if (lane == 0) red[wave] = make_double2(hi, lo);
  __syncthreads();
  if (threadIdx.x == 0) {
    double h = red[0].x, l = red[0].y;
#pragma unroll
    for (int v = 1; v < kWaves; ++v) dd_add(h, l, red[v].x, red[v].y);
    a.chunk_partials[static_cast<size_t>(w) * g.num_tiles * kChunksPerTile +
                     static_cast<size_t>(tile) * kChunksPerTile + q] = make_double2(h, l);
  }
}

template <typename G, int kMode>
__global__ __launch_bounds__(kBlock) void worker_chunk_kernel(Geometry g, WorkerArgs a) {
  __shared__ double2 red[kWaves];
  int tile, q, w;
  if (kMode == kResid) {   // worker-major: chunks along x, workers along y
    tile = static_cast<int>(blockIdx.x / kChunksPerTile);
    q = static_cast<int>(blockIdx.x % kChunksPerTile);
    w = a.w0 + static_cast<int>(blockIdx.y);
  } else {                 // worker-fastest along x
    const unsigned nw = static_cast<unsigned>(a.w1 - a.w0);
    const unsigned chunk = blockIdx.x / nw;
    tile = static_cast<int>(chunk / kChunksPerTile);
    q = static_cast<int>(chunk % kChunksPerTile);
    w = a.w0 + static_cast<int>(blockIdx.x % nw);
  }
  const Tile tl = g.tiles[tile];
  const int rem = tl.len - q * kChunk;   // uniform over the workgroup
  if (rem <= 0) {                        // past the tile's end: an empty partial
    if (kMode != kPass2Chunk && threadIdx.x == 0)
      a.chunk_partials[static_cast<size_t>(w) * g.num_tiles * kChunksPerTile +
                       static_cast<size_t>(tile) * kChunksPerTile + q] = make_double2(0.0, 0.0);
    return;
  }
  if (rem >= kChunk)
    worker_chunk<kMode, G, true>(tl, tile, q, w, g, a, red);
  else
    worker_chunk<kMode, G, false>(tl, tile, q, w, g, a, red);
}

// ---------------------------------------------------------------------------
// scale finalize: kItemWaves wavefronts per (row, tensor) item
//
// One wavefront per item when every item is small; a whole workgroup per item
// when some item has many partials (a 31 M-element embedding has 30,520
// per-chunk partials per worker, which one wavefront reads 8 KB at a time).
// ---------------------------------------------------------------------------
template <int kItemWaves>
__global__ __launch_bounds__(kBlock) void scale_finalize(Geometry g,
                                                         const double2 *__restrict__ partials,
                                                         int64_t cols, int per, int row0, int nrows,
                                                         const int32_t *__restrict__ begin,
                                                         const int64_t *__restrict__ numel,
                                                         int count, float *__restrict__ out) {
  static_assert(kItemWaves == 1 || kItemWaves == kWaves, "a wavefront or a workgroup per item");
  __shared__ double2 red[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = wave % kItemWaves;   // this wavefront's share of its item
  const int64_t id = static_cast<int64_t>(blockIdx.x) * (kWaves / kItemWaves) + wave / kItemWaves;
  if (id >= static_cast<int64_t>(nrows) * count) return;  // the item's wavefronts leave together
  const int r = static_cast<int>(id / count);
  const int item = static_cast<int>(id % count);
  const double2 *row = partials + static_cast<size_t>(row0 + r) * cols;
  // eight independent chains per thread, their loads issued together, then
  // folded in a fixed order: per thread, per wavefront, across the wavefronts
  constexpr int kChains = 8;
  constexpr int kThreads = 64 * kItemWaves;
  double ch[kChains], cl[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) ch[k] = cl[k] = 0.0;
  const int64_t end = static_cast<int64_t>(begin[item + 1]) * per;
  for (int64_t i0 = static_cast<int64_t>(begin[item]) * per + 64 * sub + lane; i0 < end;
       i0 += kThreads * kChains) {
    double2 p[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
      const int64_t i = i0 + kThreads * k;
      p[k] = i < end ? row[i] : make_double2(0.0, 0.0);
    }
#pragma unroll
    for (int k = 0; k < kChains; ++k) dd_add(ch[k], cl[k], p[k].x, p[k].y);
  }
  double hi = ch[0], lo = cl[0];
#pragma unroll
  for (int k = 1; k < kChains; ++k) dd_add(hi, lo, ch[k], cl[k]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const double oh = __shfl_xor(hi, d);
    const double ol = __shfl_xor(lo, d);
    dd_add(hi, lo, oh, ol);
  }
  if (kItemWaves > 1) {   // the whole workgroup is one item: fold the wavefronts in order
    if (lane == 0) red[sub] = make_double2(hi, lo);
    __syncthreads();
    if (threadIdx.x != 0) return;
    hi = red[0].x;
    lo = red[0].y;
#pragma unroll
    for (int v = 1; v < kItemWaves; ++v) dd_add(hi, lo, red[v].x, red[v].y);
  } else if (lane != 0) {
    return;
  }
  const double S = hi + lo;                          // fl64 of the sum of squares
  const double q = S / static_cast<double>(numel[item]);
  out[static_cast<size_t>(r) * count + item] = static_cast<float>(__builtin_sqrt(q));
}

// ---------------------------------------------------------------------------
// server kernels: y = (ascending sum over w of +-s_w) / W, z = y + e_s
//   kS1          strict: sum of z^2
//   kS2          strict: sign words of z; e_s = z - s_s*sign(z)
//   kS2Update    kS2 plus m = s_s*sign(z) and the frozen-variance update
//   kSResidFirst residual, first step: z from the stored e_s; store z, sign words, sum of z^2
//   kSResid      residual: e_s = z_prev - s_s,prev*sign(z_prev); then as kSResidFirst
// ---------------------------------------------------------------------------
enum { kS1 = 0, kS2 = 1, kS2Update = 2, kSResidFirst = 3, kSResid = 4 };

// Each wavefront expands its 32 sign words of every worker through LDS, not
// readlane: it writes the words of kLdsGroup workers into its own LDS region
// as inverted 32-bit halves (the low halves, then the high halves), and lane
// l reads back, with broadcast reads, the 32 halves that hold its bits (the
// low ones for l < 32, the high ones otherwise).  Bit l % 32 of half c,
// sign-extended, is -1 exactly when the sign bit is 0, so its top bit is the
// sign of the term: per (element, worker) one bit-field extract, one and-or
// and the add.  Through readlane it took two readlanes more per word and
// worker; on MI355X this cut the pass from 0.88 to 0.74 ms at 64 workers
// (BERT-base-sized list), from 0.115 to 0.104 ms at 32 (ResNet-50-sized) and
// from 0.59 to 0.57 ms at 8 (BERT-Large-sized), bit-identical.  No barrier is
// needed: every wavefront reads back only what it wrote itself.
constexpr int kLdsGroup = 8;

template <int kMode, bool kFull, bool kPow2>
__device__ __forceinline__ void server_tile(const Tile &tl, const Geometry &g, const ServerArgs &a,
                                            const PartialSink &sink, uint32_t (*lds)[2][kPerLane]) {
  const Lanes ln = lanes_of<kFull>(tl);
  const int t = tl.tensor;
  float acc[kPerLane];
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) acc[c] = 0.0f;
  const uint64_t *pw = a.packed_w + (ln.base >> 6);
  const int half = ln.lane >> 5;
  const int bitpos = ln.lane & 31;
  for (int w0 = 0; w0 < g.W; w0 += kLdsGroup) {
    // the group's word loads are issued together, then summed in ascending worker order
    uint64_t words[kLdsGroup];
    float sw[kLdsGroup];
#pragma unroll
    for (int j = 0; j < kLdsGroup; ++j) {
      const bool live = w0 + j < g.W;
      words[j] = live ? load_words<kFull>(pw + static_cast<size_t>(w0 + j) * g.Nw, ln) : 0ull;
      sw[j] = live ? a.scale_w[static_cast<size_t>(w0 + j) * g.T + t] : 0.0f;
    }
    __builtin_amdgcn_wave_barrier();
    if (ln.lane < kPerLane) {
#pragma unroll
      for (int j = 0; j < kLdsGroup; ++j) {
        lds[j][0][ln.lane] = ~static_cast<uint32_t>(words[j]);
        lds[j][1][ln.lane] = ~static_cast<uint32_t>(words[j] >> 32);
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < kLdsGroup; ++j) {
      if (w0 + j >= g.W) break;
      const uint32_t sbits = __float_as_uint(sw[j]);
      const uint4 *row = reinterpret_cast<const uint4 *>(lds[j][half]);
#pragma unroll
      for (int q = 0; q < kPerLane / 4; ++q) {
        const uint4 h = row[q];
        const uint32_t hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t neg = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(hv[k]), bitpos, 1));
          acc[4 * q + k] = acc[4 * q + k] + __uint_as_float((neg & 0x80000000u) | sbits);   // +-s_w
        }
      }
    }
    __builtin_amdgcn_wave_barrier();   // the group's halves are read before the next group's are written
  }
  const float wf = static_cast<float>(g.W);
  const float inv_w = 1.0f / wf;   // exact when W is a power of two
  float *es = a.err_s + ln.base + ln.lane;
  // kS2/kS2Update: this step's server scale; kSResid: the previous step's
  const float ss = (kMode == kS2 || kMode == kS2Update || kMode == kSResid)
                       ? a.scale_s[g.tile_piece[blockIdx.x]] : 0.0f;
  float z[kPerLane];
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    const bool ok = in_tile<kFull>(tl, ln, c);
    const float stored = ok ? es[64 * c] : 0.0f;
    const float e_old = (kMode == kSResid) ? onebit_error(stored, ss) : stored;
    // for W = 2^k, acc * 2^-k is the correctly rounded quotient, as the division is
    const float y = kPow2 ? acc[c] * inv_w : acc[c] / wf;
    z[c] = ok ? y + e_old : 0.0f;
  }
  if (kMode == kS1) {
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) dd_accumulate(hi, lo, z[c]);
    park_partial(sink, 0, ln.wave, hi, lo);
    flush_partials(sink, g.W, 1);
    return;
  }
  LaneWords word;
  if (kMode == kSResidFirst || kMode == kSResid) {
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const bool ok = in_tile<kFull>(tl, ln, c);
      const uint64_t bal = __ballot(ok && z[c] >= 0.0f);
      word.put(bal, c);
      dd_accumulate(hi, lo, z[c]);
      if (ok) es[64 * c] = z[c];
    }
    if (ln.lane < ln.nwords) a.packed_s[(ln.base >> 6) + ln.lane] = word.get();
    park_partial(sink, 0, ln.wave, hi, lo);
    flush_partials(sink, g.W, 1);
    return;
  }
  float vv[kPerLane], pv[kPerLane];
  if (kMode == kS2Update) {
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const bool ok = in_tile<kFull>(tl, ln, c);
      vv[c] = ok ? __builtin_nontemporal_load(&a.v[ln.base + 64 * c + ln.lane]) : 0.0f;
      pv[c] = ok ? a.params[ln.base + 64 * c + ln.lane] : 0.0f;
    }
  }
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    const bool ok = in_tile<kFull>(tl, ln, c);
    const bool bit = z[c] >= 0.0f;
    const uint64_t bal = __ballot(ok && bit);
    word.put(bal, c);
    if (ok) {
      es[64 * c] = bit ? z[c] - ss : z[c] + ss;
      if (kMode == kS2Update) {
        const float mv = bit ? ss : -ss;
        const float d = __builtin_sqrtf(vv[c]) + a.eps;
        const float u = mv / d;
        a.m[ln.base + 64 * c + ln.lane] = mv;
        a.params[ln.base + 64 * c + ln.lane] = pv[c] - a.lr * u;
      }
    }
  }
  if (ln.lane < ln.nwords) a.packed_s[(ln.base >> 6) + ln.lane] = word.get();
}

template <int kMode, bool kPow2>
__global__ __launch_bounds__(kBlock) void server_kernel(Geometry g, ServerArgs a) {
  __shared__ double2 red[1][kWaves];
  __shared__ __align__(16) uint32_t lds[kWaves][kLdsGroup][2][kPerLane];   // 8 KB: 2 KB per wavefront
  const PartialSink sink{red, a.partials, g.num_tiles, static_cast<int>(blockIdx.x)};
  uint32_t (*mine)[2][kPerLane] = lds[threadIdx.x >> 6];
  const Tile tl = g.tiles[blockIdx.x];
  if (tl.len == kTile)
    server_tile<kMode, true, kPow2>(tl, g, a, sink, mine);
  else
    server_tile<kMode, false, kPow2>(tl, g, a, sink, mine);
}

// ---------------------------------------------------------------------------
// update from a server message: m = s_s*sign (stored if kStoreM),
// p <- p - lr * (m / (sqrt(v) + eps))
// ---------------------------------------------------------------------------
// The update in chunks of kUpdChunk elements, one workgroup each (grid-stride
// past the device's grid limit): lane l of wavefront v owns element
// kUpdChunk/kWaves * v + 64*c + l of the chunk.  A single read-modify-write
// stream streams faster in small workgroups taken in address order: on
// MI355X an in-place add ran at ~5.9 TB/s with one workgroup per 4 KB piece
// against ~5.3 TB/s with one per 32 KB.
constexpr int kUpdChunk = 1024;
constexpr int kUpdPerTile = kTile / kUpdChunk;
constexpr int kUpdSub = kUpdChunk / kWaves;
constexpr int kUpdPerLane = kUpdSub / 64;
static_assert(kTile % kUpdChunk == 0 && kUpdSub % 64 == 0, "update chunk shape");

template <bool kStoreM, bool kRatio, bool kFull>
__device__ __forceinline__ void update_chunk(const Tile &tl, int tile, int q, const Geometry &g,
                                             const UpdateArgs &a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub0 = q * kUpdChunk + wave * kUpdSub;   // first element of this wavefront in the tile
  const int64_t base = tl.start + sub0;
  const int rem = tl.len - sub0;
  const int nwords = kFull ? kUpdPerLane : (rem <= 0 ? 0 : (rem >= kUpdSub ? kUpdPerLane : (rem + 63) / 64));
  auto ok = [&](int c) { return kFull || sub0 + 64 * c + lane < tl.len; };
  const float ss = a.scale_s[g.tile_piece[tile]];
  const float r = kRatio ? a.ratio[tl.tensor] : 1.0f;
  const uint64_t words = lane < nwords ? a.packed_s[(base >> 6) + lane] : 0ull;
  float vv[kUpdPerLane], pv[kUpdPerLane];
#pragma unroll
  for (int c = 0; c < kUpdPerLane; ++c) {
    vv[c] = ok(c) ? __builtin_nontemporal_load(&a.v[base + 64 * c + lane]) : 0.0f;
    pv[c] = ok(c) ? a.params[base + 64 * c + lane] : 0.0f;
  }
#pragma unroll
  for (int c = 0; c < kUpdPerLane; ++c) {
    const float mv = signed_scale(words, c, ss);  // every lane takes part in the broadcast
    if (!ok(c)) continue;
    const int64_t i = base + 64 * c + lane;
    const float d = __builtin_sqrtf(vv[c]) + a.eps;
    float u = mv / d;
    if (kStoreM) a.m[i] = mv;
    if (kRatio) {
      if (a.wd > 0.0f) u = u + a.wd * pv[c];
      a.params[i] = pv[c] - a.lr * (r * u);
    } else {
      a.params[i] = pv[c] - a.lr * u;
    }
  }
}

template <bool kStoreM, bool kRatio>
__global__ __launch_bounds__(kBlock) void update_kernel(Geometry g, UpdateArgs a) {
  const int64_t chunks = static_cast<int64_t>(g.num_tiles) * kUpdPerTile;
  for (int64_t b = blockIdx.x; b < chunks; b += gridDim.x) {   // uniform over the workgroup
    const int tile = static_cast<int>(b / kUpdPerTile);
    const int q = static_cast<int>(b % kUpdPerTile);
    const Tile tl = g.tiles[tile];
    const int rem = tl.len - q * kUpdChunk;
    if (rem <= 0) continue;   // past the tile's end
    if (rem >= kUpdChunk)
      update_chunk<kStoreM, kRatio, true>(tl, tile, q, g, a);
    else
      update_chunk<kStoreM, kRatio, false>(tl, tile, q, g, a);
  }
}

// ---------------------------------------------------------------------------
// trust ratio: per tile, compensated sums of p^2 and u^2 (partial rows 0, 1);
// per tensor, r = fp32(sqrt(sum p^2) / sqrt(sum u^2)), 1 when either is 0
// ---------------------------------------------------------------------------
template <bool kFull>
__device__ __forceinline__ void trust_norms_tile(const Tile &tl, const Geometry &g,
                                                 const UpdateArgs &a, const PartialSink &sink) {
  const Lanes ln = lanes_of<kFull>(tl);
  const float ss = a.scale_s[g.tile_piece[blockIdx.x]];
  const uint64_t words = load_words<kFull>(a.packed_s + (ln.base >> 6), ln);
  double ph = 0.0, pl = 0.0, uh = 0.0, ul = 0.0;
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    const float mv = signed_scale(words, c, ss);
    const bool ok = in_tile<kFull>(tl, ln, c);
    const float vv = ok ? a.v[ln.base + 64 * c + ln.lane] : 0.0f;
    const float pv = ok ? a.params[ln.base + 64 * c + ln.lane] : 0.0f;
    const float d = __builtin_sqrtf(vv) + a.eps;
    float u = mv / d;
    if (a.wd > 0.0f) u = u + a.wd * pv;
    dd_accumulate(ph, pl, pv);
    dd_accumulate(uh, ul, ok ? u : 0.0f);
  }
  park_partial(sink, 0, ln.wave, ph, pl);
  park_partial(sink, 1, ln.wave, uh, ul);
  flush_partials(sink, 0, 2);
}

__global__ __launch_bounds__(kBlock) void trust_norms_kernel(Geometry g, UpdateArgs a,
                                                             double2 *partials) {
  __shared__ double2 red[2][kWaves];
  const PartialSink sink{red, partials, g.num_tiles, static_cast<int>(blockIdx.x)};
  const Tile tl = g.tiles[blockIdx.x];
  if (tl.len == kTile)
    trust_norms_tile<true>(tl, g, a, sink);
  else
    trust_norms_tile<false>(tl, g, a, sink);
}

__global__ __launch_bounds__(kBlock) void trust_ratio_kernel(Geometry g,
                                                             const double2 *__restrict__ partials,
                                                             float *__restrict__ ratio) {
  const int lane = threadIdx.x & 63;
  const int t = static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (t >= g.T) return;  // whole wavefront leaves together
  double sum[2];
#pragma unroll
  for (int row = 0; row < 2; ++row) {
    const double2 *p = partials + static_cast<size_t>(row) * g.num_tiles;
    // eight independent chains per lane, their loads issued together, then
    // folded in a fixed order
    constexpr int kChains = 8;
    double ch[kChains], cl[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) ch[k] = cl[k] = 0.0;
    const int end = g.tile_begin[t + 1];
    for (int i0 = g.tile_begin[t] + lane; i0 < end; i0 += 64 * kChains) {
      double2 q[kChains];
#pragma unroll
      for (int k = 0; k < kChains; ++k) q[k] = i0 + 64 * k < end ? p[i0 + 64 * k] : make_double2(0.0, 0.0);
#pragma unroll
      for (int k = 0; k < kChains; ++k) dd_add(ch[k], cl[k], q[k].x, q[k].y);
    }
    double hi = ch[0], lo = cl[0];
#pragma unroll
    for (int k = 1; k < kChains; ++k) dd_add(hi, lo, ch[k], cl[k]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const double oh = __shfl_xor(hi, d);
      const double ol = __shfl_xor(lo, d);
      dd_add(hi, lo, oh, ol);
    }
    sum[row] = hi + lo;
  }
  if (lane == 0) {
    ratio[t] = (sum[0] == 0.0 || sum[1] == 0.0)
                   ? 1.0f
                   : static_cast<float>(__builtin_sqrt(sum[0]) / __builtin_sqrt(sum[1]));
  }
}

// ---------------------------------------------------------------------------
// materialize: residual form -> errors and momentum
//   e_w = x_w - s_w*sign(x_w), e_s = z - s_s*sign(z), m = s_s*sign(z).
// Outputs may alias the inputs (each element is read, then written, by one lane).
// ---------------------------------------------------------------------------
template <bool kFull>
__device__ __forceinline__ void materialize_tile(const Tile &tl, const Geometry &g,
                                                 const MaterializeArgs &a) {
  const Lanes ln = lanes_of<kFull>(tl);
  const int t = tl.tensor;
  for (int w = 0; w < g.W; ++w) {
    const float s = a.scale_w[static_cast<size_t>(w) * g.T + t];
    const size_t off = static_cast<size_t>(w) * g.N + ln.base + ln.lane;
#pragma unroll
    for (int c = 0; c < kPerLane; ++c)
      if (in_tile<kFull>(tl, ln, c)) a.e_w[off + 64 * c] = onebit_error(a.x_w[off + 64 * c], s);
  }
  const float ss = a.scale_s[g.tile_piece[blockIdx.x]];
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    if (!in_tile<kFull>(tl, ln, c)) continue;
    const int64_t i = ln.base + 64 * c + ln.lane;
    const float z = a.z[i];
    a.e_s[i] = onebit_error(z, ss);
    a.m[i] = z >= 0.0f ? ss : -ss;
  }
}

__global__ __launch_bounds__(kBlock) void materialize_kernel(Geometry g, MaterializeArgs a) {
  const Tile tl = g.tiles[blockIdx.x];
  if (tl.len == kTile)
    materialize_tile<true>(tl, g, a);
  else
    materialize_tile<false>(tl, g, a);
}

// ---------------------------------------------------------------------------
// warmup phase: uncompressed Adam on the workers' average gradient
//   gbar = (ascending sum over w of g_w) / W
//   m = c1*m + c2*gbar;  v = b2*v + cb2*(gbar*gbar);  p -= lr * (m / (sqrt(v) + eps))
// ---------------------------------------------------------------------------
// The warmup step in the update's chunks (one workgroup per kUpdChunk
// elements, grid-stride past the grid limit), the workers' gradients loaded
// in groups of kGroup and added in ascending worker order.
template <typename G, bool kFull, bool kPow2>
__device__ __forceinline__ void warmup_chunk(const Tile &tl, int q, const Geometry &g, const WarmupArgs &a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub0 = q * kUpdChunk + wave * kUpdSub;
  const int64_t base = tl.start + sub0;
  auto ok = [&](int c) { return kFull || sub0 + 64 * c + lane < tl.len; };
  const G *grads = static_cast<const G *>(a.grads) + base + lane;
  const float wf = static_cast<float>(g.W);
  const float inv_w = 1.0f / wf;
  // fp32 gradients: groups of 8 workers' loads in flight (7-11% faster than
  // one worker at a time); bf16 gradients: one worker at a time (grouped
  // two-byte loads were 1.7x slower at the GPT list, measured)
  constexpr int kGroup = sizeof(G) == 2 ? 1 : 8;
  float acc[kUpdPerLane];
#pragma unroll
  for (int j = 0; j < kUpdPerLane; ++j) acc[j] = 0.0f;
  for (int w0 = 0; w0 < g.W; w0 += kGroup) {
    float x[kGroup][kUpdPerLane];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const G *gw = grads + static_cast<size_t>(w0 + k) * g.N;
#pragma unroll
      for (int j = 0; j < kUpdPerLane; ++j) x[k][j] = (w0 + k < g.W && ok(j)) ? grad_value(gw + 64 * j) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      if (w0 + k >= g.W) break;
#pragma unroll
      for (int j = 0; j < kUpdPerLane; ++j) acc[j] = acc[j] + x[k][j];
    }
  }
#pragma unroll
  for (int j = 0; j < kUpdPerLane; ++j) {
    if (!ok(j)) continue;
    const int64_t i = base + 64 * j + lane;
    const float gbar = kPow2 ? acc[j] * inv_w : acc[j] / wf;
    const float m = a.c1 * a.m[i] + a.c2 * gbar;
    const float v = a.b2 * a.v[i] + a.cb2 * (gbar * gbar);
    const float d = __builtin_sqrtf(v) + a.eps;
    const float u = m / d;
    a.m[i] = m;
    a.v[i] = v;
    a.params[i] = a.params[i] - a.lr * u;
  }
}

template <typename G, bool kPow2>
__global__ __launch_bounds__(kBlock) void warmup_kernel(Geometry g, WarmupArgs a) {
  const int64_t chunks = static_cast<int64_t>(g.num_tiles) * kUpdPerTile;
  for (int64_t b = blockIdx.x; b < chunks; b += gridDim.x) {
    const int tile = static_cast<int>(b / kUpdPerTile);
    const int q = static_cast<int>(b % kUpdPerTile);
    const Tile tl = g.tiles[tile];
    const int rem = tl.len - q * kUpdChunk;
    if (rem <= 0) continue;
    if (rem >= kUpdChunk)
      warmup_chunk<G, true, kPow2>(tl, q, g, a);
    else
      warmup_chunk<G, false, kPow2>(tl, q, g, a);
  }
}

// Zero the worker and server errors (tensor ranges only; padding untouched).
template <bool kFull>
__device__ __forceinline__ void zero_errors_tile(const Tile &tl, const Geometry &g, float *err_w,
                                                 float *err_s) {
  const Lanes ln = lanes_of<kFull>(tl);
  for (int w = 0; w <= g.W; ++w) {
    float *row = (w < g.W ? err_w + static_cast<size_t>(w) * g.N : err_s) + ln.base + ln.lane;
#pragma unroll
    for (int c = 0; c < kPerLane; ++c)
      if (in_tile<kFull>(tl, ln, c)) row[64 * c] = 0.0f;
  }
}

__global__ __launch_bounds__(kBlock) void zero_errors_kernel(Geometry g, float *err_w, float *err_s) {
  const Tile tl = g.tiles[blockIdx.x];
  if (tl.len == kTile)
    zero_errors_tile<true>(tl, g, err_w, err_s);
  else
    zero_errors_tile<false>(tl, g, err_w, err_s);
}

template <typename G>
void launch_worker_mode(int mode, const Geometry &g, const WorkerArgs &a, hipStream_t s) {
  const dim3 block(kBlock);
  const int64_t chunks = static_cast<int64_t>(g.num_tiles) * kChunksPerTile;   // at most kMaxGrid
  if (mode == kResid) {
    const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(a.w1 - a.w0));
    hipLaunchKernelGGL((worker_chunk_kernel<G, kResid>), grid, block, 0, s, g, a);
    return;
  }
  if (mode == kResidFirst || (mode == kPass2 && sizeof(G) == 4)) {
    // worker-fastest, one launch per run of workers whose grid fits kMaxGrid
    worker_runs(a.w0, a.w1, chunks, kMaxGrid, [&](int b0, int b1) {
      WorkerArgs b = a;
      b.w0 = b0;
      b.w1 = b1;
      const dim3 grid(static_cast<unsigned>(chunks * (b1 - b0)));
      if (mode == kResidFirst)
        hipLaunchKernelGGL((worker_chunk_kernel<G, kResidFirst>), grid, block, 0, s, g, b);
      else
        hipLaunchKernelGGL((worker_chunk_kernel<G, kPass2Chunk>), grid, block, 0, s, g, b);
    });
    return;
  }
  const int groups = (a.w1 - a.w0 + a.wgroup - 1) / a.wgroup;
  const dim3 grid(static_cast<unsigned>(g.num_tiles) * static_cast<unsigned>(groups));
  if (mode == kPass1)
    hipLaunchKernelGGL((worker_kernel<G, kPass1>), grid, block, 0, s, g, a);
  else
    hipLaunchKernelGGL((worker_kernel<G, kPass2>), grid, block, 0, s, g, a);
}

// Scratch of the no-allocation step (ob_step_residual_noalloc): every GPU the
// library runs on holds one copy until the process ends.  In host code its
// name is only a handle for the symbol lookup below; kernels receive the
// device address that lookup returns.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

}  // namespace

hipError_t static_scratch_address(void **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *address[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (address[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    address[dev] = p;
  }
  *out = address[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
void launch_worker(WorkerPass pass, const Geometry &g, bool bf16, const WorkerArgs &a, hipStream_t s) {
  const int mode = pass == WorkerPass::kStrictSigns ? kPass1
                 : pass == WorkerPass::kStrictErrors ? kPass2
                 : pass == WorkerPass::kResidualFirst ? kResidFirst : kResid;
  if (bf16)
    launch_worker_mode<uint16_t>(mode, g, a, s);
  else
    launch_worker_mode<float>(mode, g, a, s);
}

void launch_scale_finalize(const Geometry &g, const double2 *partials, int64_t cols, int per, int row0,
                           int nrows, const int32_t *begin, const int64_t *numel, int count, float *out,
                           int64_t max_item_partials, hipStream_t s) {
  const int64_t items = static_cast<int64_t>(nrows) * count;
  const dim3 block(kBlock);
  if (max_item_partials >= kWideFinalize) {
    hipLaunchKernelGGL((scale_finalize<kWaves>), dim3(static_cast<unsigned>(items)), block, 0, s, g, partials,
                       cols, per, row0, nrows, begin, numel, count, out);
  } else {
    hipLaunchKernelGGL((scale_finalize<1>), dim3(static_cast<unsigned>((items + kWaves - 1) / kWaves)), block,
                       0, s, g, partials, cols, per, row0, nrows, begin, numel, count, out);
  }
}

template <bool kPow2>
void launch_server_w(ServerPass pass, const Geometry &g, const ServerArgs &a, hipStream_t s) {
  const dim3 grid(g.num_tiles), block(kBlock);
  switch (pass) {
    case ServerPass::kStrictSums:
      hipLaunchKernelGGL((server_kernel<kS1, kPow2>), grid, block, 0, s, g, a); break;
    case ServerPass::kStrictErrors:
      hipLaunchKernelGGL((server_kernel<kS2, kPow2>), grid, block, 0, s, g, a); break;
    case ServerPass::kStrictErrorsUpdate:
      hipLaunchKernelGGL((server_kernel<kS2Update, kPow2>), grid, block, 0, s, g, a); break;
    case ServerPass::kResidualFirst:
      hipLaunchKernelGGL((server_kernel<kSResidFirst, kPow2>), grid, block, 0, s, g, a); break;
    case ServerPass::kResidual:
      hipLaunchKernelGGL((server_kernel<kSResid, kPow2>), grid, block, 0, s, g, a); break;
  }
}

void launch_server(ServerPass pass, const Geometry &g, const ServerArgs &a, hipStream_t s) {
  if ((g.W & (g.W - 1)) == 0)
    launch_server_w<true>(pass, g, a, s);
  else
    launch_server_w<false>(pass, g, a, s);
}

void launch_update(bool store_m, bool with_ratio, const Geometry &g, const UpdateArgs &a,
                   hipStream_t s) {
  const int64_t chunks = static_cast<int64_t>(g.num_tiles) * kUpdPerTile;
  const dim3 grid(static_cast<unsigned>(chunks < kMaxGrid ? chunks : kMaxGrid)), block(kBlock);
  if (store_m && with_ratio)
    hipLaunchKernelGGL((update_kernel<true, true>), grid, block, 0, s, g, a);
  else if (store_m)
    hipLaunchKernelGGL((update_kernel<true, false>), grid, block, 0, s, g, a);
  else if (with_ratio)
    hipLaunchKernelGGL((update_kernel<false, true>), grid, block, 0, s, g, a);
  else
    hipLaunchKernelGGL((update_kernel<false, false>), grid, block, 0, s, g, a);
}

void launch_trust_norms(const Geometry &g, const UpdateArgs &a, double2 *partials, hipStream_t s) {
  hipLaunchKernelGGL(trust_norms_kernel, dim3(g.num_tiles), dim3(kBlock), 0, s, g, a, partials);
}

void launch_trust_ratio(const Geometry &g, const double2 *partials, float *ratio, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((g.T + kWaves - 1) / kWaves)), block(kBlock);
  hipLaunchKernelGGL(trust_ratio_kernel, grid, block, 0, s, g, partials, ratio);
}

void launch_materialize(const Geometry &g, const MaterializeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(materialize_kernel, dim3(g.num_tiles), dim3(kBlock), 0, s, g, a);
}

void launch_warmup(const Geometry &g, bool bf16, const WarmupArgs &a, hipStream_t s) {
  const int64_t chunks = static_cast<int64_t>(g.num_tiles) * kUpdPerTile;
  const dim3 grid(static_cast<unsigned>(chunks < kMaxGrid ? chunks : kMaxGrid)), block(kBlock);
  const bool pow2 = (g.W & (g.W - 1)) == 0;
  if (bf16) {
    if (pow2) hipLaunchKernelGGL((warmup_kernel<uint16_t, true>), grid, block, 0, s, g, a);
    else hipLaunchKernelGGL((warmup_kernel<uint16_t, false>), grid, block, 0, s, g, a);
  } else {
    if (pow2) hipLaunchKernelGGL((warmup_kernel<float, true>), grid, block, 0, s, g, a);
    else hipLaunchKernelGGL((warmup_kernel<float, false>), grid, block, 0, s, g, a);
  }
}

void launch_zero_errors(const Geometry &g, float *err_w, float *err_s, hipStream_t s) {
  hipLaunchKernelGGL(zero_errors_kernel, dim3(g.num_tiles), dim3(kBlock), 0, s, g, err_w, err_s);
}

}  // namespace ob
