// HIP kernels (gfx950) of the cyclic local top-k (CLT-k) codec: the
// commutative compressor of the review of "ScaleCom: Scalable Sparsified
// Gradient Compression ..." (Proposed method: cyclic local top-k aligns the
// workers' sparsity so that the exchange is an all-reduce).
//
// Per tensor, the leader worker (step mod W) ranks |x_leader| = |mem + g|
// and every worker sends its x at the leader's k largest positions.  The
// selection is exact: the k-th largest key (the bit pattern of |x|, which
// orders non-negative floats) is found by a radix select with 11, 11 and
// 9-bit digits (LDS histograms per tile, per 64 tiles or per wavefront,
// added into per-tensor histograms).
// Pass 1 reads the leader's memory and gradient once: the first digit's
// histogram, and for a window of first-digit bins around the previous
// exchange's threshold, per tile, a bit mask of the keys above the window and
// the keys inside it (the candidates) with their positions.  If the
// threshold's first digit falls outside the window (or at the first
// exchange), a fallback pass rebuilds that data for the tensor.  The later
// digits and the per-tile counts read only the candidates.  Ties at the
// threshold go to the lowest indices; per-tensor scans give each tile its
// first position.  Then one dense pass over all workers rebuilds each tile's
// selection from the mask and the candidates, writes the ascending index
// list, gathers the messages and updates the memories, and the server
// averages the W messages in ascending worker order.
//
// The element mapping is the one of kernels.hip: a workgroup of 4
// wavefronts owns a tile of up to kTile elements of one tensor, lane l of
// wavefront v owns element 2048 v + 64 c + l, so ballots over one c are
// natural-order 64-bit words.  Every per-tile kernel has a body for full
// tiles (no bounds tests: loads from one base address with immediate
// offsets, all issued before the first use) and one for a tensor's last,
// partial tile (guarded loads).
#include "internal.h"

#pragma clang fp contract(off)

namespace ob {
namespace {

// A gradient element (bf16: the upper half of the same fp32, exact).  Each
// pass reads a gradient row once: non-temporal loads (the gather 1-3%
// faster on MI355X, bit-identical).
template <typename G>
__device__ __forceinline__ float grad_at(const G *p);
template <>
__device__ __forceinline__ float grad_at<float>(const float *p) { return __builtin_nontemporal_load(p); }
template <>
__device__ __forceinline__ float grad_at<uint16_t>(const uint16_t *p) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_nontemporal_load(p)) << 16);
}

struct TileLanes {
  int lane, wave, sub0, nwords;
  int64_t base;
};

__device__ __forceinline__ TileLanes tile_lanes(const Tile &tl) {
  TileLanes r;
  r.lane = threadIdx.x & 63;
  r.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  r.sub0 = r.wave * kSub;
  r.base = tl.start + r.sub0;
  const int rem = tl.len - r.sub0;
  r.nwords = rem <= 0 ? 0 : (rem >= kSub ? kPerLane : (rem + 63) / 64);
  return r;
}

// Whether lane slot c holds an element of the tile.
template <bool kFull>
__device__ __forceinline__ bool slot_ok(const Tile &tl, const TileLanes &ln, int c) {
  return kFull || ln.sub0 + 64 * c + ln.lane < tl.len;
}

// Ranking key of an element: the bit pattern of |mem + g|.  The select stage
// reads the leader's rows once (non-temporal; the gather rewrites the memory
// rows much later): the stage 2-9% faster on MI355X.
template <typename G>
__device__ __forceinline__ uint32_t key_of(const float *mem, const G *grads, int64_t i) {
  return __float_as_uint(__builtin_nontemporal_load(mem + i) + grad_at(grads + i)) & 0x7fffffffu;
}

// Lane c's value of a 64-bit register, as a wave-uniform (scalar) value.
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int c) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), c);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), c);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------------------
// radix select over the 31-bit keys: digits of 11, 11 and 9 bits
//
// Pass 1 reads the leader's memory and gradient once.  Besides the histogram
// of the top 11 bits (digit 0) it prepares, per tile, the input of every
// later step for a window of digit-0 bins around the bin the threshold fell
// in at the previous exchange: a bit per element for keys above the window,
// their count, and the keys inside the window with their positions,
// compacted (the candidates).  Once digit 0 of the threshold is known, a
// tensor whose bin lies in the window needs nothing more from the dense
// data; for the others (and at the first exchange) a fallback pass rebuilds
// the same per-tile data for the window [b0, b0].  Candidates from other
// window bins never tie with the threshold: they compare above or below it.
// ---------------------------------------------------------------------------
constexpr int kMaxBins = 2048;
constexpr int kShift0 = 20, kShift1 = 9, kShift2 = 0;
constexpr uint32_t kNoBin = 0xffffffffu;     // no prediction yet
constexpr uint32_t kWindowBelow = 1, kWindowAbove = 3;   // the threshold's bin drifts upward

// Grid-stride launches (grid capped at kStrideBlocks) for the two kernels
// whose size is not a tile count.
constexpr unsigned kStrideBlocks = 65535;

__global__ __launch_bounds__(kBlock) void topk_reset(Geometry g, TopkArgs a) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
       i < static_cast<int64_t>(g.T) * kMaxBins; i += stride) {
    a.hist[i] = 0u;
    if (i < g.T) {
      a.prefix[i] = 0u;
      a.krem[i] = static_cast<uint32_t>(a.k_off[i + 1] - a.k_off[i]);
    }
  }
}

// Digit-0 window [lo, hi] of tensor t for this exchange's pass 1; lo > hi
// when there is no prediction.
struct Window {
  uint32_t lo, hi;
};

__device__ __forceinline__ Window predicted_window(const TopkArgs &a, int t) {
  const uint32_t b = a.pred[t];
  if (b == kNoBin) return Window{1u, 0u};
  return Window{b >= kWindowBelow ? b - kWindowBelow : 0u,
                b + kWindowAbove < kMaxBins ? b + kWindowAbove : kMaxBins - 1u};
}

// The tile's keys, from the leader's memory and gradient (0 past the end).
template <typename G, bool kFull>
__device__ __forceinline__ void leader_keys(const Geometry &g, const TopkArgs &a, const Tile &tl,
                                            const TileLanes &ln, uint32_t (&key)[kPerLane]) {
  const size_t row = static_cast<size_t>(a.leader) * g.N + ln.base + ln.lane;
  const float *mem = a.memory + row;
  const G *grads = static_cast<const G *>(a.grads) + row;
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {   // all loads first
    key[c] = 0u;
    if (slot_ok<kFull>(tl, ln, c)) key[c] = key_of(mem, grads, 64 * c);
  }
}

// Per tile, for the digit-0 window [w.lo, w.hi]: the bit mask of keys above
// it (a.above), their count (tile_gt), and the keys inside it with their
// positions, compacted in ascending position order (cand, cand_pos, tile_m).
// Workgroup-uniform call; wcnt holds 2 * kWaves counters (a caller that
// writes them again must pass a barrier first).
template <bool kFull>
__device__ __forceinline__ void window_tile(const TopkArgs &a, const Tile &tl, int tile,
                                            const TileLanes &ln, const uint32_t (&key)[kPerLane],
                                            Window w, uint32_t *wcnt) {
  uint32_t nm = 0, ngt = 0;
  LaneWords gtw;   // lane c: word c of the above-window mask
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    const bool ok = slot_ok<kFull>(tl, ln, c);
    const uint32_t d0 = key[c] >> kShift0;
    const uint64_t bg = __ballot(ok && d0 > w.hi);
    gtw.put(bg, c);
    nm += __popcll(__ballot(ok && d0 >= w.lo && d0 <= w.hi));
    ngt += __popcll(bg);
  }
  if (ln.lane < ln.nwords) a.above[(ln.base >> 6) + ln.lane] = gtw.get();
  if (ln.lane == 0) {
    wcnt[ln.wave] = nm;
    wcnt[kWaves + ln.wave] = ngt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0, gt = 0;
    for (int v = 0; v < kWaves; ++v) {
      m += wcnt[v];
      gt += wcnt[kWaves + v];
    }
    a.tile_m[tile] = m;
    a.tile_gt[tile] = gt;   // completed by topk_tile_counts
    a.tile_eq[tile] = 0u;
  }
  uint32_t at = 0;   // this wavefront's first slot in the tile's candidate list
  for (int v = 0; v < ln.wave; ++v) at += wcnt[v];
  uint32_t *cand = a.cand + tl.start;
  uint16_t *cand_pos = a.cand_pos + tl.start;
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    const uint32_t d0 = key[c] >> kShift0;
    const bool match = slot_ok<kFull>(tl, ln, c) && d0 >= w.lo && d0 <= w.hi;
    const uint64_t bm = __ballot(match);
    if (match) {
      // in ascending position order: wavefronts, then c, then lanes
      const uint32_t slot = at + __popcll(bm & lanemask_lt(ln.lane));
      cand[slot] = key[c];
      cand_pos[slot] = static_cast<uint16_t>(ln.sub0 + 64 * c + ln.lane);
    }
    at += __popcll(bm);
  }
}

// Pass 1: digit-0 histogram of the leader's keys, and the per-tile data for
// the predicted window (none at the first exchange).
template <typename G>
__global__ __launch_bounds__(kBlock) void topk_pass1(Geometry g, TopkArgs a) {
  __shared__ uint32_t h[kMaxBins];
  __shared__ uint32_t wcnt[2 * kWaves];
  for (int i = threadIdx.x; i < kMaxBins; i += kBlock) h[i] = 0u;
  __syncthreads();
  const int tile = static_cast<int>(blockIdx.x);
  const Tile tl = g.tiles[tile];
  const TileLanes ln = tile_lanes(tl);
  const Window w = predicted_window(a, tl.tensor);
  uint32_t key[kPerLane];
  if (tl.len == kTile)
    leader_keys<G, true>(g, a, tl, ln, key);
  else
    leader_keys<G, false>(g, a, tl, ln, key);
#pragma unroll
  for (int c = 0; c < kPerLane; ++c)
    if (ln.sub0 + 64 * c + ln.lane < tl.len) atomicAdd(&h[key[c] >> kShift0], 1u);
  if (w.lo <= w.hi) {   // uniform over the workgroup
    if (tl.len == kTile)
      window_tile<true>(a, tl, tile, ln, key, w, wcnt);
    else
      window_tile<false>(a, tl, tile, ln, key, w, wcnt);
  }
  __syncthreads();
  uint32_t *out = a.hist + static_cast<size_t>(tl.tensor) * kMaxBins;
  for (int i = threadIdx.x; i < kMaxBins; i += kBlock)
    if (h[i]) atomicAdd(&out[i], h[i]);
}

// Fallback: for the tensors whose digit 0 missed the window (topk_pick at
// digit 0 sets a.miss), the per-tile data for the window [b0, b0], from the
// leader's memory and gradient again.  A workgroup checks kRefillTiles tiles
// at once and refills those of a missed tensor, so that an exchange without a
// miss costs only the check.
constexpr int kRefillTiles = 16;

template <typename G>
__global__ __launch_bounds__(kBlock) void topk_refill(Geometry g, TopkArgs a) {
  __shared__ uint32_t wcnt[2 * kWaves];
  __shared__ uint32_t todo_s;
  const int t0 = static_cast<int>(blockIdx.x) * kRefillTiles;
  if (threadIdx.x < 64) {   // wavefront 0: which of the tiles belong to a missed tensor
    const int tile = t0 + static_cast<int>(threadIdx.x);
    const bool need = threadIdx.x < kRefillTiles && tile < g.num_tiles &&
                      a.miss[g.tiles[tile].tensor] != 0u;
    const uint64_t b = __ballot(need);
    if (threadIdx.x == 0) todo_s = static_cast<uint32_t>(b);
  }
  __syncthreads();
  for (uint32_t todo = __builtin_amdgcn_readfirstlane(todo_s); todo != 0u; todo &= todo - 1u) {
    const int tile = t0 + __builtin_ctz(todo);   // uniform over the workgroup
    const Tile tl = g.tiles[tile];
    const TileLanes ln = tile_lanes(tl);
    const uint32_t b0 = a.prefix[tl.tensor] >> kShift0;
    uint32_t key[kPerLane];
    if (tl.len == kTile) {
      leader_keys<G, true>(g, a, tl, ln, key);
      window_tile<true>(a, tl, tile, ln, key, Window{b0, b0}, wcnt);
    } else {
      leader_keys<G, false>(g, a, tl, ln, key);
      window_tile<false>(a, tl, tile, ln, key, Window{b0, b0}, wcnt);
    }
    __syncthreads();   // wcnt is read before the next tile writes it
  }
}

// ---------------------------------------------------------------------------
// kernels over the candidates only.  A tile holds a few hundred candidates,
// so each wavefront takes kWaveTiles consecutive tiles on its own (no
// workgroup barrier), keeps their counts, tensors and starts in its first
// lanes, and keeps kCandUnroll candidate loads in flight per lane.
// ---------------------------------------------------------------------------
constexpr int kCandTiles = 16;                     // tiles per workgroup
constexpr int kWaveTiles = kCandTiles / kWaves;    // tiles per wavefront
constexpr int kCandUnroll = 4;
static_assert(kWaveTiles * kWaves == kCandTiles && kWaveTiles <= 64, "tiles per wavefront");

// Orders one wavefront's LDS accesses across its lanes: the hardware runs a
// wavefront's LDS instructions in issue order; the fences keep the compiler
// from moving accesses across this point.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct WaveTile {
  uint32_t m;       // candidates in the tile (0 past the last tile)
  int32_t tensor;
  int64_t start;
};

// Lane j < kN: the wavefront's tile tw0 + j.
template <int kN>
__device__ __forceinline__ WaveTile wave_tiles(const Geometry &g, const TopkArgs &a, int tw0, int lane) {
  WaveTile r{0u, 0, 0};
  const int tile = tw0 + lane;
  if (lane < kN && tile < g.num_tiles) {
    r.m = a.tile_m[tile];
    const Tile tl = g.tiles[tile];
    r.tensor = tl.tensor;
    r.start = tl.start;
  }
  return r;
}

// Tile j of the wavefront, as wave-uniform values.
__device__ __forceinline__ WaveTile wave_tile_at(const WaveTile &w, int j) {
  WaveTile r;
  r.m = __builtin_amdgcn_readlane(w.m, j);
  r.tensor = __builtin_amdgcn_readlane(w.tensor, j);
  r.start = static_cast<int64_t>(readlane64(static_cast<uint64_t>(w.start), j));
  return r;
}

// Adds the wavefront's histogram h into out and clears it.
template <int kBins>
__device__ __forceinline__ void flush_wave_bins(uint32_t *h, uint32_t *out, int lane) {
  wave_sync();   // every count of the tensor is in
  for (int i = lane; i < kBins; i += 64) {
    const uint32_t v = h[i];
    if (v) {
      atomicAdd(&out[i], v);
      h[i] = 0u;
    }
  }
  wave_sync();   // cleared before the next tensor's counts
}

// Per-tensor histograms of (key >> kShiftD) & (2^kBits - 1) over the
// candidates whose higher bits equal the prefix found so far, one LDS
// histogram per wavefront, added to the tensor's when the wavefront's tensor
// changes and at the end.  Used for digit 2, which few candidates reach.
template <int kShiftD, int kBits>
__global__ __launch_bounds__(kBlock) void topk_hist_cand(Geometry g, TopkArgs a) {
  constexpr int kBins = 1 << kBits;
  constexpr int kHigh = kShiftD + kBits;   // bits above this digit are fixed
  __shared__ uint32_t hs[kWaves][kBins];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t *h = hs[wave];
  for (int i = lane; i < kBins; i += 64) h[i] = 0u;
  wave_sync();
  const int tw0 = static_cast<int>(blockIdx.x) * kCandTiles + wave * kWaveTiles;
  const WaveTile mine = wave_tiles<kWaveTiles>(g, a, tw0, lane);
  int cur = -1;   // tensor whose counts h holds (uniform over the wavefront)
  uint32_t want = 0u;
  for (int j = 0; j < kWaveTiles; ++j) {
    const WaveTile wt = wave_tile_at(mine, j);
    if (wt.m == 0u) continue;
    if (wt.tensor != cur) {
      if (cur >= 0) flush_wave_bins<kBins>(h, a.hist + static_cast<size_t>(cur) * kMaxBins, lane);
      cur = wt.tensor;
      want = a.prefix[cur] >> kHigh;
    }
    const uint32_t *cand = a.cand + wt.start;
    for (uint32_t j0 = 0; j0 < wt.m; j0 += 64 * kCandUnroll) {
      uint32_t key[kCandUnroll];
#pragma unroll
      for (int u = 0; u < kCandUnroll; ++u) {   // all loads first
        const uint32_t i = j0 + 64 * u + lane;
        key[u] = i < wt.m ? cand[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kCandUnroll; ++u) {
        const uint32_t i = j0 + 64 * u + lane;
        if (i < wt.m && (key[u] >> kHigh) == want) atomicAdd(&h[(key[u] >> kShiftD) & (kBins - 1)], 1u);
      }
    }
  }
  if (cur >= 0) flush_wave_bins<kBins>(h, a.hist + static_cast<size_t>(cur) * kMaxBins, lane);
}

// Digit 1: the candidates in the threshold's first-digit bin spread evenly
// over the 2048 bins, so per-wavefront histograms would add nearly one
// global atomic per candidate.  One LDS histogram per workgroup over
// kSharedTiles tiles, for the tensor of its first tile, aggregates ~4x more;
// candidates of other tensors go to their tensor's histogram directly.
constexpr int kSharedTiles = 64;
constexpr int kSharedWaveTiles = kSharedTiles / kWaves;
constexpr int kSharedUnroll = 8;
static_assert(kSharedWaveTiles * kWaves == kSharedTiles && kSharedWaveTiles <= 64, "tiles per wavefront");

template <int kShiftD, int kBits>
__global__ __launch_bounds__(kBlock) void topk_hist_shared(Geometry g, TopkArgs a) {
  constexpr int kBins = 1 << kBits;
  constexpr int kHigh = kShiftD + kBits;   // bits above this digit are fixed
  __shared__ uint32_t h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kBlock) h[i] = 0u;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = static_cast<int>(blockIdx.x) * kSharedTiles;
  const int main_t = g.tiles[t0].tensor;   // the tensor h counts for
  const uint32_t main_want = a.prefix[main_t] >> kHigh;
  const WaveTile mine = wave_tiles<kSharedWaveTiles>(g, a, t0 + wave * kSharedWaveTiles, lane);
  for (int j = 0; j < kSharedWaveTiles; ++j) {
    const WaveTile wt = wave_tile_at(mine, j);
    if (wt.m == 0u) continue;
    const bool local = wt.tensor == main_t;   // uniform over the wavefront
    const uint32_t want = local ? main_want : a.prefix[wt.tensor] >> kHigh;
    uint32_t *gh = a.hist + static_cast<size_t>(wt.tensor) * kMaxBins;
    const uint32_t *cand = a.cand + wt.start;
    for (uint32_t j0 = 0; j0 < wt.m; j0 += 64 * kSharedUnroll) {
      uint32_t key[kSharedUnroll];
#pragma unroll
      for (int u = 0; u < kSharedUnroll; ++u) {   // all loads first
        const uint32_t i = j0 + 64 * u + lane;
        key[u] = i < wt.m ? cand[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kSharedUnroll; ++u) {
        const uint32_t i = j0 + 64 * u + lane;
        if (i < wt.m && (key[u] >> kHigh) == want) {
          const uint32_t bin = (key[u] >> kShiftD) & (kBins - 1);
          if (local)
            atomicAdd(&h[bin], 1u);
          else
            atomicAdd(&gh[bin], 1u);
        }
      }
    }
  }
  __syncthreads();
  uint32_t *out = a.hist + static_cast<size_t>(main_t) * kMaxBins;
  for (int i = threadIdx.x; i < kBins; i += kBlock)
    if (h[i]) atomicAdd(&out[i], h[i]);
}

// One workgroup per tensor: the digit bin holding the krem-th largest key.
// Thread b owns bins kPer b .. kPer b + kPer - 1.  At digit 0 (kFirst) it
// also records whether the bin lies in the window pass 1 prepared (if not,
// the fallback pass rebuilds the tensor's per-tile data) and makes the bin
// the next exchange's prediction.
template <int kBits, bool kFirst>
__global__ __launch_bounds__(kBlock) void topk_pick(TopkArgs a, int shift) {
  constexpr int kBins = 1 << kBits, kPer = kBins / kBlock;
  static_assert(kPer >= 1 && kBins <= kMaxBins, "digit width");
  __shared__ uint32_t suf[kBlock + 1];
  __shared__ uint32_t krem_s;
  const int t = blockIdx.x;
  const int b = threadIdx.x;
  uint32_t *hist = a.hist + static_cast<size_t>(t) * kMaxBins;
  uint32_t cnt[kPer];
  uint32_t local = 0;
  for (int j = 0; j < kPer; ++j) {
    cnt[j] = hist[b * kPer + j];
    local += cnt[j];
  }
  suf[b] = local;
  if (b == 0) {
    suf[kBlock] = 0u;
    krem_s = a.krem[t];   // read once, before the one writer below updates it
    if (kFirst) a.miss[t] = 1u;   // overwritten below when the bin is found
  }
  __syncthreads();
  // suffix sums over threads: suf[b] = keys in the bins of threads >= b (Hillis-Steele)
  for (int d = 1; d < kBlock; d <<= 1) {
    const uint32_t add = (b + d < kBlock) ? suf[b + d] : 0u;
    __syncthreads();
    suf[b] += add;
    __syncthreads();
  }
  const uint32_t krem = krem_s;
  uint32_t above = suf[b + 1];
  if (above < krem && suf[b] >= krem) {   // exactly one thread holds the krem-th largest
    for (int j = kPer - 1; j >= 0; --j) {
      if (above + cnt[j] >= krem) {
        const uint32_t bin = static_cast<uint32_t>(b * kPer + j);
        a.prefix[t] |= bin << shift;
        a.krem[t] = krem - above;
        if (kFirst) {
          const Window w = predicted_window(a, t);
          a.miss[t] = (w.lo <= w.hi && bin >= w.lo && bin <= w.hi) ? 0u : 1u;
          a.pred[t] = bin;
        }
        break;
      }
      above += cnt[j];
    }
  }
  __syncthreads();
  for (int j = 0; j < kPer; ++j) hist[b * kPer + j] = 0u;   // ready for the next pass
}

// ---------------------------------------------------------------------------
// per-tile counts above and at the threshold, then per-tensor offsets
// ---------------------------------------------------------------------------
// Keys above the window were counted with the candidates; the candidates
// give the rest.  Wavefronts take their tiles as in topk_hist_cand.  The
// candidates above the threshold join the keys above the window in the
// tile's mask (a.above), gathered in the wavefront's own LDS words and ORed
// into the mask at the end of the tile; the ties that are taken follow in
// topk_ties, once the per-tensor scans have ranked them.
__global__ __launch_bounds__(kBlock) void topk_tile_counts(Geometry g, TopkArgs a) {
  __shared__ uint64_t bits_s[kWaves][kTile / 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint64_t *bits = bits_s[wave];
  for (int i = lane; i < kTile / 64; i += 64) bits[i] = 0ull;
  const int tw0 = static_cast<int>(blockIdx.x) * kCandTiles + wave * kWaveTiles;
  const WaveTile mine = wave_tiles<kWaveTiles>(g, a, tw0, lane);
  const uint32_t tau_l = mine.m != 0u ? a.prefix[mine.tensor] : 0u;
  for (int j = 0; j < kWaveTiles; ++j) {
    const WaveTile wt = wave_tile_at(mine, j);
    if (wt.m == 0u) continue;
    const uint32_t tau = __builtin_amdgcn_readlane(tau_l, j);
    const uint32_t *cand = a.cand + wt.start;
    const uint16_t *cand_pos = a.cand_pos + wt.start;
    uint32_t gt = 0, eq = 0;
    wave_sync();   // the words are clear
    for (uint32_t j0 = 0; j0 < wt.m; j0 += 64 * kCandUnroll) {   // uniform: ballots stay converged
      uint32_t key[kCandUnroll];
      uint16_t pos[kCandUnroll];
#pragma unroll
      for (int u = 0; u < kCandUnroll; ++u) {
        const uint32_t i = j0 + 64 * u + lane;
        key[u] = i < wt.m ? cand[i] : 0u;
        pos[u] = i < wt.m ? cand_pos[i] : uint16_t{0};
      }
#pragma unroll
      for (int u = 0; u < kCandUnroll; ++u) {
        const bool valid = j0 + 64 * u + lane < wt.m;
        const bool above = valid && key[u] > tau;
        gt += __popcll(__ballot(above));
        eq += __popcll(__ballot(valid && key[u] == tau));
        if (above) atomicOr(reinterpret_cast<unsigned long long *>(&bits[pos[u] >> 6]), 1ull << (pos[u] & 63));
      }
    }
    wave_sync();   // every bit of the tile is in
    for (int i = lane; i < kTile / 64; i += 64) {   // words past the tile's end stay 0
      const uint64_t v = bits[i];
      if (v) {
        a.above[(wt.start >> 6) + i] |= v;
        bits[i] = 0ull;
      }
    }
    if (lane == 0) {
      a.tile_gt[tw0 + j] += gt;
      a.tile_eq[tw0 + j] = eq;
    }
  }
}

// Exclusive scan of v over the workgroup's threads; total gets the sum.
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t *s, int64_t &total) {
  s[threadIdx.x] = v;
  __syncthreads();
  for (int d = 1; d < kBlock; d <<= 1) {   // inclusive (Hillis-Steele)
    const int64_t add = threadIdx.x >= static_cast<unsigned>(d) ? s[threadIdx.x - d] : 0;
    __syncthreads();
    s[threadIdx.x] += add;
    __syncthreads();
  }
  total = s[kBlock - 1];
  const int64_t incl = s[threadIdx.x];
  __syncthreads();   // s may be written again
  return incl - v;
}

// Tiles of topk_offsets per thread and round: a thread scans its run of
// consecutive tiles itself, the workgroup scans the runs' totals.
constexpr int kRun = 16;

// The number of keys at the threshold in a tile that are taken, given those
// at the threshold in earlier tiles (ties go to the lowest positions).
__device__ __forceinline__ int64_t taken_ties(int64_t r, int64_t eq_before, int64_t eq) {
  return eq_before >= r ? 0 : (r - eq_before < eq ? r - eq_before : eq);
}

// One workgroup per tensor: exclusive scans over the tensor's tiles of the
// keys at the threshold and of the selected entries.
__global__ __launch_bounds__(kBlock) void topk_offsets(Geometry g, TopkArgs a) {
  __shared__ int64_t s[kBlock];
  const int t = blockIdx.x;
  const int first = g.tile_begin[t], last = g.tile_begin[t + 1];
  const int64_t r = a.krem[t];   // keys equal to the threshold that are taken
  int64_t eq_base = 0, sel_base = a.k_off[t];
  for (int c0 = first; c0 < last; c0 += kBlock * kRun) {   // uniform over the workgroup
    const int i0 = c0 + static_cast<int>(threadIdx.x) * kRun;
    uint32_t eq[kRun], gt[kRun];
    int64_t my_eq = 0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const bool ok = i0 + j < last;
      eq[j] = ok ? a.tile_eq[i0 + j] : 0u;
      gt[j] = ok ? a.tile_gt[i0 + j] : 0u;
      my_eq += eq[j];
    }
    int64_t eq_tot, sel_tot;
    const int64_t eq0 = eq_base + block_exclusive_scan(my_eq, s, eq_tot);
    int64_t run = eq0, my_sel = 0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      my_sel += gt[j] + taken_ties(r, run, eq[j]);
      run += eq[j];
    }
    const int64_t sel0 = sel_base + block_exclusive_scan(my_sel, s, sel_tot);
    run = eq0;
    int64_t at = sel0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      if (i0 + j < last) {
        a.tile_eq_before[i0 + j] = run;
        a.tile_sel_off[i0 + j] = at;
      }
      at += gt[j] + taken_ties(r, run, eq[j]);
      run += eq[j];
    }
    eq_base += eq_tot;
    sel_base += sel_tot;
  }
}

// The ties that are taken: a key at the threshold joins the mask when its
// rank among the tensor's ties (tile_eq_before of its tile plus its count
// among the tile's earlier candidates at the threshold: candidates are in
// ascending position order) is below r.  Typically one tile per tensor holds
// any; wavefronts take their tiles as in topk_tile_counts.
__global__ __launch_bounds__(kBlock) void topk_ties(Geometry g, TopkArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tw0 = static_cast<int>(blockIdx.x) * kCandTiles + wave * kWaveTiles;
  const WaveTile mine = wave_tiles<kWaveTiles>(g, a, tw0, lane);
  int64_t take_l = 0;
  uint32_t tau_l = 0u;
  if (mine.m != 0u) {
    const int tile = tw0 + lane;
    take_l = taken_ties(a.krem[mine.tensor], a.tile_eq_before[tile], a.tile_eq[tile]);
    tau_l = a.prefix[mine.tensor];
  }
  for (int j = 0; j < kWaveTiles; ++j) {
    const WaveTile wt = wave_tile_at(mine, j);
    const int64_t take = static_cast<int64_t>(readlane64(static_cast<uint64_t>(take_l), j));
    if (wt.m == 0u || take == 0) continue;
    const uint32_t tau = __builtin_amdgcn_readlane(tau_l, j);
    const uint32_t *cand = a.cand + wt.start;
    const uint16_t *cand_pos = a.cand_pos + wt.start;
    int64_t run = 0;   // ties met so far in the tile
    for (uint32_t j0 = 0; j0 < wt.m && run < take; j0 += 64) {   // uniform
      const uint32_t i = j0 + lane;
      const bool at_tau = i < wt.m && cand[i] == tau;
      const uint64_t b = __ballot(at_tau);
      if (at_tau && run + __popcll(b & lanemask_lt(lane)) < take) {
        const uint32_t p = cand_pos[i];
        atomicOr(reinterpret_cast<unsigned long long *>(&a.above[(wt.start >> 6) + (p >> 6)]), 1ull << (p & 63));
      }
      run += __popcll(b);
    }
  }
}

// ---------------------------------------------------------------------------
// gather.  After the select stage a.above holds each tile's selection: a bit
// per element, set for the keys above the threshold and for the ties taken.
// Every worker's row is streamed once: x = memory + g, the message at the
// selected positions, the memory with them zeroed; worker 0 also writes the
// index list.  Two shapes:
//
// chunked (lists of at most kChunkedGatherTiles tiles): one workgroup per
// (chunk of kChunk elements of a tile, worker), worker-major (chunks along
// x, workers along y), lane l of wavefront v owning element kChunk/kWaves *
// v + 64 c + l of the chunk, so lane c < kChunkPerLane holds the
// wavefront's word c of the mask.  The row loads are issued first; the
// chunk's first position is tile_sel_off plus the set bits of the tile's
// earlier words, one word per thread, summed per wavefront and across them
// in LDS behind the workgroup's one barrier.  Messages are written
// directly.
//
// tiled (longer lists): workgroups are (worker group, tile), group-major as
// in the strict form's tiled worker passes; lane c of each wavefront holds word c of the
// mask and the position of its first selected entry.  A tile's selected
// entries are one contiguous run of positions in each worker's message, so
// the workgroup stages all its workers' entries in LDS and writes them with
// one coalesced pass at the end (when the run times the workers exceeds
// kStage entries they are written directly; at such densities the direct
// stores are nearly dense).
//
// Measured on MI355X side by side, bit-identical: the chunked shape takes the
// gather 10-12% faster at the BERT-Large and BERT-base lists and 3% at
// ResNet-50; at the 160k-tile GPT list it ran 20.5-20.7 ms where the tiled
// one ran 18.1-20.6.
// ---------------------------------------------------------------------------
constexpr int kStage = 4096;

struct TileSelection {
  uint64_t selw;     // lane c: word c of the wavefront's selection mask
  int64_t posw;      // lane c: position of that word's first selected entry
  int64_t first;     // position of the tile's first selected entry
  int64_t count;     // selected entries in the tile
};

// The messages and the index list are written with non-temporal stores:
// they are not read again by this exchange, and cached like the streamed
// memories they cost the gather ~5% at BERT-Large (measured).
__device__ __forceinline__ void store_nt(uint32_t *p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(float *p, float v) { __builtin_nontemporal_store(v, p); }

// Copies stage[0 .. count) to out[first + j] for first + j < k_end.
__device__ __forceinline__ void flush_stage(const uint32_t *stage, uint32_t *out, int64_t first,
                                            int64_t count, int64_t k_end) {
  __syncthreads();   // the staged entries are complete
  for (int64_t j = threadIdx.x; j < count; j += kBlock)
    if (first + j < k_end) store_nt(out + first + j, stage[j]);
  __syncthreads();   // the stage may be refilled
}

// The tile's selection from the mask: lane c of each wavefront holds word c
// of the wavefront's part and the position of its first selected entry.
// With write_index, the tile's run of the index list (positions within the
// tensor, ascending) is staged in LDS when it fits and written out.
__device__ __forceinline__ TileSelection tile_selection(const Geometry &g, const TopkArgs &a,
                                                        const Tile &tl, int tile, const TileLanes &ln,
                                                        int64_t *wcnt, uint32_t *stage, bool write_index) {
  const int t = tl.tensor;
  TileSelection sel;
  sel.selw = ln.lane < ln.nwords ? a.above[(ln.base >> 6) + ln.lane] : 0ull;
  int64_t nsel = 0;
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) nsel += __popcll(readlane64(sel.selw, c));
  if (ln.lane == 0) wcnt[ln.wave] = nsel;
  __syncthreads();
  sel.first = a.tile_sel_off[tile];
  sel.count = 0;
  int64_t pos = sel.first;
  for (int v = 0; v < kWaves; ++v) {
    if (v < ln.wave) pos += wcnt[v];
    sel.count += wcnt[v];
  }
  const int64_t tensor_start =
      tl.start - static_cast<int64_t>(tile - g.tile_begin[t]) * kTile;
  const int64_t k_end = a.k_off[t + 1];
  const bool staged = sel.count <= kStage;   // uniform over the workgroup
  sel.posw = 0;
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    const uint64_t bs = readlane64(sel.selw, c);
    if (ln.lane == c) sel.posw = pos;
    if (write_index && ((bs >> ln.lane) & 1ull)) {
      const int64_t at = pos + __popcll(bs & lanemask_lt(ln.lane));
      const int32_t local = static_cast<int32_t>(ln.base + 64 * c + ln.lane - tensor_start);
      if (staged)
        stage[at - sel.first] = static_cast<uint32_t>(local);
      else if (at < k_end)   // always true when the selection holds k_t entries
        store_nt(reinterpret_cast<uint32_t *>(a.index) + at, static_cast<uint32_t>(local));
    }
    pos += __popcll(bs);
  }
  if (write_index && staged && sel.count > 0)
    flush_stage(stage, reinterpret_cast<uint32_t *>(a.index), sel.first, sel.count, k_end);
  return sel;
}

template <typename G, bool kFull>
__device__ __forceinline__ void gather_tile(const Geometry &g, const TopkArgs &a, const Tile &tl,
                                            int tile, int w_lo, int w_hi, int64_t *wcnt, uint32_t *stage) {
  const TileLanes ln = tile_lanes(tl);
  const int64_t k_end = a.k_off[tl.tensor + 1];
  const TileSelection sel = tile_selection(g, a, tl, tile, ln, wcnt, stage, w_lo == 0);
  const int64_t staged_entries = sel.count * (w_hi - w_lo);
  const bool staged = staged_entries <= kStage;   // uniform over the workgroup
  for (int w = w_lo; w < w_hi; ++w) {
    const size_t row = static_cast<size_t>(w) * g.N + ln.base + ln.lane;
    float *mem = a.memory + row;
    const G *gw = static_cast<const G *>(a.grads) + row;
    float *vals = a.values + static_cast<size_t>(w) * a.K;
    uint32_t *wstage = stage + (w - w_lo) * sel.count;
    float x[kPerLane];
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {   // all loads first: the stores below may alias them
      x[c] = 0.0f;
      if (slot_ok<kFull>(tl, ln, c)) x[c] = mem[64 * c] + grad_at(gw + 64 * c);
    }
    // The memory first, one full-row store per slot, in a loop of its own: in
    // the same branch as the message's stores the compiler splits it into two
    // half-masked stores (0 for the selected lanes, x for the others).
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const bool mine = (readlane64(sel.selw, c) >> ln.lane) & 1ull;   // never set past the end
      if (slot_ok<kFull>(tl, ln, c)) mem[64 * c] = mine ? 0.0f : x[c];
    }
#pragma unroll
    for (int c = 0; c < kPerLane; ++c) {
      const uint64_t bs = readlane64(sel.selw, c);
      if (bs == 0) continue;   // uniform: no entry of word c is selected
      if ((bs >> ln.lane) & 1ull) {
        const int64_t at = static_cast<int64_t>(readlane64(static_cast<uint64_t>(sel.posw), c)) +
                           __popcll(bs & lanemask_lt(ln.lane));
        if (staged)
          wstage[at - sel.first] = __float_as_uint(x[c]);
        else if (at < k_end)   // always true when the selection holds k_t entries
          store_nt(vals + at, x[c]);
      }
    }
  }
  if (staged && staged_entries > 0) {
    __syncthreads();   // every worker's entries are staged
    for (int64_t e = threadIdx.x; e < staged_entries; e += kBlock) {
      const int64_t wi = e / sel.count, j = e - wi * sel.count;
      if (sel.first + j < k_end)
        store_nt(a.values + static_cast<size_t>(w_lo + wi) * a.K + sel.first + j, __uint_as_float(stage[e]));
    }
  }
}

template <typename G>
__global__ __launch_bounds__(kBlock) void topk_gather(Geometry g, TopkArgs a) {
  __shared__ int64_t wcnt[kWaves];
  __shared__ uint32_t stage[kStage];
  const int tile = static_cast<int>(blockIdx.x % static_cast<unsigned>(g.num_tiles));
  const int grp = static_cast<int>(blockIdx.x / static_cast<unsigned>(g.num_tiles));
  const int w_lo = grp * a.wgroup;
  const int w_hi = min(g.W, w_lo + a.wgroup);
  const Tile tl = g.tiles[tile];
  if (tl.len == kTile)
    gather_tile<G, true>(g, a, tl, tile, w_lo, w_hi, wcnt, stage);
  else
    gather_tile<G, false>(g, a, tl, tile, w_lo, w_hi, wcnt, stage);
}

// The chunked shape.
constexpr int kChunkedGatherTiles = 1 << 16;
constexpr int kChunkSub = kChunk / kWaves;      // elements of a wavefront in a chunk
constexpr int kChunkPerLane = kChunkSub / 64;   // mask words of a wavefront in a chunk

template <typename G, bool kFull>
__device__ __forceinline__ void gather_chunk(const Geometry &g, const TopkArgs &a, const Tile &tl, int tile,
                                             int q, int w, int *sums) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub0 = q * kChunk + wave * kChunkSub;   // first element of this wavefront in the tile
  const int64_t base = tl.start + sub0;
  const int rem = tl.len - sub0;
  const int nwords = kFull ? kChunkPerLane
                           : (rem <= 0 ? 0 : (rem >= kChunkSub ? kChunkPerLane : (rem + 63) / 64));
  auto ok = [&](int c) { return kFull || sub0 + 64 * c + lane < tl.len; };
  const size_t row = static_cast<size_t>(w) * g.N + base + lane;
  float *mem = a.memory + row;
  const G *gw = static_cast<const G *>(a.grads) + row;
  float x[kChunkPerLane];
#pragma unroll
  for (int c = 0; c < kChunkPerLane; ++c) {   // all loads first: the stores below may alias them
    x[c] = 0.0f;
    if (ok(c)) x[c] = mem[64 * c] + grad_at(gw + 64 * c);
  }
  const uint64_t selw = lane < nwords ? a.above[(base >> 6) + lane] : 0ull;
  // the tile's words before this chunk (fewer than kBlock), one per thread
  int before = static_cast<int>(threadIdx.x) < q * (kChunk / 64)
                   ? __popcll(a.above[(tl.start >> 6) + threadIdx.x]) : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o);
  int mine = 0;
#pragma unroll
  for (int c = 0; c < kChunkPerLane; ++c) mine += __popcll(readlane64(selw, c));
  if (lane == 0) {
    sums[wave] = mine;
    sums[kWaves + wave] = before;
  }
  __syncthreads();
  int64_t pos = a.tile_sel_off[tile];
  for (int v = 0; v < kWaves; ++v) pos += sums[kWaves + v] + (v < wave ? sums[v] : 0);
  // the memory in a loop of its own, one full-row store per slot
#pragma unroll
  for (int c = 0; c < kChunkPerLane; ++c) {
    const bool sel = (readlane64(selw, c) >> lane) & 1ull;   // never set past the end
    if (ok(c)) mem[64 * c] = sel ? 0.0f : x[c];
  }
  const int64_t k_end = a.k_off[tl.tensor + 1];   // pos stays below it when the selection holds k_t entries
  const int64_t tensor_start = tl.start - static_cast<int64_t>(tile - g.tile_begin[tl.tensor]) * kTile;
  float *vals = a.values + static_cast<size_t>(w) * a.K;
#pragma unroll
  for (int c = 0; c < kChunkPerLane; ++c) {
    const uint64_t bs = readlane64(selw, c);
    if ((bs >> lane) & 1ull) {
      const int64_t at = pos + __popcll(bs & lanemask_lt(lane));
      if (at < k_end) {
        store_nt(vals + at, x[c]);
        if (w == 0)
          store_nt(reinterpret_cast<uint32_t *>(a.index) + at,
                   static_cast<uint32_t>(base + 64 * c + lane - tensor_start));
      }
    }
    pos += __popcll(bs);
  }
}

template <typename G>
__global__ __launch_bounds__(kBlock) void topk_gather_chunk(Geometry g, TopkArgs a) {
  __shared__ int sums[2 * kWaves];   // per wavefront: its own entries, then the earlier words' entries
  const int tile = static_cast<int>(blockIdx.x / kChunksPerTile);
  const int q = static_cast<int>(blockIdx.x % kChunksPerTile);
  const int w = static_cast<int>(blockIdx.y);
  const Tile tl = g.tiles[tile];
  const int rem = tl.len - q * kChunk;   // uniform over the workgroup
  if (rem <= 0) return;                  // past the tile's end
  if (rem >= kChunk)
    gather_chunk<G, true>(g, a, tl, tile, q, w, sums);
  else
    gather_chunk<G, false>(g, a, tl, tile, q, w, sums);
}

// the server: average of the W messages, ascending workers from +0, then / W
template <bool kPow2>
__global__ __launch_bounds__(kBlock) void topk_average(TopkArgs a, int W) {
  const float wf = static_cast<float>(W);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  constexpr int kGroup = 8;   // workers whose loads are issued together
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j < a.K; j += stride) {
    float acc = 0.0f;
    for (int w0 = 0; w0 < W; w0 += kGroup) {
      float x[kGroup];
#pragma unroll
      for (int k = 0; k < kGroup; ++k)
        x[k] = w0 + k < W ? a.values[static_cast<size_t>(w0 + k) * a.K + j] : 0.0f;
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        if (w0 + k >= W) break;
        acc = acc + x[k];
      }
    }
    a.average[j] = kPow2 ? acc * (1.0f / wf) : acc / wf;
  }
}

unsigned stride_grid(int64_t items) {
  const int64_t blocks = (items + kBlock - 1) / kBlock;
  return static_cast<unsigned>(blocks < kStrideBlocks ? blocks : kStrideBlocks);
}

template <typename G>
void launch_select_typed(const Geometry &g, const TopkArgs &a, hipStream_t s) {
  const dim3 block(kBlock), tiles(g.num_tiles), tensors(g.T);
  hipLaunchKernelGGL(topk_reset, dim3(stride_grid(static_cast<int64_t>(g.T) * kMaxBins)), block, 0,
                     s, g, a);
  hipLaunchKernelGGL(topk_pass1<G>, tiles, block, 0, s, g, a);
  hipLaunchKernelGGL((topk_pick<11, true>), tensors, block, 0, s, a, kShift0);
  hipLaunchKernelGGL(topk_refill<G>, dim3(static_cast<unsigned>((g.num_tiles + kRefillTiles - 1) / kRefillTiles)),
                     block, 0, s, g, a);
  const dim3 cand_grid(static_cast<unsigned>((g.num_tiles + kCandTiles - 1) / kCandTiles));
  hipLaunchKernelGGL((topk_hist_shared<kShift1, 11>),
                     dim3(static_cast<unsigned>((g.num_tiles + kSharedTiles - 1) / kSharedTiles)), block, 0, s,
                     g, a);
  hipLaunchKernelGGL((topk_pick<11, false>), tensors, block, 0, s, a, kShift1);
  hipLaunchKernelGGL((topk_hist_cand<kShift2, 9>), cand_grid, block, 0, s, g, a);
  hipLaunchKernelGGL((topk_pick<9, false>), tensors, block, 0, s, a, kShift2);
  hipLaunchKernelGGL(topk_tile_counts, cand_grid, block, 0, s, g, a);
  hipLaunchKernelGGL(topk_offsets, tensors, block, 0, s, g, a);
  hipLaunchKernelGGL(topk_ties, cand_grid, block, 0, s, g, a);
}

}  // namespace

void launch_topk(TopkStage stage, const Geometry &g, bool bf16, const TopkArgs &a, hipStream_t s) {
  const dim3 block(kBlock);
  switch (stage) {
    case TopkStage::kSelect:
      if (bf16)
        launch_select_typed<uint16_t>(g, a, s);
      else
        launch_select_typed<float>(g, a, s);
      break;
    case TopkStage::kGather: {
      if (g.num_tiles <= kChunkedGatherTiles) {
        const dim3 grid(static_cast<unsigned>(g.num_tiles) * kChunksPerTile, static_cast<unsigned>(g.W));
        if (bf16)
          hipLaunchKernelGGL(topk_gather_chunk<uint16_t>, grid, block, 0, s, g, a);
        else
          hipLaunchKernelGGL(topk_gather_chunk<float>, grid, block, 0, s, g, a);
        break;
      }
      const int groups = (g.W + a.wgroup - 1) / a.wgroup;
      const dim3 grid(static_cast<unsigned>(g.num_tiles) * groups);
      if (bf16)
        hipLaunchKernelGGL(topk_gather<uint16_t>, grid, block, 0, s, g, a);
      else
        hipLaunchKernelGGL(topk_gather<float>, grid, block, 0, s, g, a);
      break;
    }
    case TopkStage::kAverage: {
      const dim3 grid(stride_grid(a.K));
      if ((g.W & (g.W - 1)) == 0)
        hipLaunchKernelGGL(topk_average<true>, grid, block, 0, s, a, g.W);
      else
        hipLaunchKernelGGL(topk_average<false>, grid, block, 0, s, a, g.W);
      break;
    }
  }
}

}  // namespace ob
