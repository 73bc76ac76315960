// HIP kernels (gfx950) of the cyclic local top-k (CLT-k) codec: the
// commutative compressor of the review of "ScaleCom: Scalable Sparsified
// Gradient Compression ..." (Proposed method: cyclic local top-k aligns the
// workers' sparsity so that the exchange is an all-reduce).
//
// Per tensor, the leader worker (step mod W) ranks |x_leader| = |mem + g|
// and every worker sends its x at the leader's k largest positions.  The
// selection is exact: the k-th largest key (the bit pattern of |x|, which
// orders non-negative floats) is found by a radix select with 11, 11 and
// 9-bit digits (per-tile LDS histograms added into per-tensor histograms).
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

template <typename G>
__device__ __forceinline__ float grad_at(const G *p);
template <>
__device__ __forceinline__ float grad_at<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float grad_at<uint16_t>(const uint16_t *p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
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

// Ranking key of an element: the bit pattern of |mem + g|.
template <typename G>
__device__ __forceinline__ uint32_t key_of(const float *mem, const G *grads, int64_t i) {
  return __float_as_uint(mem[i] + grad_at(grads + i)) & 0x7fffffffu;
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
constexpr uint32_t kWindowBelow = 2, kWindowAbove = 4;   // the threshold's bin drifts upward

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
// Workgroup-uniform call; wcnt holds 2 * kWaves counters.
template <bool kFull>
__device__ __forceinline__ void window_tile(const TopkArgs &a, const Tile &tl, const TileLanes &ln,
                                            const uint32_t (&key)[kPerLane], Window w,
                                            uint32_t *wcnt) {
  uint32_t nm = 0, ngt = 0;
  uint64_t gtw = 0;   // lane c: word c of the above-window mask
#pragma unroll
  for (int c = 0; c < kPerLane; ++c) {
    const bool ok = slot_ok<kFull>(tl, ln, c);
    const uint32_t d0 = key[c] >> kShift0;
    const uint64_t bg = __ballot(ok && d0 > w.hi);
    if (ln.lane == c) gtw = bg;
    nm += __popcll(__ballot(ok && d0 >= w.lo && d0 <= w.hi));
    ngt += __popcll(bg);
  }
  if (ln.lane < ln.nwords) a.above[(ln.base >> 6) + ln.lane] = gtw;
  if (ln.lane == 0) {
    wcnt[ln.wave] = nm;
    wcnt[kWaves + ln.wave] = ngt;
  }
  __syncthreads();
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
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0, gt = 0;
    for (int v = 0; v < kWaves; ++v) {
      m += wcnt[v];
      gt += wcnt[kWaves + v];
    }
    a.tile_m[blockIdx.x] = m;
    a.tile_gt[blockIdx.x] = gt;   // completed by topk_tile_counts
    a.tile_eq[blockIdx.x] = 0u;
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
  const Tile tl = g.tiles[blockIdx.x];
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
      window_tile<true>(a, tl, ln, key, w, wcnt);
    else
      window_tile<false>(a, tl, ln, key, w, wcnt);
  }
  __syncthreads();
  uint32_t *out = a.hist + static_cast<size_t>(tl.tensor) * kMaxBins;
  for (int i = threadIdx.x; i < kMaxBins; i += kBlock)
    if (h[i]) atomicAdd(&out[i], h[i]);
}

// After digit 0 is known: whether it fell in the predicted window (if not,
// the fallback pass rebuilds the tensor's per-tile data), and the prediction
// for the next exchange.
__global__ __launch_bounds__(kBlock) void topk_check(Geometry g, TopkArgs a) {
  const int t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= g.T) return;
  const Window w = predicted_window(a, t);
  const uint32_t b0 = a.prefix[t] >> kShift0;
  a.miss[t] = (w.lo <= w.hi && b0 >= w.lo && b0 <= w.hi) ? 0u : 1u;
  a.pred[t] = b0;
}

// Fallback: for the tensors whose digit 0 missed the window, the per-tile
// data for the window [b0, b0], from the leader's memory and gradient again.
template <typename G>
__global__ __launch_bounds__(kBlock) void topk_refill(Geometry g, TopkArgs a) {
  __shared__ uint32_t wcnt[2 * kWaves];
  const Tile tl = g.tiles[blockIdx.x];
  if (a.miss[tl.tensor] == 0u) return;   // uniform over the workgroup
  const TileLanes ln = tile_lanes(tl);
  const uint32_t b0 = a.prefix[tl.tensor] >> kShift0;
  uint32_t key[kPerLane];
  if (tl.len == kTile) {
    leader_keys<G, true>(g, a, tl, ln, key);
    window_tile<true>(a, tl, ln, key, Window{b0, b0}, wcnt);
  } else {
    leader_keys<G, false>(g, a, tl, ln, key);
    window_tile<false>(a, tl, ln, key, Window{b0, b0}, wcnt);
  }
}

// Digits 1 and 2 over the candidates only: per-tensor histograms of
// (key >> kShiftD) & (2^kBits - 1) over the candidates whose higher bits equal
// the prefix found so far.  A tile holds few candidates, so a workgroup walks
// kCandTiles consecutive tiles with one LDS histogram, added to the tensor's
// when the tensor changes and at the end.
constexpr int kCandTiles = 16;

template <int kBins>
__device__ __forceinline__ void flush_bins(uint32_t *h, uint32_t *out) {
  __syncthreads();   // every count of the tensor is in
  for (int i = threadIdx.x; i < kBins; i += kBlock) {
    if (h[i]) atomicAdd(&out[i], h[i]);
    h[i] = 0u;
  }
  __syncthreads();   // zeroed before the next tensor's counts
}

template <int kShiftD, int kBits>
__global__ __launch_bounds__(kBlock) void topk_hist_cand(Geometry g, TopkArgs a) {
  constexpr int kBins = 1 << kBits;
  constexpr int kHigh = kShiftD + kBits;   // bits above this digit are fixed
  __shared__ uint32_t h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kBlock) h[i] = 0u;
  __syncthreads();
  const int t0 = static_cast<int>(blockIdx.x) * kCandTiles;
  const int t1 = min(t0 + kCandTiles, g.num_tiles);
  int cur = -1;          // tensor whose counts h holds (uniform over the workgroup)
  uint32_t want = 0u;
  for (int tile = t0; tile < t1; ++tile) {
    const uint32_t m = a.tile_m[tile];
    if (m == 0) continue;   // uniform over the workgroup
    const Tile tl = g.tiles[tile];
    if (tl.tensor != cur) {
      if (cur >= 0) flush_bins<kBins>(h, a.hist + static_cast<size_t>(cur) * kMaxBins);
      cur = tl.tensor;
      want = a.prefix[cur] >> kHigh;
    }
    const uint32_t *cand = a.cand + tl.start;
    for (uint32_t j = threadIdx.x; j < m; j += kBlock) {
      const uint32_t key = cand[j];
      if ((key >> kHigh) == want) atomicAdd(&h[(key >> kShiftD) & (kBins - 1)], 1u);
    }
  }
  if (cur >= 0) flush_bins<kBins>(h, a.hist + static_cast<size_t>(cur) * kMaxBins);
}

// One workgroup per tensor: the digit bin holding the krem-th largest key.
// Thread b owns bins kPer b .. kPer b + kPer - 1.
template <int kBits>
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
        a.prefix[t] |= static_cast<uint32_t>(b * kPer + j) << shift;
        a.krem[t] = krem - above;
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
// give the rest.  A tile without candidates returns at once.
__global__ __launch_bounds__(kBlock) void topk_tile_counts(Geometry g, TopkArgs a) {
  __shared__ uint32_t cnt[2][kWaves];
  const uint32_t m = a.tile_m[blockIdx.x];
  if (m == 0) return;   // uniform over the workgroup
  const Tile tl = g.tiles[blockIdx.x];
  const uint32_t tau = a.prefix[tl.tensor];
  const uint32_t *cand = a.cand + tl.start;
  uint32_t gt = 0, eq = 0;
  for (uint32_t j0 = 0; j0 < m; j0 += kBlock) {   // uniform trip count: ballots stay converged
    const uint32_t j = j0 + threadIdx.x;
    const uint32_t key = j < m ? cand[j] : 0u;
    gt += __popcll(__ballot(j < m && key > tau));
    eq += __popcll(__ballot(j < m && key == tau));
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    cnt[0][wave] = gt;
    cnt[1][wave] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t sg = 0, se = 0;
    for (int v = 0; v < kWaves; ++v) {
      sg += cnt[0][v];
      se += cnt[1][v];
    }
    a.tile_gt[blockIdx.x] += sg;
    a.tile_eq[blockIdx.x] = se;
  }
}

// One workgroup per tensor: exclusive scans over the tensor's tiles of the
// keys at the threshold and of the selected entries (ties taken in order).
__global__ __launch_bounds__(kBlock) void topk_offsets(Geometry g, TopkArgs a) {
  __shared__ int64_t sa[kBlock], sb[kBlock];
  const int t = blockIdx.x;
  const int first = g.tile_begin[t], last = g.tile_begin[t + 1];
  const int64_t r = a.krem[t];   // keys equal to the threshold that are taken
  int64_t eq_base = 0, sel_base = a.k_off[t];
  for (int c0 = first; c0 < last; c0 += kBlock) {
    const int i = c0 + threadIdx.x;
    const int64_t eq = i < last ? a.tile_eq[i] : 0;
    sa[threadIdx.x] = eq;
    __syncthreads();
    for (int d = 1; d < kBlock; d <<= 1) {   // inclusive scan of eq
      const int64_t add = threadIdx.x >= d ? sa[threadIdx.x - d] : 0;
      __syncthreads();
      sa[threadIdx.x] += add;
      __syncthreads();
    }
    const int64_t eq_before = eq_base + sa[threadIdx.x] - eq;
    const int64_t take = eq_before >= r ? 0 : (r - eq_before < eq ? r - eq_before : eq);
    const int64_t sel = i < last ? a.tile_gt[i] + take : 0;
    sb[threadIdx.x] = sel;
    __syncthreads();
    for (int d = 1; d < kBlock; d <<= 1) {   // inclusive scan of sel
      const int64_t add = threadIdx.x >= d ? sb[threadIdx.x - d] : 0;
      __syncthreads();
      sb[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < last) {
      a.tile_eq_before[i] = eq_before;
      a.tile_sel_off[i] = sel_base + sb[threadIdx.x] - sel;
    }
    const int64_t eq_tot = sa[kBlock - 1], sel_tot = sb[kBlock - 1];
    __syncthreads();
    eq_base += eq_tot;
    sel_base += sel_tot;
  }
}

// ---------------------------------------------------------------------------
// selection and gather.  Workgroups are (worker group, tile), group-major as
// in the worker passes.  Each rebuilds its tile's selection from the mask of
// keys above the window and the candidates (read-only here, so groups need
// no ordering): selected = key above the threshold, or at it with tie rank
// < r; lane c of each wavefront keeps word c of the mask and the position of
// its first selected entry.  The first group writes the index list; every
// group then streams its workers.
//
// A tile's selected entries are one contiguous run of positions in each
// worker's message, so the workgroup stages all its workers' entries in LDS
// and writes them with one coalesced pass at the end: written directly, each
// would be a 4-byte store into a line that many other stores also write.
// When the run times the workers exceeds kStage entries the entries are
// written directly (at such densities the direct stores are nearly dense).
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

// The tile's selection: keys above the window (the mask), and the candidates
// above the threshold or at it with tie rank < r.  The
// candidates are in ascending position order, so a key at the threshold ranks
// after tile_eq_before[tile] of them in earlier tiles and after those at the
// threshold before it in the list.  Lane c of each wavefront then holds word c
// of the mask and the position of its first selected entry.
__device__ __forceinline__ TileSelection select_words(const Geometry &g, const TopkArgs &a,
                                                      const Tile &tl, int tile, const TileLanes &ln,
                                                      int64_t *wcnt, uint64_t *smask,
                                                      uint32_t *stage, bool write_index) {
  const int t = tl.tensor;
  const uint32_t tau = a.prefix[t];
  const int64_t r = a.krem[t];
  const int tile_words = (tl.len + 63) / 64;
  for (int i = threadIdx.x; i < tile_words; i += kBlock) smask[i] = a.above[(tl.start >> 6) + i];
  __syncthreads();
  const uint32_t m = a.tile_m[tile];   // uniform over the workgroup
  const uint32_t *cand = a.cand + tl.start;
  const uint16_t *cand_pos = a.cand_pos + tl.start;
  int64_t eq_run = a.tile_eq_before[tile];
  for (uint32_t j0 = 0; j0 < m; j0 += kBlock) {
    const uint32_t j = j0 + threadIdx.x;
    const bool valid = j < m;
    const uint32_t key = valid ? cand[j] : 0u;
    const bool at_tau = valid && key == tau;
    const uint64_t be = __ballot(at_tau);
    if (ln.lane == 0) wcnt[ln.wave] = __popcll(be);
    __syncthreads();
    int64_t before = 0, chunk = 0;
    for (int v = 0; v < kWaves; ++v) {
      if (v < ln.wave) before += wcnt[v];
      chunk += wcnt[v];
    }
    const int64_t rank = eq_run + before + __popcll(be & lanemask_lt(ln.lane));
    if (valid && (key > tau || (at_tau && rank < r))) {
      const uint32_t p = cand_pos[j];
      atomicOr(reinterpret_cast<unsigned long long *>(&smask[p >> 6]), 1ull << (p & 63));
    }
    eq_run += chunk;
    __syncthreads();   // wcnt and the mask words are complete
  }
  TileSelection sel;
  sel.selw = ln.lane < ln.nwords ? smask[ln.wave * kPerLane + ln.lane] : 0ull;
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
  // positions in ascending index order (index = position within the tensor)
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
                                            int tile, int w_lo, int w_hi, int64_t *wcnt,
                                            uint64_t *smask, uint32_t *stage) {
  const TileLanes ln = tile_lanes(tl);
  const int64_t k_end = a.k_off[tl.tensor + 1];
  const TileSelection sel = select_words(g, a, tl, tile, ln, wcnt, smask, stage, w_lo == 0);
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
  __shared__ uint64_t smask[kTile / 64];
  __shared__ uint32_t stage[kStage];
  const int tile = static_cast<int>(blockIdx.x % static_cast<unsigned>(g.num_tiles));
  const int grp = static_cast<int>(blockIdx.x / static_cast<unsigned>(g.num_tiles));
  const int w_lo = grp * a.wgroup;
  const int w_hi = min(g.W, w_lo + a.wgroup);
  const Tile tl = g.tiles[tile];
  if (tl.len == kTile)
    gather_tile<G, true>(g, a, tl, tile, w_lo, w_hi, wcnt, smask, stage);
  else
    gather_tile<G, false>(g, a, tl, tile, w_lo, w_hi, wcnt, smask, stage);
}

// the server: average of the W messages, ascending workers from +0, then / W
template <bool kPow2>
__global__ __launch_bounds__(kBlock) void topk_average(TopkArgs a, int W) {
  const float wf = static_cast<float>(W);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j < a.K; j += stride) {
    float acc = 0.0f;
    for (int w = 0; w < W; ++w) acc = acc + a.values[static_cast<size_t>(w) * a.K + j];
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
  hipLaunchKernelGGL(topk_pick<11>, tensors, block, 0, s, a, kShift0);
  hipLaunchKernelGGL(topk_check, dim3(static_cast<unsigned>((g.T + kBlock - 1) / kBlock)), block, 0, s,
                     g, a);
  hipLaunchKernelGGL(topk_refill<G>, tiles, block, 0, s, g, a);
  const dim3 cand_grid(static_cast<unsigned>((g.num_tiles + kCandTiles - 1) / kCandTiles));
  hipLaunchKernelGGL((topk_hist_cand<kShift1, 11>), cand_grid, block, 0, s, g, a);
  hipLaunchKernelGGL(topk_pick<11>, tensors, block, 0, s, a, kShift1);
  hipLaunchKernelGGL((topk_hist_cand<kShift2, 9>), cand_grid, block, 0, s, g, a);
  hipLaunchKernelGGL(topk_pick<9>, tensors, block, 0, s, a, kShift2);
  hipLaunchKernelGGL(topk_tile_counts, tiles, block, 0, s, g, a);
  hipLaunchKernelGGL(topk_offsets, tensors, block, 0, s, g, a);
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
