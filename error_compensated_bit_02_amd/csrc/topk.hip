// HIP kernels (gfx950) of the cyclic local top-k (CLT-k) codec: the
// commutative compressor of the review of "ScaleCom: Scalable Sparsified
// Gradient Compression ..." (Proposed method: cyclic local top-k aligns the
// workers' sparsity so that the exchange is an all-reduce).
//
// Per tensor, the leader worker (step mod W) ranks |x_leader| = |mem + g|
// and every worker sends its x at the leader's k largest positions.  The
// selection is exact: the k-th largest key (the bit pattern of |x|, which
// orders non-negative floats) is found by a 4-pass radix select with 8-bit
// digits (per-tile LDS histograms added into per-tensor histograms), ties at
// that key go to the lowest indices, and the positions are written in
// ascending order through per-tile offsets.  Then one dense pass over all
// workers gathers the messages and updates the memories, and the server
// averages the W messages in ascending worker order.
//
// The element mapping is the one of kernels.hip: a workgroup of 4
// wavefronts owns a tile of up to kTile elements of one tensor, lane l of
// wavefront v owns element 2048 v + 64 c + l, so ballots over one c are
// natural-order 64-bit words.
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

__device__ __forceinline__ bool valid(const Tile &tl, const TileLanes &ln, int c) {
  return ln.sub0 + 64 * c + ln.lane < tl.len;
}

// Ranking key of the leader's element: the bit pattern of |mem + g|.
template <typename G>
__device__ __forceinline__ uint32_t leader_key(const TopkArgs &a, const Geometry &g, int64_t i) {
  const size_t off = static_cast<size_t>(a.leader) * g.N + i;
  const float x = a.memory[off] + grad_at(static_cast<const G *>(a.grads) + off);
  return __float_as_uint(x) & 0x7fffffffu;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------------------
// radix select
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void topk_reset(Geometry g, TopkArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i < static_cast<int64_t>(g.T) * 256) a.hist[i] = 0u;
  if (i < g.T) {
    a.prefix[i] = 0u;
    a.krem[i] = static_cast<uint32_t>(a.k_off[i + 1] - a.k_off[i]);
  }
}

// Histogram of digit (key >> shift) & 255 over the keys whose higher digits
// equal the tensor's prefix so far.
template <typename G>
__global__ __launch_bounds__(kBlock) void topk_hist(Geometry g, TopkArgs a, int shift) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0u;
  __syncthreads();
  const Tile tl = g.tiles[blockIdx.x];
  const TileLanes ln = tile_lanes(tl);
  const uint32_t hi_mask = shift >= 24 ? 0u : ~((1u << (shift + 8)) - 1u);
  const uint32_t want = a.prefix[tl.tensor] & hi_mask;
  for (int c = 0; c < kPerLane; ++c) {
    if (!valid(tl, ln, c)) continue;
    const uint32_t key = leader_key<G>(a, g, ln.base + 64 * c + ln.lane);
    if ((key & hi_mask) == want) atomicAdd(&h[(key >> shift) & 255u], 1u);
  }
  __syncthreads();
  const uint32_t n = h[threadIdx.x];
  if (n) atomicAdd(&a.hist[static_cast<size_t>(tl.tensor) * 256 + threadIdx.x], n);
}

// One workgroup per tensor: the digit bin holding the krem-th largest key.
__global__ __launch_bounds__(kBlock) void topk_pick(Geometry g, TopkArgs a, int shift) {
  __shared__ uint32_t suf[257];
  __shared__ uint32_t krem_s;
  const int t = blockIdx.x;
  const int b = threadIdx.x;
  uint32_t *hist = a.hist + static_cast<size_t>(t) * 256;
  suf[b] = hist[b];
  if (b == 0) {
    suf[256] = 0u;
    krem_s = a.krem[t];   // read once, before the one writer below updates it
  }
  __syncthreads();
  // suffix sums: suf[b] = count of keys whose digit is >= b (Hillis-Steele)
  for (int d = 1; d < 256; d <<= 1) {
    const uint32_t add = (b + d < 256) ? suf[b + d] : 0u;
    __syncthreads();
    suf[b] += add;
    __syncthreads();
  }
  const uint32_t krem = krem_s;
  if (suf[b] >= krem && suf[b + 1] < krem) {   // exactly one bin satisfies this
    a.prefix[t] |= static_cast<uint32_t>(b) << shift;
    a.krem[t] = krem - suf[b + 1];
  }
  __syncthreads();
  hist[b] = 0u;   // ready for the next pass
}

// ---------------------------------------------------------------------------
// per-tile counts of keys above and at the threshold, then per-tensor offsets
// ---------------------------------------------------------------------------
template <typename G>
__global__ __launch_bounds__(kBlock) void topk_count(Geometry g, TopkArgs a) {
  __shared__ uint32_t cnt[2][kWaves];
  const Tile tl = g.tiles[blockIdx.x];
  const TileLanes ln = tile_lanes(tl);
  const uint32_t tau = a.prefix[tl.tensor];
  uint32_t gt = 0, eq = 0;
  for (int c = 0; c < kPerLane; ++c) {
    const bool ok = valid(tl, ln, c);
    const uint32_t key = ok ? leader_key<G>(a, g, ln.base + 64 * c + ln.lane) : 0u;
    gt += __popcll(__ballot(ok && key > tau));
    eq += __popcll(__ballot(ok && key == tau));
  }
  if (ln.lane == 0) {
    cnt[0][ln.wave] = gt;
    cnt[1][ln.wave] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t sg = 0, se = 0;
    for (int v = 0; v < kWaves; ++v) {
      sg += cnt[0][v];
      se += cnt[1][v];
    }
    a.tile_gt[blockIdx.x] = sg;
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
// selection: bitmask, per-word positions and the ascending index list
// ---------------------------------------------------------------------------
template <typename G>
__global__ __launch_bounds__(kBlock) void topk_select(Geometry g, TopkArgs a) {
  __shared__ int64_t weq[kWaves], wsel[kWaves];
  const Tile tl = g.tiles[blockIdx.x];
  const TileLanes ln = tile_lanes(tl);
  const int t = tl.tensor;
  const uint32_t tau = a.prefix[t];
  const int64_t r = a.krem[t];
  // phase 1: keys at the threshold per wavefront
  uint64_t gtw = 0, eqw = 0;   // lane c keeps word c of each mask
  int64_t neq = 0;
  for (int c = 0; c < kPerLane; ++c) {
    const bool ok = valid(tl, ln, c);
    const uint32_t key = ok ? leader_key<G>(a, g, ln.base + 64 * c + ln.lane) : 0u;
    const uint64_t bg = __ballot(ok && key > tau);
    const uint64_t be = __ballot(ok && key == tau);
    if (ln.lane == c) {
      gtw = bg;
      eqw = be;
    }
    neq += __popcll(be);
  }
  if (ln.lane == 0) weq[ln.wave] = neq;
  __syncthreads();
  int64_t eq_run = a.tile_eq_before[blockIdx.x];
  for (int v = 0; v < ln.wave; ++v) eq_run += weq[v];
  // phase 2: selected = above the threshold, or at it with tie rank < r
  uint64_t selw = 0;
  int64_t nsel = 0;
  for (int c = 0; c < kPerLane; ++c) {
    const uint64_t be = __shfl(eqw, c);
    const uint64_t bg = __shfl(gtw, c);
    const int64_t rank = eq_run + __popcll(be & lanemask_lt(ln.lane));
    const bool take_eq = ((be >> ln.lane) & 1ull) && rank < r;
    const uint64_t bs = bg | __ballot(take_eq);
    if (ln.lane == c) selw = bs;
    eq_run += __popcll(be);
    nsel += __popcll(bs);
  }
  if (ln.lane == 0) wsel[ln.wave] = nsel;
  __syncthreads();
  int64_t pos = a.tile_sel_off[blockIdx.x];
  for (int v = 0; v < ln.wave; ++v) pos += wsel[v];
  // phase 3: positions in ascending index order (index = position within the tensor)
  const int64_t tensor_start =
      tl.start - static_cast<int64_t>(static_cast<int>(blockIdx.x) - g.tile_begin[t]) * kTile;
  const int64_t k_end = a.k_off[t + 1];
  for (int c = 0; c < kPerLane; ++c) {
    const uint64_t bs = __shfl(selw, c);
    const int64_t word = (ln.base >> 6) + c;
    if (c < ln.nwords) {
      if (ln.lane == 0) {
        a.sel_words[word] = bs;
        a.word_pos[word] = pos;
      }
      if ((bs >> ln.lane) & 1ull) {
        const int64_t at = pos + __popcll(bs & lanemask_lt(ln.lane));
        if (at < k_end)   // always true when the selection holds k_t entries
          a.index[at] = static_cast<int32_t>(ln.base + 64 * c + ln.lane - tensor_start);
      }
    }
    pos += __popcll(bs);
  }
}

// ---------------------------------------------------------------------------
// gather the messages of every worker and update the memories; workgroups are
// (worker group, tile), group-major as in the worker passes
// ---------------------------------------------------------------------------
template <typename G>
__global__ __launch_bounds__(kBlock) void topk_gather(Geometry g, TopkArgs a) {
  const int tile = static_cast<int>(blockIdx.x % static_cast<unsigned>(g.num_tiles));
  const int grp = static_cast<int>(blockIdx.x / static_cast<unsigned>(g.num_tiles));
  const int w_lo = grp * a.wgroup;
  const int w_hi = min(g.W, w_lo + a.wgroup);
  const Tile tl = g.tiles[tile];
  const TileLanes ln = tile_lanes(tl);
  const int64_t k_end = a.k_off[tl.tensor + 1];
  // word c of the selection mask and its first position, held by lane c
  const uint64_t selw = ln.lane < ln.nwords ? a.sel_words[(ln.base >> 6) + ln.lane] : 0ull;
  const int64_t posw = ln.lane < ln.nwords ? a.word_pos[(ln.base >> 6) + ln.lane] : 0;
  for (int w = w_lo; w < w_hi; ++w) {
    float *mem = a.memory + static_cast<size_t>(w) * g.N + ln.base + ln.lane;
    const G *gw = static_cast<const G *>(a.grads) + static_cast<size_t>(w) * g.N + ln.base + ln.lane;
    float *vals = a.values + static_cast<size_t>(w) * a.K;
    for (int c = 0; c < kPerLane; ++c) {
      const uint64_t bs = __shfl(selw, c);
      const int64_t p0 = __shfl(posw, c);
      if (!valid(tl, ln, c)) continue;
      const float x = mem[64 * c] + grad_at(gw + 64 * c);
      if ((bs >> ln.lane) & 1ull) {
        const int64_t at = p0 + __popcll(bs & lanemask_lt(ln.lane));
        if (at < k_end) vals[at] = x;   // always true when the selection holds k_t entries
        mem[64 * c] = 0.0f;
      } else {
        mem[64 * c] = x;
      }
    }
  }
}

// the server: average of the W messages, ascending workers from +0, then / W
template <bool kPow2>
__global__ __launch_bounds__(kBlock) void topk_average(TopkArgs a, int W) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (j >= a.K) return;
  float acc = 0.0f;
  for (int w = 0; w < W; ++w) acc = acc + a.values[static_cast<size_t>(w) * a.K + j];
  const float wf = static_cast<float>(W);
  a.average[j] = kPow2 ? acc * (1.0f / wf) : acc / wf;
}

template <typename G>
void launch_topk_typed(const Geometry &g, const TopkArgs &a, hipStream_t s) {
  const dim3 block(kBlock), tiles(g.num_tiles);
  const int64_t resets = static_cast<int64_t>(g.T) * 256;
  hipLaunchKernelGGL(topk_reset, dim3(static_cast<unsigned>((resets + kBlock - 1) / kBlock)), block,
                     0, s, g, a);
  for (int shift = 24; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(topk_hist<G>, tiles, block, 0, s, g, a, shift);
    hipLaunchKernelGGL(topk_pick, dim3(g.T), block, 0, s, g, a, shift);
  }
  hipLaunchKernelGGL(topk_count<G>, tiles, block, 0, s, g, a);
  hipLaunchKernelGGL(topk_offsets, dim3(g.T), block, 0, s, g, a);
  hipLaunchKernelGGL(topk_select<G>, tiles, block, 0, s, g, a);
  const int groups = (g.W + a.wgroup - 1) / a.wgroup;
  hipLaunchKernelGGL(topk_gather<G>, dim3(static_cast<unsigned>(g.num_tiles) * groups), block, 0, s,
                     g, a);
  const dim3 avg_grid(static_cast<unsigned>((a.K + kBlock - 1) / kBlock));
  if ((g.W & (g.W - 1)) == 0)
    hipLaunchKernelGGL(topk_average<true>, avg_grid, block, 0, s, a, g.W);
  else
    hipLaunchKernelGGL(topk_average<false>, avg_grid, block, 0, s, a, g.W);
}

}  // namespace

void launch_topk(const Geometry &g, bool bf16, const TopkArgs &a, hipStream_t s) {
  if (bf16)
    launch_topk_typed<uint16_t>(g, a, s);
  else
    launch_topk_typed<float>(g, a, s);
}

}  // namespace ob
