// Internal declarations shared by the host library (api.cpp) and the HIP
// kernels (kernels.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ob {

// One workgroup handles one tile (or one chunk of one; see kChunk): kTile
// consecutive elements of one tensor (a tensor's last tile may be shorter;
// no tile spans two tensors).  Each of
// the kWaves wavefronts owns kSub consecutive elements of the tile, and lane
// l of a wavefront owns element 64*c + l of its range for c < kPerLane, so a
// wavefront-wide ballot over one c yields one packed sign word in natural
// bit order.
// Elements per tile (a multiple of 256); 8192 measured best on gfx950 for
// the worker passes (4096 and 16384 were slower or spilled).
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kTile = 8192;
constexpr int kSub = kTile / kWaves;
constexpr int kPerLane = kSub / 64;

// Lane `lane` of `old` replaced by the wavefront-uniform `value` (one
// v_writelane_b32): the LLVM intrinsic, reached through its name.
__device__ int amdgcn_writelane(int value, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// Sign word c of a wavefront goes to lane c, kept as two 32-bit halves.
struct LaneWords {
  uint32_t lo = 0, hi = 0;
  __device__ __forceinline__ void put(uint64_t word, int c) {
    lo = static_cast<uint32_t>(amdgcn_writelane(static_cast<int>(static_cast<uint32_t>(word)), c,
                                                static_cast<int>(lo)));
    hi = static_cast<uint32_t>(amdgcn_writelane(static_cast<int>(static_cast<uint32_t>(word >> 32)), c,
                                                static_cast<int>(hi)));
  }
  __device__ __forceinline__ uint64_t get() const { return (static_cast<uint64_t>(hi) << 32) | lo; }
};

struct Tile {
  int64_t start;   // first element of the tile in the flat layout
  int32_t len;     // elements in the tile (1..kTile)
  int32_t tensor;  // tensor the tile belongs to
};

// Device-side description of a tensor list.  The server's scales are one per
// "piece": a tensor, or with a C-way partitioned server one chunk of a tensor
// (a run of whole tiles); with C = 1 the pieces are the tensors.
struct Geometry {
  const Tile *tiles;
  const int32_t *tile_begin;  // [T+1]: tiles of tensor t are tile_begin[t] .. tile_begin[t+1]-1
  const int64_t *numel;       // [T]
  const int32_t *tile_piece;  // [num_tiles]: server-scale index of each tile
  const int32_t *piece_begin; // [S+1]: tiles of piece j are piece_begin[j] .. piece_begin[j+1]-1
  const int64_t *piece_numel; // [S]
  int32_t S;                  // number of server scales
  int32_t num_tiles;
  int32_t T;
  int32_t W;
  int64_t N;                  // padded elements per flat buffer row
  int64_t Nw;                 // N / 64 sign words per packed row
};

// Partial sums of squares: (W+1) rows (workers, then the server) of
// num_tiles compensated fp64 pairs (hi, lo), one per tile.
inline size_t partials_count(int W, int num_tiles) {
  return static_cast<size_t>(W + 1) * static_cast<size_t>(num_tiles);
}

// The chunked worker passes (the residual form's, the first residual step's
// and, with fp32 gradients, the strict pass 2) and the chunked CLT-k gather:
// one workgroup per (chunk of kChunk elements of a tile, worker), lane l of
// wavefront v owning element kChunk/kWaves * v + 64*c + l of the chunk.  The
// passes with sums of squares keep one partial per chunk: W rows of
// num_tiles * kChunksPerTile pairs (chunks past a tile's end hold 0).
constexpr int kChunk = 1024;
constexpr int kChunksPerTile = kTile / kChunk;
static_assert(kTile % kChunk == 0 && kChunk % (64 * kWaves) == 0, "chunk shape");
inline size_t chunk_partials_count(int W, int num_tiles) {
  return static_cast<size_t>(W) * static_cast<size_t>(num_tiles) * kChunksPerTile;
}

enum Kind {
  K_WORKER_PASS1 = 0,
  K_SCALE_FINALIZE,
  K_WORKER_PASS2,
  K_SERVER_PASS1,
  K_SERVER_PASS2,
  K_SERVER_PASS2_UPDATE,
  K_APPLY_UPDATE,
  K_WORKER_RESIDUAL,
  K_SERVER_RESIDUAL,
  K_UPDATE_RESIDUAL,
  K_MATERIALIZE,
  K_WARMUP,
  K_ZERO_ERRORS,
  K_TRUST_NORMS,
  K_TRUST_RATIO,
  K_TOPK_SELECT,
  K_TOPK_GATHER,
  K_TOPK_AVERAGE,
  K_NUM_KINDS
};

enum class WorkerPass { kStrictSigns, kStrictErrors, kResidualFirst, kResidual };
enum class ServerPass { kStrictSums, kStrictErrors, kStrictErrorsUpdate, kResidualFirst, kResidual };

struct WorkerArgs {
  const void *grads;         // [W][N] fp32 or bf16
  const float *m;            // [N] momentum (strict and first residual step)
  float *err_w;              // [W][N] errors (strict) or compressed values (residual)
  uint64_t *packed_w;        // [W][Nw]
  const float *scale_w;      // [W][T]: this step's (strict errors) or the previous step's (residual)
  const uint64_t *packed_s;  // [Nw] previous server message (residual)
  const float *scale_s;      // [T]  previous server scales (residual)
  double2 *partials;         // per-tile partials (strict passes)
  double2 *chunk_partials;   // per-chunk partials (residual passes)
  int w0, w1;                // workers [w0, w1)
  int wgroup;                // workers per workgroup of the tiled strict passes (see worker_group_size)
  float c1, c2;
};

// Workers handled by one workgroup of a tiled worker pass (the strict form's
// two passes, and the tiled CLT-k gather of long lists).  At most kMaxGroup, so
// the workgroups resident at once stream few rows; fewer when the tile count
// alone would leave the launch short of kMinBlocks workgroups (many small
// launches of a small list would leave most of the 256 CUs idle at the tail).
constexpr int kMaxGroup = 16;
constexpr int kMinBlocks = 8192;
// A launch's work-items per dimension must fit in 32 bits: at most this many
// workgroups of kBlock threads.
constexpr int64_t kMaxGrid = 0xffffffffLL / kBlock;

inline int worker_group_size(int workers, int num_tiles) {
  int groups = (workers + kMaxGroup - 1) / kMaxGroup;
  const int want = (kMinBlocks + num_tiles - 1) / num_tiles;
  if (groups < want) groups = want < workers ? want : workers;
  return (workers + groups - 1) / groups;
}

struct ServerArgs {
  const uint64_t *packed_w;  // [W][Nw]
  const float *scale_w;      // [W][T] this step's worker scales
  float *err_s;              // [N] error (strict) or compressed value (residual)
  double2 *partials;
  const float *scale_s;      // [T] this step's (strict) or the previous step's (residual)
  uint64_t *packed_s;        // [Nw] written
  const float *v;            // fused strict update only
  float *m;
  float *params;
  float lr, eps;
};

struct UpdateArgs {
  const uint64_t *packed_s;
  const float *scale_s;
  const float *v;
  float *m;                  // written when the momentum is stored
  float *params;
  float lr, eps;
  const float *ratio;        // [T] per-tensor trust ratios (trust-ratio update only)
  float wd;                  // weight decay added to the direction (trust-ratio update only)
};

struct MaterializeArgs {     // inputs and outputs may alias
  const float *x_w;
  const float *scale_w;
  const float *z;
  const float *scale_s;
  float *e_w;
  float *e_s;
  float *m;
};

struct WarmupArgs {
  const void *grads;         // [W][N] fp32 or bf16
  float *m;                  // [N]
  float *v;                  // [N]
  float *params;             // [N]
  float c1, c2, b2, cb2, lr, eps;
};

// Cyclic local top-k codec (topk.hip).
struct TopkArgs {
  const void *grads;         // [W][N] fp32 or bf16
  float *memory;             // [W][N] local memories, read and overwritten
  int32_t *index;            // [K] positions within each tensor, ascending per tensor
  float *values;             // [W][K] messages
  float *average;            // [K] the server's average
  int64_t K;                 // total entries over the tensor list
  const int64_t *k_off;      // [T+1] tensor t's entries are k_off[t] .. k_off[t+1]-1
  uint32_t *hist;            // [T][2048] radix histograms
  uint32_t *prefix;          // [T] key prefix found so far, then the k-th largest key
  uint32_t *krem;            // [T] rank still to find, then the ties to take
  uint32_t *cand;            // [N] per tile, its keys inside the first-digit window, compacted
  uint16_t *cand_pos;        // [N] their positions within the tile, ascending
  uint32_t *tile_m;          // [num_tiles] number of those keys
  uint64_t *above;           // [Nw] bit per element: key above the window; after the select stage, the selection
  uint32_t *pred;            // [T] first digit of the last threshold (the window's centre); kept
  uint32_t *miss;            // [T] 1 when this exchange's first digit fell outside the window
  uint32_t *tile_gt;         // [num_tiles] keys above the threshold
  uint32_t *tile_eq;         // [num_tiles] keys at the threshold
  int64_t *tile_eq_before;   // [num_tiles] keys at the threshold in earlier tiles of the tensor
  int64_t *tile_sel_off;     // [num_tiles] position of the tile's first selected entry
  int leader;                // worker whose values rank the positions
  int wgroup;                // workers per workgroup in the tiled gather (see worker_group_size)
};

// The codec's three stages: the leader's threshold and the selection (radix
// select, per-tile counts and offsets, the selection mask), the gather of the
// index list and every worker's message with the memory update, and the
// server's average.
enum class TopkStage { kSelect, kGather, kAverage };
void launch_topk(TopkStage stage, const Geometry &g, bool bf16, const TopkArgs &a, hipStream_t s);

void launch_worker(WorkerPass pass, const Geometry &g, bool bf16, const WorkerArgs &a, hipStream_t s);
// Scales of rows [row0, row0 + nrows) of the partials (rows of `cols` pairs,
// `per` pairs per tile) over `count` items whose tile ranges are begin[i] ..
// begin[i+1]-1 and sizes numel[i]; row r's scale of item i goes to
// out[(r - row0) * count + i].
// Scales from partial sums: items [row0, row0 + nrows) x [0, count), item i
// of a row summing partials [begin[i] * per, begin[i + 1] * per).  A whole
// workgroup per item when the largest item has at least kWideFinalize
// partials, one wavefront per item otherwise.
constexpr int64_t kWideFinalize = 4096;
void launch_scale_finalize(const Geometry &g, const double2 *partials, int64_t cols, int per, int row0,
                           int nrows, const int32_t *begin, const int64_t *numel, int count, float *out,
                           int64_t max_item_partials, hipStream_t s);
void launch_server(ServerPass pass, const Geometry &g, const ServerArgs &a, hipStream_t s);
// with_ratio: p -= lr * (ratio[t] * u), u = m / (sqrt(v) + eps) (+ wd * p)
void launch_update(bool store_m, bool with_ratio, const Geometry &g, const UpdateArgs &a,
                   hipStream_t s);
// Per-tile sums of p^2 and u^2 into partial rows 0 and 1, then per-tensor ratios.
void launch_trust_norms(const Geometry &g, const UpdateArgs &a, double2 *partials, hipStream_t s);
void launch_trust_ratio(const Geometry &g, const double2 *partials, float *ratio, hipStream_t s);
void launch_materialize(const Geometry &g, const MaterializeArgs &a, hipStream_t s);
void launch_warmup(const Geometry &g, bool bf16, const WarmupArgs &a, hipStream_t s);
void launch_zero_errors(const Geometry &g, float *err_w, float *err_s, hipStream_t s);

// The no-allocation step's scratch: one static device array of this many
// bytes per GPU (kernels.hip), which holds the step's partial sums and trust
// ratios.  static_scratch_address resolves its device address on the current
// device (once per device; later calls return the cached address) and
// returns hipSuccess or the error of the lookup.
constexpr size_t kStaticScratchBytes = size_t{64} << 20;
hipError_t static_scratch_address(void **out);

}  // namespace ob
