// Host side of the C ABI declared in include/ob.h: argument checks, the
// padded layout and tile table, scratch ownership, launch sequencing and the
// optional per-kernel event timing.
#include "ob.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>
#include <utility>
#include <vector>

#include "internal.h"

namespace {

struct EventPair {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

}  // namespace

struct ob_ctx {
  int32_t T = 0;
  int32_t W = 0;
  bool bf16 = false;
  float c1 = 0.0f;
  float c2 = 0.0f;
  float eps = 0.0f;
  std::vector<int64_t> numel;
  std::vector<int64_t> off;
  int64_t N = 0;
  int32_t num_tiles = 0;
  int32_t max_tensor_tiles = 0;      // tiles of the largest tensor
  int32_t max_piece_tiles = 0;       // tiles of the largest server piece
  std::vector<int32_t> tile_begin;   // host copy [T+1]
  int32_t server_chunks = 1;
  int32_t S = 0;                     // server scales (pieces)
  bool trust_ratio = false;          // layer-wise trust-ratio update
  float weight_decay = 0.0f;
  float *d_ratio = nullptr;          // [T] trust ratios (device scratch)
  // cyclic local top-k codec (allocated by ob_cltk_configure)
  void *topk_scratch = nullptr;
  ob::TopkArgs topk{};
  std::vector<int64_t> k_off;        // host copy [T+1]
  int32_t *d_tile_piece = nullptr;   // device views into scratch
  int32_t *d_piece_begin = nullptr;
  int64_t *d_piece_numel = nullptr;
  void *scratch = nullptr;         // one device allocation: tiles | tile_begin | numel | partials
  ob::Geometry geo{};
  double2 *partials = nullptr;     // (W+1) x num_tiles
  double2 *chunk_partials = nullptr;   // W x num_tiles * kChunksPerTile (chunked worker passes)
  void *static_scratch = nullptr;  // the device's static no-allocation scratch (null if unresolved)
  size_t static_need = 0;          // bytes of it the no-allocation step uses for this list
  bool profiling = false;
  bool launched = false;             // some kernel was enqueued, on last_stream the latest
  hipStream_t last_stream = nullptr;
  std::vector<EventPair> pending[ob::K_NUM_KINDS];
  std::vector<EventPair> pool;
};

namespace {

const char *const kKindNames[] = {
    "worker_pass1", "scale_finalize", "worker_pass2", "server_pass1",
    "server_pass2", "server_pass2_update", "apply_update", "worker_residual",
    "server_residual", "update_residual", "materialize", "warmup", "zero_errors",
    "trust_norms", "trust_ratio", "cltk_select", "cltk_gather", "cltk_average"};
static_assert(sizeof(kKindNames) / sizeof(kKindNames[0]) == ob::K_NUM_KINDS,
              "one name per kernel kind");

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Scratch sections start on 256-byte boundaries.
size_t scratch_bytes(size_t b) { return (b + 255) / 256 * 256; }

int check_ptr(const void *p) {
  if (p == nullptr) return OB_ERR_INVALID;
  if (!aligned16(p)) return OB_ERR_ALIGN;
  return OB_OK;
}

template <typename... P>
int check_ptrs(const P *...ps) {
  int st = OB_OK;
  const void *list[] = {static_cast<const void *>(ps)...};
  for (const void *p : list) {
    const int r = check_ptr(p);
    if (r == OB_ERR_INVALID) return r;
    if (r != OB_OK) st = r;
  }
  return st;
}

// Brackets one launch with events when profiling is on.  On a failure the
// event pair goes back to the pool.
template <typename F>
int timed(ob_ctx *c, ob::Kind kind, hipStream_t s, F &&launch, bool events = true) {
  EventPair ev;
  const bool profiling = events && c->profiling;
  if (profiling) {
    if (!c->pool.empty()) {
      ev = c->pool.back();
      c->pool.pop_back();
    } else {
      if (hipEventCreate(&ev.start) != hipSuccess) return OB_ERR_DEVICE;
      if (hipEventCreate(&ev.stop) != hipSuccess) {
        (void)hipEventDestroy(ev.start);
        return OB_ERR_DEVICE;
      }
    }
    if (hipEventRecord(ev.start, s) != hipSuccess) {
      c->pool.push_back(ev);
      return OB_ERR_DEVICE;
    }
  }
  launch();
  c->launched = true;
  c->last_stream = s;
  const bool launched = hipGetLastError() == hipSuccess;
  if (profiling) {
    if (!launched || hipEventRecord(ev.stop, s) != hipSuccess) {
      c->pool.push_back(ev);
      return OB_ERR_DEVICE;
    }
    c->pending[kind].push_back(ev);
  }
  return launched ? OB_OK : OB_ERR_DEVICE;
}

// Per-step scratch of one call: the context's own, or the static buffer of
// the no-allocation step.
struct StepScratch {
  double2 *partials;         // (W+1) x num_tiles
  double2 *chunk_partials;   // W x num_tiles * kChunksPerTile
  float *ratio;              // [T]
};

StepScratch own_scratch(ob_ctx *c) { return StepScratch{c->partials, c->chunk_partials, c->d_ratio}; }

ob::WorkerArgs worker_args(ob_ctx *c, int w0, int w1, const void *grads, const float *m,
                          float *err_w, uint64_t *packed_w, const float *scale_w,
                          const uint64_t *packed_s, const float *scale_s) {
  ob::WorkerArgs a{};
  a.grads = grads;
  a.m = m;
  a.err_w = err_w;
  a.packed_w = packed_w;
  a.scale_w = scale_w;
  a.packed_s = packed_s;
  a.scale_s = scale_s;
  a.partials = c->partials;
  a.chunk_partials = c->chunk_partials;
  a.w0 = w0;
  a.w1 = w1;
  a.wgroup = ob::worker_group_size(w1 - w0, c->num_tiles);
  a.c1 = c->c1;
  a.c2 = c->c2;
  return a;
}

ob::ServerArgs server_args(ob_ctx *c, const uint64_t *packed_w, const float *scale_w, float *err_s,
                          const float *scale_s, uint64_t *packed_s) {
  ob::ServerArgs a{};
  a.packed_w = packed_w;
  a.scale_w = scale_w;
  a.err_s = err_s;
  a.partials = c->partials;
  a.scale_s = scale_s;
  a.packed_s = packed_s;
  a.eps = c->eps;
  return a;
}

int do_compress(ob_ctx *c, int w0, int w1, const void *grads, const float *m, float *err_w,
                uint64_t *packed_w, float *scale_w, hipStream_t s) {
  const ob::Geometry &g = c->geo;
  const ob::WorkerArgs a = worker_args(c, w0, w1, grads, m, err_w, packed_w, scale_w, nullptr, nullptr);
  int st = timed(c, ob::K_WORKER_PASS1, s, [&] {
    ob::launch_worker(ob::WorkerPass::kStrictSigns, g, c->bf16, a, s);
  });
  if (st) return st;
  st = timed(c, ob::K_SCALE_FINALIZE, s, [&] {
    ob::launch_scale_finalize(g, c->partials, g.num_tiles, 1, w0, w1 - w0, g.tile_begin, g.numel, c->T,
                              scale_w + static_cast<size_t>(w0) * c->T, c->max_tensor_tiles, s);
  });
  if (st) return st;
  return timed(c, ob::K_WORKER_PASS2, s, [&] {
    ob::launch_worker(ob::WorkerPass::kStrictErrors, g, c->bf16, a, s);
  });
}

int do_server_first(ob_ctx *c, const uint64_t *packed_w, const float *scale_w, float *err_s,
                    float *scale_s, hipStream_t s) {
  const ob::Geometry &g = c->geo;
  const ob::ServerArgs a = server_args(c, packed_w, scale_w, err_s, nullptr, nullptr);
  int st = timed(c, ob::K_SERVER_PASS1, s, [&] {
    ob::launch_server(ob::ServerPass::kStrictSums, g, a, s);
  });
  if (st) return st;
  return timed(c, ob::K_SCALE_FINALIZE, s, [&] {
    ob::launch_scale_finalize(g, c->partials, g.num_tiles, 1, c->W, 1, g.piece_begin, g.piece_numel, c->S,
                              scale_s, c->max_piece_tiles, s);
  });
}

// The update from the server message: plain, or scaled per tensor by the
// trust ratio (two more launches: per-tile norms, per-tensor ratios).
int do_update(ob_ctx *c, bool store_m, ob::Kind kind, const uint64_t *packed_s,
              const float *scale_s, const float *v, float *m, float *params, double lr,
              hipStream_t s, const StepScratch &x, bool events = true) {
  const ob::UpdateArgs a{packed_s, scale_s, v, m, params, static_cast<float>(lr), c->eps,
                         x.ratio, c->weight_decay};
  if (c->trust_ratio) {
    int st = timed(c, ob::K_TRUST_NORMS, s, [&] { ob::launch_trust_norms(c->geo, a, x.partials, s); }, events);
    if (st) return st;
    st = timed(c, ob::K_TRUST_RATIO, s, [&] { ob::launch_trust_ratio(c->geo, x.partials, x.ratio, s); },
               events);
    if (st) return st;
  }
  return timed(c, kind, s, [&] { ob::launch_update(store_m, c->trust_ratio, c->geo, a, s); }, events);
}

// The residual-form step over the whole list with the given scratch; events
// = false records no timing events (the no-allocation step creates none).
int do_step_residual(ob_ctx *c, bool first, const void *grads, const float *m, const float *v,
                     float *params, float *err_w, float *err_s, uint64_t *packed_w, float *scale_w,
                     uint64_t *packed_s, float *scale_s, double lr, hipStream_t s, const StepScratch &x,
                     bool events) {
  const ob::Geometry &g = c->geo;
  // worker: x = (c1*m + c2*g) + e, with e and m formed from the previous step's residual form
  ob::WorkerArgs wa = worker_args(c, 0, c->W, grads, first ? m : nullptr, err_w, packed_w,
                                  scale_w, packed_s, scale_s);
  wa.partials = x.partials;
  wa.chunk_partials = x.chunk_partials;
  int r = timed(c, ob::K_WORKER_RESIDUAL, s, [&] {
    ob::launch_worker(first ? ob::WorkerPass::kResidualFirst : ob::WorkerPass::kResidual, g,
                      c->bf16, wa, s);
  }, events);
  if (r) return r;
  r = timed(c, ob::K_SCALE_FINALIZE, s, [&] {
    ob::launch_scale_finalize(g, x.chunk_partials, static_cast<int64_t>(g.num_tiles) * ob::kChunksPerTile,
                              ob::kChunksPerTile, 0, c->W, g.tile_begin, g.numel, c->T, scale_w,
                              static_cast<int64_t>(c->max_tensor_tiles) * ob::kChunksPerTile, s);
  }, events);
  if (r) return r;
  ob::ServerArgs sa = server_args(c, packed_w, scale_w, err_s, scale_s, packed_s);
  sa.partials = x.partials;
  r = timed(c, ob::K_SERVER_RESIDUAL, s, [&] {
    ob::launch_server(first ? ob::ServerPass::kResidualFirst : ob::ServerPass::kResidual, g, sa, s);
  }, events);
  if (r) return r;
  r = timed(c, ob::K_SCALE_FINALIZE, s, [&] {
    ob::launch_scale_finalize(g, x.partials, g.num_tiles, 1, c->W, 1, g.piece_begin, g.piece_numel, c->S,
                              scale_s, c->max_piece_tiles, s);
  }, events);
  if (r) return r;
  return do_update(c, false, ob::K_UPDATE_RESIDUAL, packed_s, scale_s, v, nullptr, params, lr, s, x, events);
}

// Server pieces for a C-way partitioned server: chunk j of tensor t is a run
// of q_t = ceil(k_t / C) of its k_t tiles (whole 8192-element tiles, the last
// run shorter), so tensor t has ceil(k_t / q_t) <= C pieces.  C = 1 gives one
// piece per tensor; any C at or above a tensor's tile count gives one piece
// per tile.  Builds the three tables on the host, then uploads them
// (synchronous copies).
struct PieceTables {
  std::vector<int32_t> tile_piece, piece_begin;
  std::vector<int64_t> piece_numel;
  int32_t max_piece = 0;
};

PieceTables build_pieces(const ob_ctx *c, int32_t chunks) {
  PieceTables pt;
  pt.tile_piece.resize(static_cast<size_t>(c->num_tiles));
  for (int32_t t = 0; t < c->T; ++t) {
    const int64_t k = c->tile_begin[t + 1] - c->tile_begin[t];
    const int64_t q = (k + chunks - 1) / chunks;   // int64: chunks may be up to INT32_MAX
    for (int64_t i = 0; i < k; i += q) {
      const int32_t piece = static_cast<int32_t>(pt.piece_begin.size());
      const int64_t end = std::min(i + q, k);
      pt.piece_begin.push_back(c->tile_begin[t] + static_cast<int32_t>(i));
      pt.piece_numel.push_back(std::min(end * ob::kTile, c->numel[t]) - i * ob::kTile);
      pt.max_piece = std::max(pt.max_piece, static_cast<int32_t>(end - i));
      for (int64_t j = i; j < end; ++j) pt.tile_piece[c->tile_begin[t] + j] = piece;
    }
  }
  pt.piece_begin.push_back(c->num_tiles);
  return pt;
}

int copy_pieces(ob_ctx *c, const PieceTables &pt) {
  if (hipMemcpy(c->d_tile_piece, pt.tile_piece.data(), pt.tile_piece.size() * sizeof(int32_t),
                hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(c->d_piece_begin, pt.piece_begin.data(), pt.piece_begin.size() * sizeof(int32_t),
                hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(c->d_piece_numel, pt.piece_numel.data(), pt.piece_numel.size() * sizeof(int64_t),
                hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipGetLastError();
    return OB_ERR_DEVICE;
  }
  return OB_OK;
}

// Switches the server to `chunks` pieces per tensor.  If an upload fails, the
// tables of the previous setting are uploaded again so the device tables and
// the host's counts keep agreeing; the call still reports the failure.
int upload_pieces(ob_ctx *c, int32_t chunks) {
  const int32_t eff = std::min(chunks, std::max<int32_t>(1, c->max_tensor_tiles));
  PieceTables pt;
  try {
    pt = build_pieces(c, eff);
  } catch (const std::bad_alloc &) {
    return OB_ERR_NOMEM;
  }
  if (copy_pieces(c, pt) != OB_OK) {
    if (c->S > 0) {   // a configured context: restore what it held
      try {
        (void)copy_pieces(c, build_pieces(c, c->server_chunks));
      } catch (const std::bad_alloc &) {
      }
    }
    return OB_ERR_DEVICE;
  }
  c->server_chunks = eff;
  c->max_piece_tiles = pt.max_piece;
  c->S = static_cast<int32_t>(pt.piece_numel.size());
  c->geo.S = c->S;
  return OB_OK;
}

// Waits for the work this context last enqueued (the stream of its latest
// launch) before its tables are rewritten; nothing else on the device waits.
int wait_for_last_launch(ob_ctx *c) {
  if (!c->launched) return OB_OK;
  return hipStreamSynchronize(c->last_stream) == hipSuccess ? OB_OK : OB_ERR_DEVICE;
}

}  // namespace

extern "C" {

const char *ob_status_string(int status) {
  switch (status) {
    case OB_OK: return "ok";
    case OB_ERR_INVALID: return "invalid argument";
    case OB_ERR_ALIGN: return "device pointer not aligned to 16 bytes";
    case OB_ERR_NOMEM: return "out of memory";
    case OB_ERR_DEVICE: return "HIP runtime or launch failure";
    case OB_ERR_SCRATCH:
      return "the tensor list needs more scratch than the 64 MiB static buffer of ob_step_residual_noalloc";
    default: return "unknown status";
  }
}

int ob_layout(int32_t num_tensors, const int64_t *numel, int64_t *elem_off) {
  if (num_tensors < 1 || numel == nullptr || elem_off == nullptr) return OB_ERR_INVALID;
  int64_t off = 0;
  for (int32_t t = 0; t < num_tensors; ++t) {
    if (numel[t] < 1 || numel[t] > (int64_t{1} << 40)) return OB_ERR_INVALID;
  }
  for (int32_t t = 0; t < num_tensors; ++t) {
    elem_off[t] = off;
    off += (numel[t] + 63) / 64 * 64;
  }
  elem_off[num_tensors] = off;
  return OB_OK;
}

int ob_init(ob_ctx **out, int32_t num_tensors, const int64_t *numel, int32_t num_workers,
            int32_t grad_dtype, double beta1, double eps) {
  if (out == nullptr) return OB_ERR_INVALID;
  *out = nullptr;
  if (num_workers < 1 || num_workers > 4096) return OB_ERR_INVALID;
  if (grad_dtype != OB_GRAD_F32 && grad_dtype != OB_GRAD_BF16) return OB_ERR_INVALID;
  if (!std::isfinite(beta1) || beta1 < 0.0 || beta1 >= 1.0) return OB_ERR_INVALID;
  if (!std::isfinite(eps) || !(static_cast<float>(eps) > 0.0f)) return OB_ERR_INVALID;   // eps > 0 in fp32
  std::vector<int64_t> off(static_cast<size_t>(num_tensors > 0 ? num_tensors : 0) + 1);
  const int lay = ob_layout(num_tensors, numel, off.data());
  if (lay != OB_OK) return lay;

  ob_ctx *c = new (std::nothrow) ob_ctx();
  if (c == nullptr) return OB_ERR_NOMEM;
  c->T = num_tensors;
  c->W = num_workers;
  c->bf16 = grad_dtype == OB_GRAD_BF16;
  c->c1 = static_cast<float>(beta1);
  c->c2 = static_cast<float>(1.0 - beta1);
  c->eps = static_cast<float>(eps);
  c->numel.assign(numel, numel + num_tensors);
  c->off = off;
  c->N = off[num_tensors];

  // The largest launches must fit the device's grid limit: (worker group,
  // tile) workgroups of the tiled worker passes, the chunks of one worker
  // (the chunked passes put workers along y, or split their worker-fastest
  // grids into runs of workers that fit), and the scale finalize's up to one
  // workgroup per (worker, tensor).
  int64_t nt = 0;
  for (int32_t t = 0; t < num_tensors; ++t) nt += (numel[t] + ob::kTile - 1) / ob::kTile;
  if (nt * ob::kChunksPerTile > ob::kMaxGrid) {
    delete c;
    return OB_ERR_INVALID;
  }
  const int64_t wgroup = ob::worker_group_size(num_workers, static_cast<int>(nt));
  const int64_t finalize = static_cast<int64_t>(num_workers) * num_tensors;
  if (nt * ((num_workers + wgroup - 1) / wgroup) > ob::kMaxGrid || finalize > ob::kMaxGrid) {
    delete c;
    return OB_ERR_INVALID;
  }

  std::vector<ob::Tile> tiles;
  tiles.reserve(static_cast<size_t>(nt));
  std::vector<int32_t> tile_begin(static_cast<size_t>(num_tensors) + 1);
  for (int32_t t = 0; t < num_tensors; ++t) {
    tile_begin[t] = static_cast<int32_t>(tiles.size());
    for (int64_t k = 0; k < numel[t]; k += ob::kTile) {
      const int64_t len = numel[t] - k < ob::kTile ? numel[t] - k : ob::kTile;
      tiles.push_back(ob::Tile{off[t] + k, static_cast<int32_t>(len), t});
    }
  }
  tile_begin[num_tensors] = static_cast<int32_t>(tiles.size());
  c->num_tiles = static_cast<int32_t>(tiles.size());
  c->tile_begin = tile_begin;
  for (int32_t t = 0; t < num_tensors; ++t)
    c->max_tensor_tiles = std::max(c->max_tensor_tiles, tile_begin[t + 1] - tile_begin[t]);

  // one allocation, 256-byte aligned sections
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const size_t b_tiles = up(tiles.size() * sizeof(ob::Tile));
  const size_t b_begin = up(tile_begin.size() * sizeof(int32_t));
  const size_t b_numel = up(c->numel.size() * sizeof(int64_t));
  // server-piece tables, sized for the most pieces (one per tile)
  const size_t b_tpiece = up(tiles.size() * sizeof(int32_t));
  const size_t b_pbegin = up((tiles.size() + 1) * sizeof(int32_t));
  const size_t b_pnumel = up(tiles.size() * sizeof(int64_t));
  const size_t b_pieces = b_tpiece + b_pbegin + b_pnumel;
  const size_t b_ratio = up(c->numel.size() * sizeof(float));
  const size_t b_part =
      up(ob::partials_count(num_workers, static_cast<int>(tiles.size())) * sizeof(double2));
  const size_t b_cpart =
      up(ob::chunk_partials_count(num_workers, static_cast<int>(tiles.size())) * sizeof(double2));
  std::vector<unsigned char> host(b_tiles + b_begin + b_numel, 0);
  std::copy(reinterpret_cast<const unsigned char *>(tiles.data()),
            reinterpret_cast<const unsigned char *>(tiles.data() + tiles.size()), host.data());
  std::copy(reinterpret_cast<const unsigned char *>(tile_begin.data()),
            reinterpret_cast<const unsigned char *>(tile_begin.data() + tile_begin.size()),
            host.data() + b_tiles);
  std::copy(reinterpret_cast<const unsigned char *>(c->numel.data()),
            reinterpret_cast<const unsigned char *>(c->numel.data() + c->numel.size()),
            host.data() + b_tiles + b_begin);
  if (hipMalloc(&c->scratch, host.size() + b_pieces + b_ratio + b_part + b_cpart) != hipSuccess) {
    (void)hipGetLastError();
    delete c;
    return OB_ERR_NOMEM;
  }
  if (hipMemcpy(c->scratch, host.data(), host.size(), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(c->scratch);
    delete c;
    return OB_ERR_DEVICE;
  }
  unsigned char *base = static_cast<unsigned char *>(c->scratch);
  c->geo.tiles = reinterpret_cast<const ob::Tile *>(base);
  c->geo.tile_begin = reinterpret_cast<const int32_t *>(base + b_tiles);
  c->geo.numel = reinterpret_cast<const int64_t *>(base + b_tiles + b_begin);
  unsigned char *pieces = base + b_tiles + b_begin + b_numel;
  c->d_tile_piece = reinterpret_cast<int32_t *>(pieces);
  c->d_piece_begin = reinterpret_cast<int32_t *>(pieces + b_tpiece);
  c->d_piece_numel = reinterpret_cast<int64_t *>(pieces + b_tpiece + b_pbegin);
  c->geo.tile_piece = c->d_tile_piece;
  c->geo.piece_begin = c->d_piece_begin;
  c->geo.piece_numel = c->d_piece_numel;
  c->d_ratio = reinterpret_cast<float *>(pieces + b_pieces);
  c->partials = reinterpret_cast<double2 *>(pieces + b_pieces + b_ratio);
  c->chunk_partials = reinterpret_cast<double2 *>(pieces + b_pieces + b_ratio + b_part);
  c->geo.num_tiles = c->num_tiles;
  c->geo.T = c->T;
  c->geo.W = c->W;
  c->geo.N = c->N;
  c->geo.Nw = c->N / 64;
  // the no-allocation step's static scratch on this device, and what this list needs of it
  c->static_need = b_part + b_cpart + b_ratio;
  if (ob::static_scratch_address(&c->static_scratch) != hipSuccess) {
    (void)hipGetLastError();
    c->static_scratch = nullptr;   // ob_step_residual_noalloc then reports OB_ERR_DEVICE
  }
  const int pr = upload_pieces(c, 1);
  if (pr != OB_OK) {
    (void)hipFree(c->scratch);
    delete c;
    return pr;
  }
  *out = c;
  return OB_OK;
}

void ob_destroy(ob_ctx *c) {
  if (c == nullptr) return;
  for (auto &v : c->pending)
    for (auto &e : v) c->pool.push_back(e);
  for (auto &e : c->pool) {
    if (e.start) (void)hipEventDestroy(e.start);
    if (e.stop) (void)hipEventDestroy(e.stop);
  }
  if (c->scratch) (void)hipFree(c->scratch);
  if (c->topk_scratch) (void)hipFree(c->topk_scratch);
  delete c;
}

int ob_compress_worker(ob_ctx *c, int32_t w_begin, int32_t w_end, const void *grads,
                       const float *m, float *err_w, uint64_t *packed_w, float *scale_w,
                       void *stream) {
  if (c == nullptr) return OB_ERR_INVALID;
  if (w_begin < 0 || w_end > c->W || w_begin >= w_end) return OB_ERR_INVALID;
  const int st = check_ptrs(grads, m, err_w, packed_w, scale_w);
  if (st) return st;
  return do_compress(c, w_begin, w_end, grads, m, err_w, packed_w, scale_w,
                     static_cast<hipStream_t>(stream));
}

int ob_server_reduce(ob_ctx *c, const uint64_t *packed_w, const float *scale_w, float *err_s,
                     uint64_t *packed_s, float *scale_s, void *stream) {
  if (c == nullptr) return OB_ERR_INVALID;
  const int st = check_ptrs(packed_w, scale_w, err_s, packed_s, scale_s);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int r = do_server_first(c, packed_w, scale_w, err_s, scale_s, s);
  if (r) return r;
  const ob::ServerArgs a = server_args(c, packed_w, scale_w, err_s, scale_s, packed_s);
  return timed(c, ob::K_SERVER_PASS2, s, [&] {
    ob::launch_server(ob::ServerPass::kStrictErrors, c->geo, a, s);
  });
}

int ob_apply_update(ob_ctx *c, const uint64_t *packed_s, const float *scale_s, const float *v,
                    float *m, float *params, double lr, void *stream) {
  if (c == nullptr || !std::isfinite(lr)) return OB_ERR_INVALID;
  const int st = check_ptrs(packed_s, scale_s, v, m, params);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return do_update(c, true, ob::K_APPLY_UPDATE, packed_s, scale_s, v, m, params, lr, s, own_scratch(c));
}

int ob_step(ob_ctx *c, const void *grads, float *m, const float *v, float *params, float *err_w,
            float *err_s, uint64_t *packed_w, float *scale_w, uint64_t *packed_s, float *scale_s,
            double lr, void *stream) {
  if (c == nullptr || !std::isfinite(lr)) return OB_ERR_INVALID;
  const int st = check_ptrs(grads, m, v, params, err_w, err_s, packed_w, scale_w, packed_s, scale_s);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int r = do_compress(c, 0, c->W, grads, m, err_w, packed_w, scale_w, s);
  if (r) return r;
  r = do_server_first(c, packed_w, scale_w, err_s, scale_s, s);
  if (r) return r;
  if (c->trust_ratio) {   // the ratio needs the whole tensor's update: no fusion
    const ob::ServerArgs a = server_args(c, packed_w, scale_w, err_s, scale_s, packed_s);
    r = timed(c, ob::K_SERVER_PASS2, s, [&] {
      ob::launch_server(ob::ServerPass::kStrictErrors, c->geo, a, s);
    });
    if (r) return r;
    return do_update(c, true, ob::K_APPLY_UPDATE, packed_s, scale_s, v, m, params, lr, s, own_scratch(c));
  }
  ob::ServerArgs a = server_args(c, packed_w, scale_w, err_s, scale_s, packed_s);
  a.v = v;
  a.m = m;
  a.params = params;
  a.lr = static_cast<float>(lr);
  return timed(c, ob::K_SERVER_PASS2_UPDATE, s, [&] {
    ob::launch_server(ob::ServerPass::kStrictErrorsUpdate, c->geo, a, s);
  });
}

int ob_step_residual(ob_ctx *c, int32_t first, const void *grads, const float *m, const float *v,
                     float *params, float *err_w, float *err_s, uint64_t *packed_w, float *scale_w,
                     uint64_t *packed_s, float *scale_s, double lr, void *stream) {
  if (c == nullptr || !std::isfinite(lr)) return OB_ERR_INVALID;
  int st = check_ptrs(grads, v, params, err_w, err_s, packed_w, scale_w, packed_s, scale_s);
  if (st) return st;
  if (first && (st = check_ptr(m)) != OB_OK) return st;
  return do_step_residual(c, first != 0, grads, m, v, params, err_w, err_s, packed_w, scale_w, packed_s,
                          scale_s, lr, static_cast<hipStream_t>(stream), own_scratch(c), true);
}

int ob_step_residual_noalloc(ob_ctx *c, int32_t first, const void *grads, const float *m, const float *v,
                             float *params, float *err_w, float *err_s, uint64_t *packed_w, float *scale_w,
                             uint64_t *packed_s, float *scale_s, double lr, void *stream) {
  if (c == nullptr || !std::isfinite(lr)) return OB_ERR_INVALID;
  int st = check_ptrs(grads, v, params, err_w, err_s, packed_w, scale_w, packed_s, scale_s);
  if (st) return st;
  if (first && (st = check_ptr(m)) != OB_OK) return st;
  if (c->static_need > ob::kStaticScratchBytes) return OB_ERR_SCRATCH;
  if (c->static_scratch == nullptr) return OB_ERR_DEVICE;   // the address lookup at ob_init failed
  // the static buffer, laid out as the context's scratch: partials | chunk partials | ratios
  unsigned char *base = static_cast<unsigned char *>(c->static_scratch);
  const size_t b_part = scratch_bytes(ob::partials_count(c->W, c->num_tiles) * sizeof(double2));
  const size_t b_cpart = scratch_bytes(ob::chunk_partials_count(c->W, c->num_tiles) * sizeof(double2));
  const StepScratch x{reinterpret_cast<double2 *>(base), reinterpret_cast<double2 *>(base + b_part),
                      reinterpret_cast<float *>(base + b_part + b_cpart)};
  return do_step_residual(c, first != 0, grads, m, v, params, err_w, err_s, packed_w, scale_w, packed_s,
                          scale_s, lr, static_cast<hipStream_t>(stream), x, false);
}

int ob_materialize(ob_ctx *c, const float *x_w, const float *scale_w, const float *z,
                   const float *scale_s, float *err_w, float *err_s, float *m, void *stream) {
  if (c == nullptr) return OB_ERR_INVALID;
  const int st = check_ptrs(x_w, scale_w, z, scale_s, err_w, err_s, m);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ob::MaterializeArgs a{x_w, scale_w, z, scale_s, err_w, err_s, m};
  return timed(c, ob::K_MATERIALIZE, s, [&] { ob::launch_materialize(c->geo, a, s); });
}

int ob_warmup_step(ob_ctx *c, const void *grads, float *m, float *v, float *params, double beta2,
                   double lr, void *stream) {
  if (c == nullptr || !std::isfinite(lr)) return OB_ERR_INVALID;
  if (!std::isfinite(beta2) || beta2 < 0.0 || beta2 >= 1.0) return OB_ERR_INVALID;
  const int st = check_ptrs(grads, m, v, params);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ob::WarmupArgs a{grads, m, v, params, c->c1, c->c2, static_cast<float>(beta2),
                         static_cast<float>(1.0 - beta2), static_cast<float>(lr), c->eps};
  return timed(c, ob::K_WARMUP, s, [&] { ob::launch_warmup(c->geo, c->bf16, a, s); });
}

int ob_begin_compression(ob_ctx *c, float *err_w, float *err_s, void *stream) {
  if (c == nullptr) return OB_ERR_INVALID;
  const int st = check_ptrs(err_w, err_s);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(c, ob::K_ZERO_ERRORS, s, [&] { ob::launch_zero_errors(c->geo, err_w, err_s, s); });
}

int ob_set_server_chunks(ob_ctx *c, int32_t chunks) {
  if (c == nullptr || chunks < 1) return OB_ERR_INVALID;
  if (wait_for_last_launch(c) != OB_OK) return OB_ERR_DEVICE;   // the tables may be in use
  return upload_pieces(c, chunks);
}

int32_t ob_server_scale_count(const ob_ctx *c) { return c == nullptr ? -1 : c->S; }

int ob_set_trust_ratio(ob_ctx *c, int32_t enable, double weight_decay) {
  if (c == nullptr || !std::isfinite(weight_decay) || weight_decay < 0.0) return OB_ERR_INVALID;
  c->trust_ratio = enable != 0;
  c->weight_decay = static_cast<float>(weight_decay);
  return OB_OK;
}

int ob_cltk_configure(ob_ctx *c, double density, int64_t *k_total) {
  if (c == nullptr || !std::isfinite(density) || density <= 0.0 || density > 1.0)
    return OB_ERR_INVALID;
  for (int32_t t = 0; t < c->T; ++t)   // index entries are int32 positions within a tensor
    if (c->numel[t] > INT32_MAX) return OB_ERR_INVALID;
  if (wait_for_last_launch(c) != OB_OK) return OB_ERR_DEVICE;   // the old tables may be in use
  std::vector<int64_t> k_off(static_cast<size_t>(c->T) + 1, 0);
  for (int32_t t = 0; t < c->T; ++t) {
    const int64_t k = std::max<int64_t>(1, static_cast<int64_t>(std::ceil(density * static_cast<double>(c->numel[t]))));
    k_off[t + 1] = k_off[t] + std::min(k, c->numel[t]);
  }
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const size_t T = static_cast<size_t>(c->T), tiles = static_cast<size_t>(c->num_tiles);
  const size_t nw = static_cast<size_t>(c->N / 64);
  const size_t sizes[] = {up((T + 1) * 8), up(T * 2048 * 4), up(T * 4),     up(T * 4),
                          up(tiles * 4),     up(tiles * 4),    up(tiles * 8), up(tiles * 8),
                          up(T * 4),         up(nw * 64 * 4),  up(tiles * 4), up(nw * 64 * 2),
                          up(nw * 8),        up(T * 4)};
  size_t total = 0;
  for (size_t b : sizes) total += b;
  if (c->topk_scratch) {
    (void)hipFree(c->topk_scratch);
    c->topk_scratch = nullptr;
  }
  if (hipMalloc(&c->topk_scratch, total) != hipSuccess) {
    (void)hipGetLastError();
    return OB_ERR_NOMEM;
  }
  unsigned char *p = static_cast<unsigned char *>(c->topk_scratch);
  ob::TopkArgs &a = c->topk;
  a = ob::TopkArgs{};
  constexpr int kSections = sizeof(sizes) / sizeof(sizes[0]);
  unsigned char *at[kSections];
  for (int i = 0; i < kSections; ++i) {
    at[i] = p;
    p += sizes[i];
  }
  a.k_off = reinterpret_cast<const int64_t *>(at[0]);
  a.hist = reinterpret_cast<uint32_t *>(at[1]);
  a.prefix = reinterpret_cast<uint32_t *>(at[2]);
  a.krem = reinterpret_cast<uint32_t *>(at[3]);
  a.tile_gt = reinterpret_cast<uint32_t *>(at[4]);
  a.tile_eq = reinterpret_cast<uint32_t *>(at[5]);
  a.tile_eq_before = reinterpret_cast<int64_t *>(at[6]);
  a.tile_sel_off = reinterpret_cast<int64_t *>(at[7]);
  a.pred = reinterpret_cast<uint32_t *>(at[8]);
  a.cand = reinterpret_cast<uint32_t *>(at[9]);
  a.tile_m = reinterpret_cast<uint32_t *>(at[10]);
  a.cand_pos = reinterpret_cast<uint16_t *>(at[11]);
  a.above = reinterpret_cast<uint64_t *>(at[12]);
  a.miss = reinterpret_cast<uint32_t *>(at[13]);
  a.K = k_off[T];
  const std::vector<uint32_t> no_prediction(T, 0xffffffffu);   // the first exchange has none
  if (hipMemcpy(at[0], k_off.data(), (T + 1) * 8, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(at[8], no_prediction.data(), T * 4, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(c->topk_scratch);   // leave the codec unconfigured
    c->topk_scratch = nullptr;
    return OB_ERR_DEVICE;
  }
  c->k_off = k_off;
  if (k_total) *k_total = a.K;
  return OB_OK;
}

int ob_cltk_layout(const ob_ctx *c, int64_t *k_off) {
  if (c == nullptr || k_off == nullptr || c->topk_scratch == nullptr) return OB_ERR_INVALID;
  std::copy(c->k_off.begin(), c->k_off.end(), k_off);
  return OB_OK;
}

int ob_cltk_step(ob_ctx *c, int64_t step, const void *grads, float *memory, int32_t *index,
                 float *values, float *average, void *stream) {
  if (c == nullptr || c->topk_scratch == nullptr || step < 0) return OB_ERR_INVALID;
  const int st = check_ptrs(grads, memory, index, values, average);
  if (st) return st;
  ob::TopkArgs a = c->topk;
  a.grads = grads;
  a.memory = memory;
  a.index = index;
  a.values = values;
  a.average = average;
  a.leader = static_cast<int>(step % c->W);
  a.wgroup = ob::worker_group_size(c->W, c->num_tiles);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st2 = timed(c, ob::K_TOPK_SELECT, s,
                  [&] { ob::launch_topk(ob::TopkStage::kSelect, c->geo, c->bf16, a, s); });
  if (st2 == OB_OK)
    st2 = timed(c, ob::K_TOPK_GATHER, s,
                [&] { ob::launch_topk(ob::TopkStage::kGather, c->geo, c->bf16, a, s); });
  if (st2 == OB_OK)
    st2 = timed(c, ob::K_TOPK_AVERAGE, s,
                [&] { ob::launch_topk(ob::TopkStage::kAverage, c->geo, c->bf16, a, s); });
  return st2;
}

int ob_profile_enable(ob_ctx *c, int32_t enable) {
  if (c == nullptr) return OB_ERR_INVALID;
  c->profiling = enable != 0;
  return OB_OK;
}

int32_t ob_profile_kinds(void) { return ob::K_NUM_KINDS; }

const char *ob_profile_kind_name(int32_t kind) {
  if (kind < 0 || kind >= ob::K_NUM_KINDS) return nullptr;
  return kKindNames[kind];
}

int ob_profile_read(ob_ctx *c, double *total_ms, int64_t *launches, int32_t reset) {
  if (c == nullptr || total_ms == nullptr || launches == nullptr) return OB_ERR_INVALID;
  for (int k = 0; k < ob::K_NUM_KINDS; ++k) {
    double sum = 0.0;
    for (auto &e : c->pending[k]) {
      float ms = 0.0f;
      if (hipEventSynchronize(e.stop) != hipSuccess) return OB_ERR_DEVICE;
      if (hipEventElapsedTime(&ms, e.start, e.stop) != hipSuccess) return OB_ERR_DEVICE;
      sum += ms;
    }
    total_ms[k] = sum;
    launches[k] = static_cast<int64_t>(c->pending[k].size());
    if (reset) {
      for (auto &e : c->pending[k]) c->pool.push_back(e);
      c->pending[k].clear();
    }
  }
  return OB_OK;
}

}  // extern "C"
