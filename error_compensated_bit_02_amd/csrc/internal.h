// Internal declarations shared by the host library (api.cpp) and the HIP
// kernels (kernels.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ob {

// One workgroup handles one tile: kTile consecutive elements of one tensor
// (a tensor's last tile may be shorter; no tile spans two tensors).  Each of
// the kWaves wavefronts owns kSub consecutive elements of the tile, and lane
// l of a wavefront owns element 64*c + l of its range for c < kPerLane, so a
// wavefront-wide ballot over one c yields one packed sign word in natural
// bit order.
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kTile = 8192;
constexpr int kSub = kTile / kWaves;
constexpr int kPerLane = kSub / 64;

struct Tile {
  int64_t start;   // first element of the tile in the flat layout
  int32_t len;     // elements in the tile (1..kTile)
  int32_t tensor;  // tensor the tile belongs to
};

// Device-side description of a tensor list.
struct Geometry {
  const Tile *tiles;
  const int32_t *tile_begin;  // [T+1]: tiles of tensor t are tile_begin[t] .. tile_begin[t+1]-1
  const int64_t *numel;       // [T]
  int32_t num_tiles;
  int32_t T;
  int32_t W;
  int64_t N;                  // padded elements per flat buffer row
  int64_t Nw;                 // N / 64 sign words per packed row
};

enum Kind {
  K_WORKER_PASS1 = 0,
  K_SCALE_FINALIZE,
  K_WORKER_PASS2,
  K_SERVER_PASS1,
  K_SERVER_PASS2,
  K_SERVER_PASS2_UPDATE,
  K_APPLY_UPDATE,
  K_NUM_KINDS
};

// Kernel launchers (kernels.hip).  partials holds (W+1) rows of num_tiles
// compensated fp64 sums (hi, lo): rows 0..W-1 for workers, row W for the server.
void launch_worker_pass1(const Geometry &g, bool bf16, int w0, int w1, const void *grads,
                         const float *m, const float *err_w, uint64_t *packed_w,
                         double2 *partials, float c1, float c2, hipStream_t s);
void launch_scale_finalize(const Geometry &g, const double2 *partials, int row0, int nrows,
                           float *out, hipStream_t s);
void launch_worker_pass2(const Geometry &g, bool bf16, int w0, int w1, const void *grads,
                         const float *m, float *err_w, const float *scale_w, float c1, float c2,
                         hipStream_t s);
void launch_server_pass1(const Geometry &g, const uint64_t *packed_w, const float *scale_w,
                         const float *err_s, double2 *partials, hipStream_t s);
// update == false: writes err_s and packed_s only; update == true: also m and params.
void launch_server_pass2(const Geometry &g, bool update, const uint64_t *packed_w,
                         const float *scale_w, float *err_s, const float *scale_s,
                         uint64_t *packed_s, const float *v, float *m, float *params, float lr,
                         float eps, hipStream_t s);
void launch_apply_update(const Geometry &g, const uint64_t *packed_s, const float *scale_s,
                         const float *v, float *m, float *params, float lr, float eps,
                         hipStream_t s);

}  // namespace ob
