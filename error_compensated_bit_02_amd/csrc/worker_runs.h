// Splitting a worker-fastest launch (one workgroup per (chunk, worker),
// workers fastest) into runs of workers whose grids each fit the device's
// grid limit.  Plain C++ so that the host tests can check it.
#pragma once

#include <cstdint>

namespace ob {

// Calls f(b0, b1) for consecutive runs [b0, b1) covering [w0, w1) in
// ascending order, each with chunks * (b1 - b0) <= max_grid.  Requires
// 1 <= chunks <= max_grid.
template <typename F>
inline void worker_runs(int w0, int w1, int64_t chunks, int64_t max_grid, F f) {
  const int64_t per = max_grid / chunks;   // >= 1
  for (int b0 = w0; b0 < w1;) {
    const int b1 = static_cast<int>(w1 - b0 <= per ? w1 : b0 + per);
    f(b0, b1);
    b0 = b1;
  }
}

}  // namespace ob
