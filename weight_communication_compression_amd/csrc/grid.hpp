// grid.hpp -- launch-grid arithmetic of the codec kernels.  Host-only integer
// code with no HIP dependency, so that a CPU test can check it.
#pragma once

#include <stdint.h>

namespace lowbit {

// HIP limits the work-items of one grid dimension to 2^32 - 1.
constexpr int64_t kMaxGridItems = ((int64_t)1 << 32) - 1;

// Workgroups for `ntrips` units of work at one wave per unit, `threads`
// threads (threads / 64 waves) per workgroup: enough for one trip per wave,
// capped so that blocks * threads stays within kMaxGridItems (the kernels walk
// whatever lies beyond the grid in a grid-stride loop), and at least 1.
inline int64_t grid_blocks(int64_t ntrips, int threads) {
  const int64_t waves_per_block = threads / 64;
  int64_t blocks = ntrips > 0 ? (ntrips + waves_per_block - 1) / waves_per_block : 1;
  const int64_t cap = kMaxGridItems / threads;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return blocks;
}

}  // namespace lowbit
