// Host build of the kernels' launch-grid arithmetic for a CPU test.
#include "../weight_communication_compression_amd/csrc/grid.hpp"

extern "C" long long lowbit_test_grid_blocks(long long ntrips, int threads) {
  return (long long)lowbit::grid_blocks((int64_t)ntrips, threads);
}
