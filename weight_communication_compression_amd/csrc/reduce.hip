// local reduce + requantize kernels
#include "launch.hpp"
#include "reduce.hpp"

namespace lowbit {

// Main kernel over the complete trips of full tiles; one-wave tail kernel for
// whatever remains.
template <int BITS, int LOG2B, bool SR>
static lowbit_status launch_r(const ReduceArgs& a, hipStream_t s) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int U = reduce_tiles_per_trip<S::R * S::E>();
  const int64_t full_tiles = a.n / S::TILE;
  const int64_t ntrips = full_tiles / U;
  if (ntrips > 0) {
    hipLaunchKernelGGL((reduce_kernel<BITS, LOG2B, SR, false>), dim3(grid_for_tiles(ntrips)),
                       dim3(kBlockThreads), 0, s, a, full_tiles);
  }
  if (ntrips * U * S::TILE < a.n) {
    hipLaunchKernelGGL((reduce_kernel<BITS, LOG2B, SR, true>), dim3(1), dim3(kWave), 0, s, a,
                       ntrips * U);
  }
  return launch_status();
}

template <int BITS>
static lowbit_status launch_r_b(int log2b, bool sr, const ReduceArgs& a, hipStream_t s) {
  switch (log2b) {
#define LOWBIT_CASE(LB)                                                       \
  case LB:                                                                    \
    return (BITS > 1 && sr) ? launch_r<BITS, LB, (BITS > 1)>(a, s)            \
                            : launch_r<BITS, LB, false>(a, s);
    LOWBIT_FOR_EACH_LOG2B(LOWBIT_CASE)
#undef LOWBIT_CASE
  }
  return LOWBIT_EUNSUPPORTED;
}

lowbit_status launch_reduce(int bits, int log2b, bool sr, const ReduceArgs& a, hipStream_t s) {
  switch (bits) {
    case 1: return launch_r_b<1>(log2b, sr, a, s);
    case 2: return launch_r_b<2>(log2b, sr, a, s);
    case 4: return launch_r_b<4>(log2b, sr, a, s);
    case 8: return launch_r_b<8>(log2b, sr, a, s);
  }
  return LOWBIT_EUNSUPPORTED;
}

}  // namespace lowbit
