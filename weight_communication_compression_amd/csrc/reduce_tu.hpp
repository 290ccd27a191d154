// reduce_tu.hpp -- launch helpers for the local-reduce kernels; each
// translation unit instantiates one family (same width, same width with a
// residual, mixed widths).
#pragma once

#include "launch.hpp"
#include "reduce.hpp"
#include "rowr.hpp"

namespace lowbit {

// 4-bit same-width reduce in the row layout when a binary32 stream is part
// of it (the stage-2 residual or the sum output) and blocks are at most 1024
// elements.  8 x 32 Mi peers, row layout against the general tile, with the
// residual / with the sum: B128 68.6 / 56.0 against 77.4 / 68.2 us, B512
// 67.7 / 54.7 against 78.3 / 67.6, B1024 67.2 / 53.2 against 76.8 / 62.7,
// B2048 101 / 65 against 74 / 62, B4096 163 / 99 against 84 / 77 (a trip of
// B/256 rows holds few peers' loads in flight).  The plain reduce keeps the
// general tile (40 -> 49 us in the row layout, where two lanes load each
// code word and every lane its scale; at 2 bits 33 -> 58 us).
template <int BITS, int LOG2B, bool SR, bool EF>
static lowbit_status launch_rr(bool stream_input, const ReduceArgs& a, hipStream_t s) {
  using S = RowrShape<BITS, LOG2B, EF>;
  const int64_t full_trips = a.n / S::TILE;
  lowbit_status st = LOWBIT_OK;
  if (full_trips > 0) {
    const int64_t grid = grid_for_tiles(full_trips);
    st = stream_input
             ? launch(&rowr_kernel<BITS, LOG2B, SR, EF, false, true>, grid, kBlockThreads, s, a,
                      full_trips)
             : launch(&rowr_kernel<BITS, LOG2B, SR, EF, false>, grid, kBlockThreads, s, a,
                      full_trips);
  }
  if (st == LOWBIT_OK && full_trips * S::TILE < a.n)
    st = launch(&rowr_kernel<BITS, LOG2B, SR, EF, true>, 1, kWave, s, a, full_trips);
  return st;
}

// Main kernel over the complete trips of full tiles; one-wave tail kernel for
// whatever remains.  stream_input: the main kernel reads the peers' code
// words non-temporally.  (In a step that decompresses those same codes right
// after the reduce, normal loads keep them in the Infinity Cache for it:
// 8 Mi shares at 1-8 bits, the four decompresses 7-16 % slower after
// streaming reduces.)
template <int IN_BITS, int BITS, int LOG2B, bool SR, bool EF>
static lowbit_status launch_r(bool stream_input, const ReduceArgs& a, hipStream_t s) {
  if constexpr (IN_BITS == BITS && BITS == 4 && LOG2B <= 10) {
    if (EF || a.out_sum) return launch_rr<BITS, LOG2B, SR, EF>(stream_input, a, s);
  }
  {
    using S = TileShape<BITS, LOG2B>;
    constexpr int U = reduce_tiles_per_trip<S::R * S::E>();
    const int64_t full_tiles = a.n / S::TILE;
    const int64_t ntrips = full_tiles / U;
    lowbit_status st = LOWBIT_OK;
    if (ntrips > 0) {
      const int64_t grid = grid_for_tiles(ntrips);
      st = stream_input ? launch(&reduce_kernel<IN_BITS, BITS, LOG2B, SR, EF, false, true>, grid,
                                 kBlockThreads, s, a, full_tiles)
                        : launch(&reduce_kernel<IN_BITS, BITS, LOG2B, SR, EF, false>, grid,
                                 kBlockThreads, s, a, full_tiles);
    }
    if (st == LOWBIT_OK && ntrips * U * S::TILE < a.n)
      st = launch(&reduce_kernel<IN_BITS, BITS, LOG2B, SR, EF, true>, 1, kWave, s, a, ntrips * U);
    return st;
  }
}

// stochastic rounding does not apply to a 1-bit output
template <int IN_BITS, int BITS, bool EF>
static lowbit_status launch_r_b(int log2b, bool sr, bool si, const ReduceArgs& a,
                                hipStream_t s) {
  switch (log2b) {
#define LOWBIT_CASE(LB)                                                             \
  case LB:                                                                          \
    return (BITS > 1 && sr) ? launch_r<IN_BITS, BITS, LB, (BITS > 1), EF>(si, a, s) \
                            : launch_r<IN_BITS, BITS, LB, false, EF>(si, a, s);
    LOWBIT_FOR_EACH_LOG2B(LOWBIT_CASE)
#undef LOWBIT_CASE
  }
  return LOWBIT_EUNSUPPORTED;
}

}  // namespace lowbit
