// quantize_tu.hpp -- one translation unit's worth of compress-kernel
// instantiations for the mode LOWBIT_TU_MODE, exposed through the launcher
// LOWBIT_TU_LAUNCHER(bits, log2b, sr, dtype, args, stream).
#pragma once

#include "launch.hpp"
#include "quantize.hpp"
#include "rowq.hpp"
#include "sign.hpp"

namespace lowbit {

// Main kernel over the complete trips of full tiles; one-wave tail kernel for
// whatever remains (fewer than U full tiles and a partial last tile).
// 1-bit compress (every mode but Hadamard smoothing, whose butterflies work
// on the general tile): one coalesced tile per wave, tail kernel likewise.
template <int LOG2B, int DT, int MODE>
static lowbit_status launch_sign(const QuantArgs& a, hipStream_t s) {
  using S = SignShape<LOG2B>;
  const int64_t full_tiles = a.n / S::TILE;
  if (full_tiles > 0) {
    hipLaunchKernelGGL((sign_kernel<LOG2B, DT, MODE, false>), dim3(grid_for_tiles(full_tiles)),
                       dim3(kBlockThreads), 0, s, a, full_tiles);
  }
  if (full_tiles * S::TILE < a.n) {
    hipLaunchKernelGGL((sign_kernel<LOG2B, DT, MODE, true>), dim3(1), dim3(kWave), 0, s, a,
                       full_tiles);
  }
  return launch_status();
}

// 2- and 4-bit compress in the row layout: the error-feedback and EF21
// modes (LOWBIT_ROW_LAYOUT_EF), the plain and weight-difference modes
// (LOWBIT_ROW_LAYOUT_PLAIN); Hadamard smoothing keeps the general tile.
#ifndef LOWBIT_ROW_LAYOUT_EF
#define LOWBIT_ROW_LAYOUT_EF 1
#endif
#ifndef LOWBIT_ROW_LAYOUT_PLAIN
#define LOWBIT_ROW_LAYOUT_PLAIN 0
#endif
template <int MODE>
constexpr bool use_row_layout() {
  return (MODE == kErrorFeedback || MODE == kEF21) ? LOWBIT_ROW_LAYOUT_EF
         : (MODE == kPlain || MODE == kWeightDiff) ? LOWBIT_ROW_LAYOUT_PLAIN
                                                   : false;
}
template <int BITS, int LOG2B, bool SR, int DT, int MODE>
static lowbit_status launch_row(const QuantArgs& a, hipStream_t s) {
  using S = RowShape<BITS, LOG2B, MODE>;
  const int64_t full_trips = a.n / S::TILE;
  if (full_trips > 0) {
    hipLaunchKernelGGL((row_kernel<BITS, LOG2B, SR, DT, MODE, false>),
                       dim3(grid_for_tiles(full_trips)), dim3(kBlockThreads), 0, s, a, full_trips);
  }
  if (full_trips * S::TILE < a.n) {
    hipLaunchKernelGGL((row_kernel<BITS, LOG2B, SR, DT, MODE, true>), dim3(1), dim3(kWave), 0, s,
                       a, full_trips);
  }
  return launch_status();
}

template <int BITS, int LOG2B, bool SR, int DT, int MODE>
static lowbit_status launch_q(const QuantArgs& a, hipStream_t s) {
  if constexpr (BITS == 1 && MODE != kHadamard) {
    return launch_sign<LOG2B, DT, MODE>(a, s);
  } else if constexpr ((BITS == 2 || BITS == 4) && use_row_layout<MODE>()) {
    return launch_row<BITS, LOG2B, SR, DT, MODE>(a, s);
  } else {
    using S = TileShape<BITS, LOG2B>;
    constexpr int U = compress_tiles_per_trip<S::R * S::E, SR, DT, MODE>();
    const int64_t full_tiles = a.n / S::TILE;
    const int64_t ntrips = full_tiles / U;
    if (ntrips > 0) {
      hipLaunchKernelGGL((quantize_kernel<BITS, LOG2B, SR, DT, MODE, false>),
                         dim3(grid_for_tiles(ntrips)), dim3(kBlockThreads), 0, s, a, full_tiles);
    }
    if (ntrips * U * S::TILE < a.n) {
      hipLaunchKernelGGL((quantize_kernel<BITS, LOG2B, SR, DT, MODE, true>), dim3(1), dim3(kWave),
                         0, s, a, ntrips * U);
    }
    return launch_status();
  }
}

template <int BITS, int LOG2B, int MODE>
static lowbit_status launch_q_rd(bool sr, int dt, const QuantArgs& a, hipStream_t s) {
  // stochastic rounding does not apply to the 1-bit sign code
  if (BITS == 1 || !sr) {
    return dt == kF32 ? launch_q<BITS, LOG2B, false, kF32, MODE>(a, s)
                      : launch_q<BITS, LOG2B, false, kBF16, MODE>(a, s);
  }
  return dt == kF32 ? launch_q<BITS, LOG2B, (BITS > 1), kF32, MODE>(a, s)
                    : launch_q<BITS, LOG2B, (BITS > 1), kBF16, MODE>(a, s);
}

template <int BITS, int MODE>
static lowbit_status launch_q_b(int log2b, bool sr, int dt, const QuantArgs& a, hipStream_t s) {
  switch (log2b) {
#define LOWBIT_CASE(LB) \
  case LB:              \
    return launch_q_rd<BITS, LB, MODE>(sr, dt, a, s);
    LOWBIT_FOR_EACH_LOG2B(LOWBIT_CASE)
#undef LOWBIT_CASE
  }
  return LOWBIT_EUNSUPPORTED;
}

lowbit_status LOWBIT_TU_LAUNCHER(int bits, int log2b, bool sr, int dt, const QuantArgs& a,
                                 hipStream_t s) {
  switch (bits) {
    case 1: return launch_q_b<1, LOWBIT_TU_MODE>(log2b, sr, dt, a, s);
    case 2: return launch_q_b<2, LOWBIT_TU_MODE>(log2b, sr, dt, a, s);
    case 4: return launch_q_b<4, LOWBIT_TU_MODE>(log2b, sr, dt, a, s);
    case 8: return launch_q_b<8, LOWBIT_TU_MODE>(log2b, sr, dt, a, s);
  }
  return LOWBIT_EUNSUPPORTED;
}

}  // namespace lowbit
