// quantize_tu.hpp -- one translation unit's worth of compress-kernel
// instantiations for the mode LOWBIT_TU_MODE, exposed through the launcher
// LOWBIT_TU_LAUNCHER(bits, log2b, sr, dtype, stream_input, args, stream).
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
// stream_input: read x non-temporally where the kernel can (stream_capable).
template <int LOG2B, int DT, int MODE>
static lowbit_status launch_sign(const QuantArgs& a, bool stream_input, hipStream_t s) {
  using S = SignShape<LOG2B>;
  const int64_t full_tiles = a.n / S::TILE;
  lowbit_status st = LOWBIT_OK;
  if (full_tiles > 0) {
    const int64_t grid = grid_for_tiles(full_tiles);
    bool streamed = false;
    if constexpr (stream_capable<MODE, DT, 4, 1>()) {
      if (stream_input) {
        st = launch(&sign_kernel<LOG2B, DT, MODE, false, true>, grid, kBlockThreads, s, a,
                    full_tiles);
        streamed = true;
      }
    }
    if (!streamed)
      st = launch(&sign_kernel<LOG2B, DT, MODE, false>, grid, kBlockThreads, s, a, full_tiles);
  }
  if (st == LOWBIT_OK && full_tiles * S::TILE < a.n)
    st = launch(&sign_kernel<LOG2B, DT, MODE, true>, 1, kWave, s, a, full_tiles);
  return st;
}

// 2- and 4-bit compress in the row layout for the error-feedback and EF21
// modes (coalesced rows for the gradient and the residual or state: the EF
// compress of the 64 Mi bucket 131.5 -> 125-129 us); the plain and
// weight-difference modes keep the general tile, which measured faster for
// them both alone and inside the whole-path step (row layout, 64 Mi bucket
// alone: 2 bits 50.7 -> 54.5 us, 4 bits 55.2 -> 56.4 us; 1, 2 or 4 rows per
// trip all slower); Hadamard smoothing keeps the general tile.
template <int MODE>
constexpr bool use_row_layout() {
  return MODE == kErrorFeedback || MODE == kEF21;
}
template <int BITS, int LOG2B, bool SR, int DT, int MODE>
static lowbit_status launch_row(const QuantArgs& a, hipStream_t s) {
  using S = RowShape<BITS, LOG2B, MODE>;
  const int64_t full_trips = a.n / S::TILE;
  lowbit_status st = LOWBIT_OK;
  if (full_trips > 0)
    st = launch(&row_kernel<BITS, LOG2B, SR, DT, MODE, false>, grid_for_tiles(full_trips),
                kBlockThreads, s, a, full_trips);
  if (st == LOWBIT_OK && full_trips * S::TILE < a.n)
    st = launch(&row_kernel<BITS, LOG2B, SR, DT, MODE, true>, 1, kWave, s, a, full_trips);
  return st;
}

template <int BITS, int LOG2B, bool SR, int DT, int MODE>
static lowbit_status launch_q(const QuantArgs& a, bool stream_input, hipStream_t s) {
  if constexpr (BITS == 1 && MODE != kHadamard) {
    return launch_sign<LOG2B, DT, MODE>(a, stream_input, s);
  } else if constexpr ((BITS == 2 || BITS == 4) && use_row_layout<MODE>()) {
    return launch_row<BITS, LOG2B, SR, DT, MODE>(a, s);
  } else {
    using S = TileShape<BITS, LOG2B>;
    constexpr int U = compress_tiles_per_trip<S::R * S::E, SR, DT, MODE>();
    const int64_t full_tiles = a.n / S::TILE;
    const int64_t ntrips = full_tiles / U;
    lowbit_status st = LOWBIT_OK;
    if (ntrips > 0) {
      const int64_t grid = grid_for_tiles(ntrips);
      bool streamed = false;
      if constexpr (stream_capable<MODE, DT, S::E, S::R>()) {
        if (stream_input) {
          st = launch(&quantize_kernel<BITS, LOG2B, SR, DT, MODE, false, true>, grid,
                      kBlockThreads, s, a, full_tiles);
          streamed = true;
        }
      }
      if (!streamed)
        st = launch(&quantize_kernel<BITS, LOG2B, SR, DT, MODE, false>, grid, kBlockThreads, s, a,
                    full_tiles);
    }
    if (st == LOWBIT_OK && ntrips * U * S::TILE < a.n)
      st = launch(&quantize_kernel<BITS, LOG2B, SR, DT, MODE, true>, 1, kWave, s, a, ntrips * U);
    return st;
  }
}

template <int BITS, int LOG2B, int MODE>
static lowbit_status launch_q_rd(bool sr, int dt, bool si, const QuantArgs& a, hipStream_t s) {
  // stochastic rounding does not apply to the 1-bit sign code
  if (BITS == 1 || !sr) {
    return dt == kF32 ? launch_q<BITS, LOG2B, false, kF32, MODE>(a, si, s)
                      : launch_q<BITS, LOG2B, false, kBF16, MODE>(a, si, s);
  }
  return dt == kF32 ? launch_q<BITS, LOG2B, (BITS > 1), kF32, MODE>(a, si, s)
                    : launch_q<BITS, LOG2B, (BITS > 1), kBF16, MODE>(a, si, s);
}

template <int BITS, int MODE>
static lowbit_status launch_q_b(int log2b, bool sr, int dt, bool si, const QuantArgs& a,
                                hipStream_t s) {
  switch (log2b) {
#define LOWBIT_CASE(LB) \
  case LB:              \
    return launch_q_rd<BITS, LB, MODE>(sr, dt, si, a, s);
    LOWBIT_FOR_EACH_LOG2B(LOWBIT_CASE)
#undef LOWBIT_CASE
  }
  return LOWBIT_EUNSUPPORTED;
}

lowbit_status LOWBIT_TU_LAUNCHER(int bits, int log2b, bool sr, int dt, bool stream_input,
                                 const QuantArgs& a, hipStream_t s) {
  switch (bits) {
    case 1: return launch_q_b<1, LOWBIT_TU_MODE>(log2b, sr, dt, stream_input, a, s);
    case 2: return launch_q_b<2, LOWBIT_TU_MODE>(log2b, sr, dt, stream_input, a, s);
    case 4: return launch_q_b<4, LOWBIT_TU_MODE>(log2b, sr, dt, stream_input, a, s);
    case 8: return launch_q_b<8, LOWBIT_TU_MODE>(log2b, sr, dt, stream_input, a, s);
  }
  return LOWBIT_EUNSUPPORTED;
}

}  // namespace lowbit
