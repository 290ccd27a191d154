// rowr.hpp -- local reduce + requantize of 2- and 4-bit peers into the same
// width, in the row layout of rowq.hpp.
//
// Lane l of row r owns output elements r*256 + 4l + j (j < 4).  For each peer
// it loads the code word holding its four codes (the 8/b lanes of a word read
// the same address) and the scale of their input block, decodes the four
// codes as the general reduce does (fields lifted to the top of a byte,
// sign-extending byte converts, sums scaled by 2^(8-b) exactly, peers added
// in order), then hands the unscaled sums -- plus the stage-2 residual read
// in the same coalesced rows -- to the row-layout requantization.
#pragma once

#include "reduce.hpp"
#include "rowq.hpp"

namespace lowbit {

// acc[j] (+)= 2^(8-b) * q_j * s for the four b-bit codes in the low 4b bits of
// `piece` (as accumulate_word, on four fields).
template <int BITS, bool FIRST>
__device__ __forceinline__ void accumulate_piece(uint32_t piece, float s, float* acc) {
  using G = Grid<BITS>;
  constexpr int PER_BYTE = 8 / BITS;
  constexpr int NB = 4 * BITS / 8;                          // bytes of the piece
  constexpr uint32_t TOP = (uint32_t)((0xFFu << (8 - BITS)) & 0xFFu) * 0x01010101u;
  const uint32_t tw = piece ^ G::FLIP;                      // two's-complement fields
#pragma unroll
  for (int p = 0; p < PER_BYTE; ++p) {
    const uint32_t t = (tw << (8 - BITS * (p + 1))) & TOP;  // field p of each byte on top
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const float qb = (float)(signed char)(t >> (8 * k));  // 2^(8-b) * q
      const int j = PER_BYTE * k + p;
      acc[j] = FIRST ? qb * s : __builtin_fmaf(qb, s, acc[j]);
    }
  }
}

template <int BITS, int LOG2B, bool SR, bool EF, bool FULL>
__device__ __forceinline__ void rowr_trip(const ReduceArgs& a, int64_t t0) {
  constexpr int MODE = EF ? kErrorFeedback : kPlain;
  using S = RowShape<BITS, LOG2B, MODE>;
  constexpr int RT = S::RT, E = Grid<BITS>::E, G = 8;
  constexpr float UNSCALE = 1.0f / (float)(1 << acc_shift<BITS>());   // exact
  const int lane = lane_id();
  const int lbi = a.in_log2b;
  const int np = a.npeers;
  const int64_t n = a.n;
  const uint32_t lo = 4u * (uint32_t)lane;
  const int sh = (int)(lo % E) * BITS;                      // the lane's piece in its word

  float acc[RT][4];
#pragma unroll 1
  for (int g = 0; g < np; g += G) {
    uint32_t w[G][RT], sc[G][RT];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (g + q < np) {                                     // wave-uniform
        const uint32_t* cp = a.codes[g + q];
        const uint16_t* sp = a.scales[g + q];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const int64_t i0 = t0 + r * S::ROW + lo;
          w[q][r] = 0;
          sc[q][r] = 0;
          if (FULL || i0 < n) {
            w[q][r] = cp[i0 / E];
            sc[q][r] = sp[i0 >> lbi];
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (g + q < np) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const float s = f16_bits_to_f32(sc[q][r]);
          if (q == 0 && g == 0) accumulate_piece<BITS, true>(w[q][r] >> sh, s, acc[r]);
          else accumulate_piece<BITS, false>(w[q][r] >> sh, s, acc[r]);
        }
      }
    }
  }

  // unscaled sums (exact); positions past the end are +0
  float v[RT][4], h[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[r][j] = acc[r][j] * UNSCALE;
      if (!FULL && t0 + r * S::ROW + lo + j >= n) v[r][j] = 0.0f;
    }
  if (a.out_sum) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint32_t off = (uint32_t)(r * S::ROW) + lo;
      if (FULL) store_vec_f32<4>(a.out_sum, t0, off, v[r]);
      else store_tail_f32<4>(a.out_sum, t0, off, n - t0, v[r]);
    }
  }
  if constexpr (EF) {
    // a = fl(sum + e); the residual past the end reads 0
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint32_t off = (uint32_t)(r * S::ROW) + lo;
      float e[4];
      if (FULL) load_vec<kF32, 4>(a.resid, t0, off, e);
      else load_tail<kF32, 4>(a.resid, t0, off, n - t0, e);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[r][j] = v[r][j] + e[j];
    }
  }
  QuantArgs qa{};
  qa.n = n;
  qa.resid = a.resid;
  qa.out = a.out;
  row_finish<BITS, LOG2B, SR, MODE, FULL>(qa, t0, v, h);
  (void)h;
}

// Main kernel (TAIL = false): one full trip per wave; the grid covers the
// `first` full trips.  Tail kernel (TAIL = true, one wave): the trips from
// `first` on, the last of which may be partial.
template <int BITS, int LOG2B, bool SR, bool EF, bool TAIL>
__global__ __launch_bounds__(kBlockThreads) void rowr_kernel(ReduceArgs a, int64_t first) {
  using S = RowShape<BITS, LOG2B, EF ? kErrorFeedback : kPlain>;
  if constexpr (TAIL) {
    if (global_wave_id() != 0) return;
    const int64_t ntrips = (a.n + S::TILE - 1) / S::TILE;
    for (int64_t trip = first; trip < ntrips; ++trip) {
      const int64_t t0 = trip * S::TILE;
      if (t0 + S::TILE <= a.n) rowr_trip<BITS, LOG2B, SR, EF, true>(a, t0);
      else rowr_trip<BITS, LOG2B, SR, EF, false>(a, t0);
    }
  } else {
    const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
    for (int64_t trip = global_wave_id(); trip < first; trip += nwaves)
      rowr_trip<BITS, LOG2B, SR, EF, true>(a, trip * S::TILE);
  }
}

}  // namespace lowbit
