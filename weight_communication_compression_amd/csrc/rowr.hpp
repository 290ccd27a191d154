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

// Workgroups per XCD run (logical_block): a 128-byte line of one peer's
// scales serves 8 workgroups of this kernel, so runs of 8 fetch each line into
// one L2 instead of up to eight (8 x 32 Mi peers with the stage-2 residual:
// 70.4 -> 68.8 us).  The other kernels keep the hardware order, which
// measured as fast or faster for them.
constexpr int kRowrXcdChunk = 8;

// Rows of 256 per trip for blocks shorter than that: 2 in both modes.  With
// the stage-2 residual (8 x 32 Mi peers, b4 B128) 2 rows take 66.8 us against
// 70.5 us for the single row of the error-feedback compress, whose trip has
// no peer loads to keep in flight, and 68.8 us for 4 rows.  Streamed peers'
// code words (non-temporal loads, without LOWBIT_HINT_INPUT_REUSED): the
// reduce with the binary32 sum output 60 -> 56 us, the stage-2 one unchanged.
constexpr int kRowrRows = 2;
template <int BITS, int LOG2B, bool EF>
using RowrShape = RowShape<BITS, LOG2B, EF ? kErrorFeedback : kPlain, kRowrRows>;

template <int BITS, int LOG2B, bool SR, bool EF, bool FULL, int NPC = 0, bool STREAM = false>
__device__ __forceinline__ void rowr_trip(const ReduceArgs& a, int64_t t0) {
  constexpr int MODE = EF ? kErrorFeedback : kPlain;
  using S = RowrShape<BITS, LOG2B, EF>;
  // peers whose loads are in flight together: 8, fewer for trips of more
  // than two rows, so that a lane holds at most 16 code words and 16 scales
  constexpr int RT = S::RT, E = Grid<BITS>::E, G = RT <= 2 ? 8 : (16 / RT > 1 ? 16 / RT : 1);
  constexpr float UNSCALE = 1.0f / (float)(1 << acc_shift<BITS>());   // exact
  const int lane = lane_id();
  const int lbi = a.in_log2b;
  const int np = peer_count<NPC>(a);
  const int64_t n = a.n;
  const uint32_t lo = 4u * (uint32_t)lane;
  const int sh = (int)(lo % E) * BITS;                      // the lane's piece in its word

  float acc[RT][4];
  // the stage-2 residual, loaded with the first peers (positions past the
  // end read 0)
  float e[RT][4];
  if constexpr (EF) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint32_t off = (uint32_t)(r * S::ROW) + lo;
      if (FULL) load_vec<kF32, 4>(a.resid, t0, off, e[r]);
      else load_tail<kF32, 4>(a.resid, t0, off, n - t0, e[r]);
    }
  }
  static_assert(kMaxPeers % G == 0, "peer groups tile the argument block");
#pragma unroll(NPC > 0 ? 16 : 1)
  for (int g = 0; g < np; g += G) {
    uint32_t w[G][RT], sc[G][RT];
    const uint32_t* cps[G];
    const uint16_t* sps[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      cps[q] = a.codes[g + q];
      sps[q] = a.scales[g + q];
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
      if (g + q < np) {                                     // wave-uniform
        const uint32_t* cp = cps[q];
        const uint16_t* sp = sps[q];
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const int64_t i0 = t0 + r * S::ROW + lo;
          w[q][r] = 0;
          sc[q][r] = 0;
          if (FULL || i0 < n) {
            w[q][r] = load_once<STREAM>(cp + i0 / E);
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
    // a = fl(sum + e)
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[r][j] = v[r][j] + e[r][j];
  }
  QuantArgs qa{};
  qa.n = n;
  qa.resid = a.resid;
  qa.out = a.out;
  row_finish<BITS, LOG2B, SR, MODE, FULL, kRowrRows>(qa, t0, v, h);
  (void)h;
}

// Main kernel (TAIL = false): one full trip per wave; the grid covers the
// `first` full trips.  Tail kernel (TAIL = true, one wave): the trips from
// `first` on, the last of which may be partial.
// STREAM: the peers' code words are read non-temporally (main kernel only).
template <int BITS, int LOG2B, bool SR, bool EF, bool TAIL, bool STREAM = false>
__global__ __launch_bounds__(kBlockThreads) void rowr_kernel(ReduceArgs a, int64_t first) {
  using S = RowrShape<BITS, LOG2B, EF>;
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
    const int64_t trip = global_wave_id<kBlockThreads, kRowrXcdChunk>();
    // eight peers (one per GPU of an 8-GPU node): the straight-line form.
    // The first trip is kept out of the loop (see for_each_trip), which only
    // runs where the grid was capped.
    if (trip < first) {
      if (a.npeers == 8) rowr_trip<BITS, LOG2B, SR, EF, true, 8, STREAM>(a, trip * S::TILE);
      else rowr_trip<BITS, LOG2B, SR, EF, true, 0, STREAM>(a, trip * S::TILE);
    }
    for (int64_t t = trip + nwaves; t < first; t += nwaves)
      rowr_trip<BITS, LOG2B, SR, EF, true, 0, STREAM>(a, t * S::TILE);
  }
}

}  // namespace lowbit
