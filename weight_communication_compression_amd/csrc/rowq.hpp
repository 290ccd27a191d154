// rowq.hpp -- 2- and 4-bit compress with fully coalesced loads (row layout).
//
// The general compress tile gives each lane whole output words: 16 (2 bits)
// or 8 (4 bits) consecutive elements, so a wave's 16-byte loads stride 64 or
// 32 bytes from lane to lane.  Here, as in the 1-bit compress, a row is 256
// consecutive elements, four per lane (one 16-byte binary32 or 8-byte
// bfloat16 load per lane and row, consecutive lanes on consecutive bytes):
//
//   lane l, row r holds elements r*256 + 4l + j, j < 4, and codes them into
//   a 4b-bit piece; the 8/b lanes of a code word (aligned groups of 2 or 4)
//   OR their pieces, shifted to 4b*(l mod 8/b), with one or two DPP moves,
//   and the group's first lane stores the word.
//
// The residual of the error-feedback modes is read and written in the same
// coalesced rows.  (Measured on the in-place y += x pattern of the EF
// compress, 64 Mi binary32: one coalesced row per wave 121.5 us, two rows
// 125.6, the 32-byte lane stride of the general tile 130 us.)
//
// A trip is max(kRowRows or kRowRowsEf, B/256) rows, so it holds whole blocks;
// the block statistic is the integer DPP maximum over the B/4 lanes of a
// block within a row, then over the block's rows.  The arithmetic per element
// is that of the general tile: v = x * fl(1/s); nearest: clamp, then round by
// adding 1.5 * 2^23; stochastic: floor(fma(r, 2^-24, v)) and clamp; the same
// packing constant, restricted to the lane's four fields.
#pragma once

#include "args.hpp"
#include "device.hpp"
#include "sign.hpp"

namespace lowbit {

// rows of 256 per trip (at least one block), plain / weight-difference and
// error-feedback / EF21 modes
constexpr int kRowRows = 2;
constexpr int kRowRowsEf = 1;
template <int MODE>
constexpr int row_rows_min() {
  return (MODE == kErrorFeedback || MODE == kEF21) ? kRowRowsEf : kRowRows;
}

// RMIN: rows per trip when blocks are shorter than that (a caller with other
// loads in flight per row may choose its own)
template <int BITS, int LOG2B, int MODE, int RMIN = row_rows_min<MODE>()>
struct RowShape {
  static constexpr int B = 1 << LOG2B;
  static constexpr int ROW = kWave * 4;                  // elements per row
  static constexpr int RT = B > RMIN * ROW ? B / ROW : RMIN;   // rows per trip
  static constexpr int TILE = ROW * RT;
  static constexpr int LB = B >= ROW ? kWave : B / 4;    // lanes of a block within a row
  static constexpr int RB = B >= ROW ? B / ROW : 1;      // rows of a block
  static constexpr int LPW = 8 / BITS;                   // lanes per code word
};

// Codes, scales and (error feedback / EF21) the residual or state of one
// loaded trip of RT rows.
template <int BITS, int LOG2B, bool SR, int MODE, bool FULL, int RMIN = row_rows_min<MODE>()>
__device__ __forceinline__ void row_finish(
    const QuantArgs& a, int64_t t0, const float (&v)[RowShape<BITS, LOG2B, MODE, RMIN>::RT][4],
    const float (&h)[RowShape<BITS, LOG2B, MODE, RMIN>::RT][4]) {
  using G = Grid<BITS>;
  using S = RowShape<BITS, LOG2B, MODE, RMIN>;
  constexpr int RT = S::RT, RB = S::RB, LB = S::LB, B = S::B, LPW = S::LPW;
  constexpr float QMAX = (float)G::QMAX;
  constexpr bool WANT_DEQ = MODE == kErrorFeedback || MODE == kEF21;
  // packing constant of a four-code piece (see Grid::PACK_BIAS)
  constexpr uint32_t BIAS4 = [] {
    uint32_t c = 0;
    for (int j = 0; j < 4; ++j) c += (G::HALF - kMagicBits) << (j * BITS);
    return c;
  }();
  static_assert(BITS == 2 || BITS == 4, "row layout for 2- and 4-bit codes");
  const int lane = lane_id();

  // ---- block statistic and scale (one per group of RB rows) ---------------
  float m[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float x = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) x = fmaxf(x, fabsf(v[r][j]));
    m[r] = group_max_nonneg<LB>(x);
  }
  // B < 256: a row holds several blocks and the first lane of each stores
  // its scale; otherwise lane k stores the trip's k-th scale, in one store.
  constexpr bool PER_ROW = RB == 1 && LB < kWave;
  BlockScale sc[RT / RB];
  uint32_t s16_lane = 0;
#pragma unroll
  for (int k = 0; k < RT / RB; ++k) {
    float mk = m[k * RB];
#pragma unroll
    for (int q = 1; q < RB; ++q) mk = fmaxf(mk, m[k * RB + q]);
    sc[k] = make_scale(div_by_grid<G::QMAX>(mk));
    if constexpr (PER_ROW) {
      const int64_t blk0 = t0 + (int64_t)k * S::ROW + (int64_t)(lane / LB) * B;
      if ((lane & (LB - 1)) == 0 && (FULL || blk0 < a.n))
        a.out.scales[blk0 >> LOG2B] = (uint16_t)sc[k].s16;
    } else {
      if (lane == k) s16_lane = sc[k].s16;
    }
  }
  if constexpr (!PER_ROW) {
    const int64_t b0 = t0 >> LOG2B;   // the trip's first block
    if (lane < RT / RB && (FULL || ((b0 + lane) << LOG2B) < a.n))
      a.out.scales[b0 + lane] = (uint16_t)s16_lane;
  }

  // ---- codes: a 4b-bit piece per lane, words across 8/b lanes -------------
  const int g = lane & (LPW - 1);   // the lane's place in its word
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const BlockScale& s = sc[r / RB];
    const int64_t i0 = t0 + (int64_t)(r * S::ROW + lane * 4);   // the lane's first element
    // SR: h_j = fmix32((lo + j) ^ hk); lo is a multiple of 4, so lo + j =
    // lo ^ j and the first fmix32 step is c ^ j with c computed once
    uint32_t c = 0;
    if constexpr (SR) {
      const uint64_t gi = a.out.index_offset + (uint64_t)i0;
      const uint32_t x0 = (uint32_t)gi ^ fmix32((uint32_t)(gi >> 32) ^ a.out.key);
      c = x0 ^ (x0 >> 16);
    }
    uint32_t piece = BIAS4;
    float deq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = v[r][j] * s.inv;
      float q;
      if constexpr (SR) {
        const uint32_t hh = fmix32_after_first_step(c ^ (uint32_t)j);
        const float y = __builtin_fmaf((float)(hh >> 8), 0x1p-24f, x);
        q = __builtin_amdgcn_fmed3f(floorf(y), -QMAX, QMAX);
      } else {
        q = __builtin_amdgcn_fmed3f(x, -QMAX, QMAX);
      }
      const float t = q + kMagic;               // nearest: the rounding; SR: exact
      piece += __float_as_uint(t) << (j * BITS);
      deq[j] = (t - kMagic) * s.s;
    }
    uint32_t w = piece << (4 * BITS * g);
    w |= dpp_u32<0xB1>(w);                      // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (LPW == 4) w |= dpp_u32<0x4E>(w);   // quad_perm [2,3,0,1]: lane ^ 2
    if (g == 0) {
      uint32_t* const p = a.out.codes + (i0 * BITS) / 32;
      if (FULL) {
        store_stream(p, w);
      } else if (i0 < a.n) {
        const int64_t valid = a.n - i0;
        if (valid < G::E) w &= (1u << (valid * BITS)) - 1u;
        store_stream(p, w);
      }
    }
    if constexpr (WANT_DEQ) {
      const uint32_t off = (uint32_t)(r * S::ROW + lane * 4);
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (MODE == kErrorFeedback) e[j] = v[r][j] - deq[j];   // e = a - deq
        else e[j] = h[r][j] + deq[j];                                    // h + deq
      }
      if constexpr (FULL) store_vec_f32<4>(a.resid, t0, off, e);
      else store_tail_f32<4>(a.resid, t0, off, a.n - t0, e);
    }
    (void)deq;
  }
  (void)h;
}

// Main kernel (TAIL = false): one full trip per wave, no bounds checks; the
// grid covers the `first` full trips.  Tail kernel (TAIL = true, one wave):
// the remaining trips from trip `first`, the last of which may be partial.
template <int BITS, int LOG2B, bool SR, int DT, int MODE, bool TAIL>
__global__ __launch_bounds__(kBlockThreads) void row_kernel(QuantArgs a, int64_t first) {
  using S = RowShape<BITS, LOG2B, MODE>;
  constexpr int RT = S::RT;
  if constexpr (TAIL) {
    if (global_wave_id() != 0) return;
    const int64_t ntrips = (a.n + S::TILE - 1) / S::TILE;
    for (int64_t trip = first; trip < ntrips; ++trip) {
      const int64_t t0 = trip * S::TILE;
      float v[RT][4], h[RT][4];
      if (t0 + S::TILE <= a.n) {
        row_load<RT, DT, MODE, true>(a, t0, v, h);
        row_finish<BITS, LOG2B, SR, MODE, true>(a, t0, v, h);
      } else {
        row_load<RT, DT, MODE, false>(a, t0, v, h);
        row_finish<BITS, LOG2B, SR, MODE, false>(a, t0, v, h);
      }
    }
  } else {
    const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
    for_each_trip(global_wave_id(), first, nwaves, [&](int64_t trip) __attribute__((always_inline)) {
      const int64_t t0 = trip * S::TILE;
      float v[RT][4], h[RT][4];
      row_load<RT, DT, MODE, true>(a, t0, v, h);
      row_finish<BITS, LOG2B, SR, MODE, true>(a, t0, v, h);
    });
  }
}

}  // namespace lowbit
