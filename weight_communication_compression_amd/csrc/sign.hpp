// sign.hpp -- 1-bit (sign + mean|x| scale) compress with fully coalesced loads.
//
// The general compress tile gives each lane whole output words; at one bit a
// word is 32 elements, so a wave's 16-byte loads would stride 128 bytes from
// lane to lane and every load instruction would touch 64 cache lines.  Here a
// row is 256 consecutive elements, four per lane (one 16-byte binary32 load
// or one 8-byte bfloat16 load per lane, consecutive lanes on consecutive
// bytes), and the 32 sign bits of a word are gathered across the 8 lanes
// that hold them:
//
//   lane l, row r holds elements r*256 + 4l + j, j < 4;
//   its nibble of signs sits at bits 4*(l mod 8) + j of word 8r + l/8;
//   an OR over each aligned group of 8 lanes (quad_perm xor 1, xor 2, then
//   row_half_mirror) leaves the whole word in all 8 lanes;
//   lane l keeps the word of the row r with r mod 8 = l mod 8.
//
// So after 8 rows each lane holds one word, and the wave's 64 words (256
// contiguous bytes, permuted across lanes) go out in one store.  A tile is
// max(8, B/256) rows; for B = 4096 each lane keeps two words.
//
// The block statistic is the same adjacent-pairs tree as the general tile:
// an in-lane tree over the lane's 4 leaves, the butterfly over the B/4 lanes
// of a block (a 256-element row at most), then a tree over the block's rows.
#pragma once

#include "args.hpp"
#include "device.hpp"

namespace lowbit {

template <int LOG2B>
struct SignShape {
  static constexpr int B = 1 << LOG2B;
  static constexpr int ROW = kWave * 4;                  // elements per row
  static constexpr int RT = B > 8 * ROW ? B / ROW : 8;   // rows per tile
  static constexpr int TILE = ROW * RT;                  // 2048, or 4096 for B = 4096
  static constexpr int LB = B >= ROW ? kWave : B / 4;    // lanes of a block within a row
  static constexpr int RB = B >= ROW ? B / ROW : 1;      // rows of a block
  static constexpr int WPL = RT / 8;                     // code words kept per lane
};

// Load RT rows of 256 elements from element t0, four consecutive elements
// per lane and row (plus the residual, minus the old weights, or minus the
// EF21 state, as in the general compress); positions at or past n read +0.
template <int RT, int DT, int MODE, bool FULL, bool NTX = false>
__device__ __forceinline__ void row_load(const QuantArgs& a, int64_t t0, float (&v)[RT][4],
                                         float (&h)[RT][4]) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const uint32_t off = (uint32_t)(r * kWave * 4 + lane * 4);
    float w[4];
    if constexpr (FULL) {
      constexpr bool RMW = MODE == kErrorFeedback || MODE == kEF21;
      load_vec<DT, 4, NTX && stream_capable<MODE, DT, 4, 1>()>(a.x, t0, off, v[r]);
      if constexpr (RMW) load_vec<kF32, 4>(a.resid, t0, off, w);
      if constexpr (MODE == kWeightDiff) load_vec<DT, 4>(a.x2, t0, off, w);
    } else {
      load_tail<DT, 4>(a.x, t0, off, a.n - t0, v[r]);
      if constexpr (MODE == kErrorFeedback || MODE == kEF21)
        load_tail<kF32, 4>(a.resid, t0, off, a.n - t0, w);
      if constexpr (MODE == kWeightDiff) load_tail<DT, 4>(a.x2, t0, off, a.n - t0, w);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (MODE == kErrorFeedback) v[r][j] = v[r][j] + w[j];   // a = g + e
      if constexpr (MODE == kWeightDiff) v[r][j] = v[r][j] - w[j];      // w_new - w_old
      if constexpr (MODE == kEF21) {
        v[r][j] = v[r][j] - w[j];                                       // d = g - h
        h[r][j] = w[j];
      }
    }
  }
}

// Codes, scales and (error feedback / EF21) the residual or state of one
// loaded tile.
template <int LOG2B, int MODE, bool FULL>
__device__ __forceinline__ void sign_finish(const QuantArgs& a, int64_t t0,
                                            const float (&v)[SignShape<LOG2B>::RT][4],
                                            const float (&h)[SignShape<LOG2B>::RT][4]) {
  using S = SignShape<LOG2B>;
  constexpr int RT = S::RT, RB = S::RB, LB = S::LB, B = S::B, WPL = S::WPL;
  const int lane = lane_id();
  const int m = lane & 7;

  // ---- codes: nibbles of signs, gathered into words across 8 lanes --------
  uint32_t nib[RT];
  uint32_t keep[WPL];
#pragma unroll
  for (int k = 0; k < WPL; ++k) keep[k] = 0;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    nib[r] = sign_codes<4>(v[r]);
    uint32_t c = nib[r] << (4 * m);
    c |= dpp_u32<0xB1>(c);    // quad_perm [1,0,3,2]
    c |= dpp_u32<0x4E>(c);    // quad_perm [2,3,0,1]: the quad's OR
    c |= dpp_u32<0x141>(c);   // row_half_mirror: the other quad of the 8
    if (m == (r & 7)) keep[r >> 3] = c;
  }

  // ---- block statistic and scale (one per group of RB rows) ---------------
  float g[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) g[r] = group_reduce<LB, true>(lane_abs_tree<4>(v[r]));
  // B < 256: a row holds several blocks and the first lane of each stores
  // its scale; otherwise a block's scale is the same in every lane and lane k
  // stores the tile's k-th scale, all in one store.
  constexpr bool PER_ROW = RB == 1 && LB < kWave;
  float sv[RT / RB];   // the block's scale value, per row group
  uint32_t s16_lane = 0;
#pragma unroll
  for (int k = 0; k < RT / RB; ++k) {
    const float Ssum = reg_tree<RB>(g + k * RB);
    const int64_t blk0 = t0 + (int64_t)k * RB * S::ROW + (RB == 1 ? (int64_t)(lane / LB) * B : 0);
    float t = Ssum * (1.0f / (float)B);    // exact: B is a power of two
    if (!FULL) {
      const int64_t rem = a.n - blk0;
      if (rem > 0 && rem < B) t = Ssum / (float)rem;
    }
    const BlockScale sc = make_scale(t);
    sv[k] = sc.s;
    if constexpr (PER_ROW) {
      if ((lane & (LB - 1)) == 0 && (FULL || blk0 < a.n))
        a.out.scales[blk0 >> LOG2B] = (uint16_t)sc.s16;
    } else {
      if (lane == k) s16_lane = sc.s16;
    }
  }
  if constexpr (!PER_ROW) {
    const int64_t b0 = t0 >> LOG2B;   // the tile's first block
    if (lane < RT / RB && (FULL || ((b0 + lane) << LOG2B) < a.n))
      a.out.scales[b0 + lane] = (uint16_t)s16_lane;
  }

  // ---- store the words: lane l holds word 64*k + 8*(l mod 8) + l/8 --------
  uint32_t* const cbase = a.out.codes + t0 / 32;
#pragma unroll
  for (int k = 0; k < WPL; ++k) {
    const uint32_t wi = (uint32_t)(64 * k + 8 * m + (lane >> 3));
    if (FULL) {
      store_stream(cbase + wi, keep[k]);
    } else {
      const int64_t i0 = t0 + (int64_t)wi * 32;
      if (i0 < a.n) {
        const int64_t valid = a.n - i0;
        uint32_t word = keep[k];
        if (valid < 32) word &= (1u << valid) - 1u;
        store_stream(cbase + wi, word);
      }
    }
  }

  // ---- residual (a - deq) or EF21 state (h + deq), deq = u ? s : -s ------
  if constexpr (MODE == kErrorFeedback || MODE == kEF21) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint32_t off = (uint32_t)(r * S::ROW + lane * 4);
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d = signed_scale(nib[r], j, sv[r / RB]);
        if constexpr (MODE == kErrorFeedback) e[j] = v[r][j] - d;
        else e[j] = h[r][j] + d;
      }
      if constexpr (FULL) store_vec_f32<4>(a.resid, t0, off, e);
      else store_tail_f32<4>(a.resid, t0, off, a.n - t0, e);
    }
  }
  (void)h;
}

// Main kernel (TAIL = false): one full tile per wave, no bounds checks; the
// grid covers the `first` full tiles.  Tail kernel (TAIL = true, one wave):
// the remaining tiles from tile `first`, the last of which may be partial.
// NTX: read x with non-temporal loads where stream_capable.
template <int LOG2B, int DT, int MODE, bool TAIL, bool NTX = false>
__global__ __launch_bounds__(kBlockThreads) void sign_kernel(QuantArgs a, int64_t first) {
  using S = SignShape<LOG2B>;
  constexpr int RT = S::RT;
  if constexpr (TAIL) {
    if (global_wave_id() != 0) return;
    const int64_t ntiles = (a.n + S::TILE - 1) / S::TILE;
    for (int64_t tile = first; tile < ntiles; ++tile) {
      const int64_t t0 = tile * S::TILE;
      float v[RT][4], h[RT][4];
      if (t0 + S::TILE <= a.n) {
        row_load<RT, DT, MODE, true>(a, t0, v, h);
        sign_finish<LOG2B, MODE, true>(a, t0, v, h);
      } else {
        row_load<RT, DT, MODE, false>(a, t0, v, h);
        sign_finish<LOG2B, MODE, false>(a, t0, v, h);
      }
    }
  } else {
    const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
    for_each_trip(global_wave_id(), first, nwaves, [&](int64_t tile) __attribute__((always_inline)) {
      const int64_t t0 = tile * S::TILE;
      float v[RT][4], h[RT][4];
      row_load<RT, DT, MODE, true, NTX>(a, t0, v, h);
      sign_finish<LOG2B, MODE, true>(a, t0, v, h);
    });
  }
}

}  // namespace lowbit
