// quantize.hpp -- blockwise compress of one tile held in registers, and the
// compress kernel built on it (plain / error feedback / weight difference).
// Templated on bitwidth, block size, rounding, input dtype and mode so that
// the inner loop has no run-time branches.
//
// Work layout (gfx950, wave64): lane l of a wave owns whole output words.
// A "tile" is R rows of 64 words; row r, lane l holds word r*64 + l of the
// tile, i.e. E = 32/b consecutive elements, loaded with 16-byte vector loads.
//   B <= 64*E (R = 1): a block is L = B/E consecutive lanes; its statistic
//     is a DPP reduction over those lanes.
//   B  > 64*E (R = B/(64E)): one tile is one block; the statistic is
//     reduced over the rows in registers and then over the wave.
// Each lane then computes its block's scale (the same value in every lane of
// the block), quantizes its E elements, packs them into one word per row and
// stores it; lane 0 of each block stores the binary16 scale.
#pragma once

#include "args.hpp"
#include "device.hpp"

namespace lowbit {

template <int BITS, int LOG2B>
struct TileShape {
  static constexpr int E = Grid<BITS>::E;
  static constexpr int B = 1 << LOG2B;
  static constexpr int ROW = kWave * E;                  // elements per row of words
  static constexpr int R = B > ROW ? B / ROW : 1;        // rows per tile
  static constexpr int TILE = ROW * R;                   // elements per tile
  static constexpr int L = B > ROW ? kWave : B / E;      // lanes per block
};

// Quantize the tile starting at element t0 whose values are v[r][j] (element
// t0 + (r*64 + lane)*E + j; positions at or past n must hold +0).  Stores the
// codes and scales; when WANT_DEQ, deq[r][j] receives the dequantized values.
template <int BITS, int LOG2B, bool SR, bool WANT_DEQ>
__device__ __forceinline__ void quantize_tile(
    const float (&v)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E], int64_t t0, int64_t n,
    bool full, const TileOut& o, float (&deq)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E]) {
  using G = Grid<BITS>;
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R, L = S::L, B = S::B;
  constexpr float QMAX = (float)G::QMAX;
  const int lane = lane_id();

  // ---- block statistic and scale ----------------------------------------
  const int64_t blk0 = (R == 1) ? t0 + (int64_t)(lane / L) * B : t0;   // block's first element
  float t;   // fl(statistic / divisor)
  if constexpr (BITS == 1) {
    float g[R];
#pragma unroll
    for (int r = 0; r < R; ++r) g[r] = group_reduce<L, true>(lane_abs_tree<E>(v[r]));
    const float S = reg_tree<R>(g);
    // mean over the valid elements; for a full block the divisor is the
    // power of two B and the multiply by 1/B is exact
    t = S * (1.0f / (float)B);
    if (!full) {
      const int64_t rem = n - blk0;
      if (rem < B) t = S / (float)rem;
    }
  } else {
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < E; ++j) m = fmaxf(m, fabsf(v[r][j]));
    t = div_by_grid<G::QMAX>(group_max_nonneg<L>(m));
  }
  const BlockScale sc = make_scale(t);
  if ((lane & (L - 1)) == 0 && blk0 < n) o.scales[blk0 >> LOG2B] = (uint16_t)sc.s16;

  // ---- codes and packing ---------------------------------------------------
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t w0 = t0 / E + r * kWave + lane;     // word index
    const int64_t i0 = w0 * E;                        // its first element
    uint32_t word;
    if constexpr (BITS == 1) {
      word = 0;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const bool pos = v[r][j] >= 0.0f;
        word |= (pos ? 1u : 0u) << j;
        if constexpr (WANT_DEQ) deq[r][j] = pos ? sc.s : -sc.s;
      }
    } else {
      word = G::PACK_BIAS;
      uint32_t hk = 0, lo = 0;
      if constexpr (SR) {
        const uint64_t gi = o.index_offset + (uint64_t)i0;
        hk = fmix32((uint32_t)(gi >> 32) ^ o.key);
        lo = (uint32_t)gi;
      }
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const float x = v[r][j] * sc.inv;
        float q;
        if constexpr (SR) {
          const uint32_t h = fmix32((lo + (uint32_t)j) ^ hk);
          // the random offset (h >> 8) * 2^-24 is exact, so the fused form
          // rounds once, exactly like adding it in binary32.
          const float y = __builtin_fmaf((float)(h >> 8), 0x1p-24f, x);
          q = __builtin_amdgcn_fmed3f(floorf(y), -QMAX, QMAX);
        } else {
          // clamp, then round: the same as rounding then clamping because the
          // bounds are integers; with |q| <= QMAX adding 1.5 * 2^23 rounds to
          // the nearest integer, ties to even.
          q = __builtin_amdgcn_fmed3f(x, -QMAX, QMAX);
        }
        const float t = q + kMagic;               // RTN: the rounding; SR: exact
        word += __float_as_uint(t) << (j * BITS);
        if constexpr (WANT_DEQ) deq[r][j] = (t - kMagic) * sc.s;
      }
    }
    if (full) {
      o.codes[w0] = word;
    } else if (i0 < n) {
      const int64_t valid = n - i0;
      if (valid < E) word &= (1u << (valid * BITS)) - 1u;
      o.codes[w0] = word;
    }
  }
}

// Each wave handles U consecutive tiles per loop trip: all of their loads are
// issued before any of them is quantized, so a wave keeps U tiles of HBM
// reads in flight while it computes.
template <int BITS, int LOG2B, bool SR, int DT, int MODE>
__global__ __launch_bounds__(kBlockThreads) void quantize_kernel(QuantArgs a) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R;
  constexpr int U = tiles_per_trip<R * E>();
  constexpr bool EF = MODE == kErrorFeedback;

  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * (kBlockThreads / kWave) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t n = a.n;
  const int64_t ntiles = (n + S::TILE - 1) / S::TILE;

  for (int64_t base = wave * U; base < ntiles; base += nwaves * U) {
    float v[U][R][E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t0 = (base + u) * S::TILE;
      if (base + u >= ntiles) break;                 // wave-uniform
      const bool full = t0 + S::TILE <= n;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t i0 = t0 + (int64_t)(r * kWave + lane) * E;
        float w[E];
        if (full) {
          load_vec<DT, E>(a.x, i0, v[u][r]);
          if constexpr (MODE == kErrorFeedback) load_vec<kF32, E>(a.resid, i0, w);
          if constexpr (MODE == kWeightDiff) load_vec<DT, E>(a.x2, i0, w);
        } else {
          load_tail<DT, E>(a.x, i0, n, v[u][r]);
          if constexpr (MODE == kErrorFeedback) load_tail<kF32, E>(a.resid, i0, n, w);
          if constexpr (MODE == kWeightDiff) load_tail<DT, E>(a.x2, i0, n, w);
        }
#pragma unroll
        for (int j = 0; j < E; ++j) {
          if constexpr (MODE == kErrorFeedback) v[u][r][j] = v[u][r][j] + w[j];  // a = g + e
          if constexpr (MODE == kWeightDiff) v[u][r][j] = v[u][r][j] - w[j];     // w_new - w_old
        }
      }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t0 = (base + u) * S::TILE;
      if (base + u >= ntiles) break;
      const bool full = t0 + S::TILE <= n;
      float deq[R][E];
      quantize_tile<BITS, LOG2B, SR, EF>(v[u], t0, n, full, a.out, deq);
      if constexpr (EF) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t i0 = t0 + (int64_t)(r * kWave + lane) * E;
          float e[E];
#pragma unroll
          for (int j = 0; j < E; ++j) e[j] = v[u][r][j] - deq[r][j];     // e = a - deq
          if (full) store_vec_f32<E>(a.resid, i0, e);
          else store_tail_f32<E>(a.resid, i0, n, e);
        }
      }
      (void)deq;
    }
  }
}

}  // namespace lowbit
