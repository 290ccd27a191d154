// quantize.hpp -- blockwise compress of one tile held in registers, and the
// compress kernel built on it (plain, error feedback, weight difference,
// EF21, Hadamard-smoothed).
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
#include "hadamard.hpp"

namespace lowbit {

// Hadamard-smoothed compress spends more vector-ALU work per element; it
// takes more tiles per trip to keep more loads in flight per wave (32
// elements per lane: 65 % of peak against 59 % with 8).
constexpr int kHsElemsPerTrip = 32;

// Error-feedback compresses read two streams and write one; a single tile
// per trip keeps their register use and per-wave footprint small.
constexpr int kEfElemsPerTrip = 8;

// Tiles per trip of the compress kernel for a tile of PER_LANE elements per
// lane, by rounding, input type and mode.
template <int PER_LANE, bool SR, int DT, int MODE>
constexpr int compress_tiles_per_trip() {
  if constexpr (MODE == kErrorFeedback || MODE == kEF21) {
    constexpr int want = kEfElemsPerTrip;
    return PER_LANE >= want ? 1 : want / PER_LANE;
  } else if constexpr (MODE == kHadamard) {
    constexpr int want = kHsElemsPerTrip;
    return PER_LANE >= want ? 1 : want / PER_LANE;
  } else {
    return tiles_per_trip<PER_LANE, SR>();
  }
}

template <int BITS, int LOG2B>
struct TileShape {
  static constexpr int E = Grid<BITS>::E;
  static constexpr int B = 1 << LOG2B;
  static constexpr int ROW = kWave * E;                  // elements per row of words
  static constexpr int R = B > ROW ? B / ROW : 1;        // rows per tile
  static constexpr int TILE = ROW * R;                   // elements per tile
  static constexpr int L = B > ROW ? kWave : B / E;      // lanes per block
};

// Quantize the tile starting at element t0 whose values are 2^-K * v[r][j]
// (element t0 + (r*64 + lane)*E + j; positions at or past n must hold +0).
// Stores the codes and scales; when WANT_DEQ, deq[r][j] receives the
// dequantized values.  K > 0 lets a caller hand over values it accumulated
// scaled by 2^K: the statistic and the reciprocal absorb the exact factor, so
// the codes are those of the unscaled values (no value here is subnormal).
// GRAY: the first products of the SR hash by GrayProducts (one add per
// element instead of a multiply, a few more instructions per word): the
// Hadamard-smoothed compress, bound by the vector ALU, 58.4 -> 57.5 us (4-bit
// B128, 64 Mi); the other compresses are faster with the multiplies (4-bit
// B256 alone 49.6 -> 50.0 us).
template <int BITS, int LOG2B, bool SR, bool WANT_DEQ, int K = 0, bool GRAY = false>
__device__ __forceinline__ void quantize_tile(
    const float (&v)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E], int64_t t0, int64_t n,
    bool full, const TileOut& o, float (&deq)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E]) {
  using G = Grid<BITS>;
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R, L = S::L, B = S::B;
  constexpr float QMAX = (float)G::QMAX;
  constexpr float UNSCALE = 1.0f / (float)(1 << K);       // exact power of two
  static_assert(K == 0 || BITS > 1, "scaled input is only for the max statistic");
  const int lane = lane_id();

  // ---- 1 bit: the codes are the signs and need no scale; take them first so
  // that the values are only needed by the sum tree afterwards
  uint32_t sign_word[R];
  if constexpr (BITS == 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) sign_word[r] = sign_codes<E>(v[r]);
  }

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
    t = div_by_grid<G::QMAX>(group_max_nonneg<L>(m) * UNSCALE);
  }
  const BlockScale sc = make_scale(t);
  const float inv = sc.inv * UNSCALE;
  if ((lane & (L - 1)) == 0 && blk0 < n)
    (o.scales + (t0 >> LOG2B))[R == 1 ? lane / L : 0] = (uint16_t)sc.s16;

  // ---- codes and packing ---------------------------------------------------
  uint32_t* const cbase = o.codes + t0 / E;           // the tile's first word
  const HiMix hm(o.index_offset + (uint64_t)t0, o.key);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t wl = (uint32_t)(r * kWave + lane);  // word within the tile
    const int64_t i0 = t0 + (int64_t)wl * E;           // its first element
    uint32_t word;
    if constexpr (BITS == 1) {
      word = sign_word[r];
      if constexpr (WANT_DEQ) {
#pragma unroll
        for (int j = 0; j < E; ++j) deq[r][j] = signed_scale(word, j, sc.s);
      }
    } else {
      // SR packs the codes' signed integer values onto the offset of every
      // field (FLIP); nearest rounding packs bit patterns of q + kMagic onto
      // PACK_BIAS.  Either way the fields never carry into one another.
      word = SR ? G::FLIP : G::PACK_BIAS;
      // SR: h_j = fmix32((lo + j) ^ hk) for the word's elements j < E.  lo
      // (the low half of the first element's global index) is a multiple of
      // E, so lo + j = lo ^ j, and j < 2^16 leaves x >> 16 unchanged: the
      // first fmix32 step, x ^ (x >> 16), is c ^ j with c computed once.
      // The word's elements go in Gray-code order, so that the first hash
      // products can follow one another by an add (GrayProducts); the
      // packing adds are exact, so the order does not change the word.
      uint32_t c = 0;
      if constexpr (SR) {
        const uint32_t x0 = hm.x0(wl * (uint32_t)E);
        c = x0 ^ (x0 >> 16);
      }
      GrayProducts<E> gp(c);
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const int j = GrayProducts<E>::index(k);
        if (k > 0) gp.step(k);
        const float x = v[r][j] * inv;
        if constexpr (SR) {
          const uint32_t h = GRAY ? fmix32_after_first_multiply(gp.p)
                                  : fmix32_after_first_step(c ^ (uint32_t)j);
          // the random offset (h >> 8) * 2^-24 is exact, so the fused form
          // rounds once, exactly like adding it in binary32.
          const float y = __builtin_fmaf((float)(h >> 8), 0x1p-24f, x);
          const int q = min(max(floor_to_int(y), -G::QMAX), G::QMAX);
          word += (uint32_t)q << (j * BITS);
          if constexpr (WANT_DEQ) deq[r][j] = (float)q * sc.s;
        } else {
          // clamp, then round: the same as rounding then clamping because the
          // bounds are integers; with |q| <= QMAX adding 1.5 * 2^23 rounds to
          // the nearest integer, ties to even.
          const float q = __builtin_amdgcn_fmed3f(x, -QMAX, QMAX);
          const float t = q + kMagic;
          word += __float_as_uint(t) << (j * BITS);
          if constexpr (WANT_DEQ) deq[r][j] = (t - kMagic) * sc.s;
        }
      }
    }
    if (full) {
      store_stream(cbase + wl, word);
    } else if (i0 < n) {
      const int64_t valid = n - i0;
      if (valid < E) word &= (1u << (valid * BITS)) - 1u;
      store_stream(cbase + wl, word);
    }
  }
}

// The plain and Hadamard-smoothed compresses of binary32 input with more than
// four elements per lane (1, 2 and 4 bits: a lane's word spans 128, 64 or 32
// bytes, so each 16-byte load instruction of a wave would touch half lines
// that the next one fetches again) read their tiles through LDS (the
// Hadamard compress a whole trip of tiles at once: 4-bit B128 on 64 Mi
// elements 57.0 -> 54.2 us, streamed): the wave loads the tile with coalesced
// 16-byte loads (lane l takes bytes 16 * (64 k + l) of the tile, each
// instruction one contiguous kilobyte) -- non-temporal when streamed --,
// writes them to its own LDS slice and reads back its E consecutive elements.
// A wave's LDS accesses execute in order, so no barrier is needed; the wave
// barriers keep the compiler from moving the reads above the writes, or a
// row's writes above the previous row's reads (the R rows of a tile pass
// through the wave's one slice in turn, after all their global loads have
// been issued).
template <int MODE, int DT, int E, int R>
constexpr bool staged_tile() {
  return (MODE == kPlain || MODE == kHadamard) && DT == kF32 && E > 4;
}

// The R rows of 64 words of the tile at element t0.
template <int E, int R, bool NT>
__device__ __forceinline__ void load_tile_staged(const float* x, int64_t t0, float (&v)[R][E]) {
  constexpr int Q = E / 4;                               // 16-byte pieces per lane
  __shared__ f32x4 stage[kBlockThreads / kWave][kWave * Q];
  f32x4* st = stage[threadIdx.x >> 6];
  const int lane = lane_id();
  const f32x4* src = reinterpret_cast<const f32x4*>(x + t0);
  f32x4 t[R][Q];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int k = 0; k < Q; ++k) {
      const f32x4* p = src + (r * Q + k) * kWave + lane;
      t[r][k] = NT ? __builtin_nontemporal_load(p) : *p;
    }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < Q; ++k) st[k * kWave + lane] = t[r][k];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      const f32x4 u = st[lane * Q + j];
      v[r][4 * j + 0] = u.x;
      v[r][4 * j + 1] = u.y;
      v[r][4 * j + 2] = u.z;
      v[r][4 * j + 3] = u.w;
    }
  }
}

// Load one tile's values (x, plus the residual or minus the old weights or
// minus the EF21 state).  EF21 keeps the state in `h` for finish_tile.
template <int BITS, int LOG2B, int DT, int MODE, bool FULL, bool NTX = false>
__device__ __forceinline__ void load_tile(const QuantArgs& a, int64_t t0,
                                          float (&v)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E],
                                          float (&h)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E]) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R;
  const int lane = lane_id();
  if constexpr (FULL && MODE == kPlain && staged_tile<MODE, DT, E, R>()) {
    // the plain mode: x alone
    load_tile_staged<E, R, NTX>(static_cast<const float*>(a.x), t0, v);
    (void)h;
    return;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t off = (uint32_t)(r * kWave + lane) * E;
    float w[E];
    if constexpr (FULL) {
      constexpr bool RMW = MODE == kErrorFeedback || MODE == kEF21;
      load_vec<DT, E, NTX && E == 4 && stream_capable<MODE, DT, E, R>()>(a.x, t0, off, v[r]);
      if constexpr (RMW) load_vec<kF32, E>(a.resid, t0, off, w);
      if constexpr (MODE == kWeightDiff) load_vec<DT, E>(a.x2, t0, off, w);
    } else {
      load_tail<DT, E>(a.x, t0, off, a.n - t0, v[r]);
      if constexpr (MODE == kErrorFeedback || MODE == kEF21)
        load_tail<kF32, E>(a.resid, t0, off, a.n - t0, w);
      if constexpr (MODE == kWeightDiff) load_tail<DT, E>(a.x2, t0, off, a.n - t0, w);
    }
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if constexpr (MODE == kErrorFeedback) v[r][j] = v[r][j] + w[j];   // a = g + e
      if constexpr (MODE == kWeightDiff) v[r][j] = v[r][j] - w[j];      // w_new - w_old
      if constexpr (MODE == kEF21) {
        v[r][j] = v[r][j] - w[j];                                       // d = g - h
        h[r][j] = w[j];
      }
    }
  }
  // the tile holds whole blocks: B / E lanes of one row, or all R rows
  if constexpr (MODE == kHadamard) {
    if constexpr (FULL) {
      hadamard_rows<R, E, S::L, R>(v, hadamard_forward_scale<LOG2B>());
    } else {
      // a partial last block is compressed untransformed: every lane takes
      // part in the exchanges, then that block's lanes take back their loads
      float v0[R][E];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < E; ++j) v0[r][j] = v[r][j];
      hadamard_rows<R, E, S::L, R>(v, hadamard_forward_scale<LOG2B>());
      const int64_t blk0 = (R == 1) ? t0 + (int64_t)(lane / S::L) * S::B : t0;
      if (blk0 + S::B > a.n) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int j = 0; j < E; ++j) v[r][j] = v0[r][j];
      }
    }
  }
}

// Quantize one loaded tile; in error-feedback mode also write e = a - deq,
// in EF21 mode h + deq.
template <int BITS, int LOG2B, bool SR, int MODE, bool FULL>
__device__ __forceinline__ void finish_tile(const QuantArgs& a, int64_t t0,
                                            const float (&v)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E],
                                            const float (&h)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E]) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R;
  constexpr bool WANT_DEQ = MODE == kErrorFeedback || MODE == kEF21;
  const int lane = lane_id();
  float deq[R][E];
  quantize_tile<BITS, LOG2B, SR, WANT_DEQ, 0, MODE == kHadamard>(v, t0, a.n, FULL, a.out, deq);
  if constexpr (WANT_DEQ) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t off = (uint32_t)(r * kWave + lane) * E;
      float e[E];
#pragma unroll
      for (int j = 0; j < E; ++j) {
        if constexpr (MODE == kErrorFeedback) e[j] = v[r][j] - deq[r][j];   // e = a - deq
        else e[j] = h[r][j] + deq[r][j];                                    // h + deq
      }
      if constexpr (FULL) store_vec_f32<E>(a.resid, t0, off, e);
      else store_tail_f32<E>(a.resid, t0, off, a.n - t0, e);
    }
  }
  (void)deq;
  (void)h;
}

// Main kernel (TAIL = false): each wave takes one trip of U full tiles -- all
// of their loads are issued before any of them is quantized -- and the grid
// covers the complete trips of full tiles only, so this code has no bounds
// checks.  Tail kernel (TAIL = true, launched with one wave when needed):
// the remaining tiles from tile `first`, the last of which may be partial.
// NTX: read x with non-temporal loads where stream_capable.
template <int BITS, int LOG2B, bool SR, int DT, int MODE, bool TAIL, bool NTX = false>
__global__ __launch_bounds__(kBlockThreads) void quantize_kernel(QuantArgs a, int64_t first) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R;
  constexpr int U = compress_tiles_per_trip<R * E, SR, DT, MODE>();

  if constexpr (TAIL) {
    if (global_wave_id() != 0) return;
    const int64_t ntiles = (a.n + S::TILE - 1) / S::TILE;
    for (int64_t tile = first; tile < ntiles; ++tile) {
      const int64_t t0 = tile * S::TILE;
      float v[R][E], h[R][E];
      if (t0 + S::TILE <= a.n) {
        load_tile<BITS, LOG2B, DT, MODE, true>(a, t0, v, h);
        finish_tile<BITS, LOG2B, SR, MODE, true>(a, t0, v, h);
      } else {
        load_tile<BITS, LOG2B, DT, MODE, false>(a, t0, v, h);
        finish_tile<BITS, LOG2B, SR, MODE, false>(a, t0, v, h);
      }
    }
  } else {
    const int64_t ntrips = first / U;                 // first = number of full tiles
    const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
    for_each_trip(global_wave_id(), ntrips, nwaves, [&](int64_t trip) __attribute__((always_inline)) {
      float v[U][R][E], h[U][R][E];
      if constexpr (MODE == kHadamard && staged_tile<MODE, DT, E, R>()) {
        // the trip's U tiles are U * R consecutive rows of words: all their
        // loads are issued first, then each row passes through LDS
        load_tile_staged<E, U * R, NTX>(static_cast<const float*>(a.x), trip * U * S::TILE,
                                        reinterpret_cast<float (&)[U * R][E]>(v));
#pragma unroll
        for (int u = 0; u < U; ++u)
          hadamard_rows<R, E, S::L, R>(v[u], hadamard_forward_scale<LOG2B>());
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u)
          load_tile<BITS, LOG2B, DT, MODE, true, NTX>(a, (trip * U + u) * S::TILE, v[u], h[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        finish_tile<BITS, LOG2B, SR, MODE, true>(a, (trip * U + u) * S::TILE, v[u], h[u]);
    });
  }
}

}  // namespace lowbit
