// reduce.hpp -- local reduce + requantize kernel: the middle stage of a
// low-bit all-reduce.  Up to 16 peer chunks of the same element range are
// decoded, summed in binary32 in peer order and compressed again, in one pass
// over HBM.  Same tile layout as the compress kernel, on the output's
// bitwidth and block size: lane l owns output word r*64 + l of the tile.
//
// The peers may be packed with more bits than the output (8-bit intra-node
// codes requantized to 4 bits for the inter-node exchange): an output word
// of E = 32/b_out elements then covers M = b_in/b_out input words, which the
// lane loads as one vector.  The input block size is a run-time value; a
// lane's E elements always lie in one input block (E <= 32 <= input block).
//
// With a residual (stage-2 error feedback) the sum plus the residual is
// quantized and the residual becomes what quantization left behind.
#pragma once

#include "quantize.hpp"

namespace lowbit {

// output elements per lane per trip.  Measured on 8 x 32 Mi peers, b4 B128,
// with the integer sums and scalar scale pointers: 8 elements per lane 34.4
// us with separately allocated peers and 33.1 us in one receive buffer, 16
// elements 33.3 and 32.4 us (the per-wave set-up is shared by twice the
// elements; the kernel issues vector-ALU work most of its time); 8-bit
// B512 -> 4-bit B128: 52-55 us against 50.3 us.
constexpr int kReduceElemsPerTrip = 16;

template <int PER_LANE>
constexpr int reduce_tiles_per_trip() {
  return PER_LANE >= kReduceElemsPerTrip ? 1 : kReduceElemsPerTrip / PER_LANE;
}

// Power of two by which the reduce accumulates: each b-bit code is moved to
// the top of a byte, where the convert reads 2^(8-b) * q as a sign-extended
// byte (b = 1 decodes to +-s directly).
template <int BITS>
constexpr int acc_shift() { return BITS == 1 ? 0 : 8 - BITS; }

// acc[j] (+)= 2^k * q_j * s for the E codes of one packed word, k =
// acc_shift<BITS>().  Every product is exact and every partial sum is zero or
// a normal multiple of 2^-24, so the scaled sums are exactly 2^k times the
// sums acc + q * s rounded in peer order (the fused form rounds once, like the
// plain add of the exact product).  FIRST: acc[j] = 2^k * q_j * s.
template <int BITS, bool FIRST>
__device__ __forceinline__ void accumulate_word(uint32_t word, float s, float* acc) {
  using G = Grid<BITS>;
  if constexpr (BITS == 1) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float d = signed_scale(word, j, s);          // set: +s, clear: -s
      acc[j] = FIRST ? d : acc[j] + d;
    }
  } else {
    constexpr int PER_BYTE = 8 / BITS;
    constexpr uint32_t TOP = (uint32_t)((0xFFu << (8 - BITS)) & 0xFFu) * 0x01010101u;
    const uint32_t tw = word ^ G::FLIP;                          // two's-complement fields
#pragma unroll
    for (int p = 0; p < PER_BYTE; ++p) {
      const uint32_t t = (tw << (8 - BITS * (p + 1))) & TOP;     // field p of each byte on top
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float qb = (float)(signed char)(t >> (8 * k));    // 2^(8-b) * q
        const int j = PER_BYTE * k + p;
        acc[j] = FIRST ? qb * s : __builtin_fmaf(qb, s, acc[j]);
      }
    }
  }
}

// Input words per output word, and their vector load.
template <int IN_BITS, int BITS>
constexpr int in_words() { return IN_BITS / BITS; }

// Load *p: STREAM, non-temporally (the caller reads the line once).
template <bool STREAM, typename T>
__device__ __forceinline__ T load_once(const T* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(p);
  else return *p;
}

// M consecutive code words of one peer.
template <int M, bool STREAM>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t* w) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (M == 1) {
    w[0] = load_once<STREAM>(p);
  } else if constexpr (M == 2) {
    const u32x2* q = reinterpret_cast<const u32x2*>(p);
    const u32x2 t = load_once<STREAM>(q);
    w[0] = t.x;
    w[1] = t.y;
  } else {
#pragma unroll
    for (int k = 0; k < M / 4; ++k) {
      const u32x4* q = reinterpret_cast<const u32x4*>(p) + k;
      const u32x4 t = load_once<STREAM>(q);
      w[4 * k + 0] = t.x;
      w[4 * k + 1] = t.y;
      w[4 * k + 2] = t.z;
      w[4 * k + 3] = t.w;
    }
  }
}

// Peer loop of one trip: W output words per lane, each fed by M input words
// per peer.  Peers are taken in groups of G; all loads of a group are issued
// before any of its peers is decoded, so a whole group's reads are in flight
// together (the group's peer pointers come from the kernel-argument block by
// scalar loads).  G is 8, fewer when a lane's share of a trip is large, so
// that at most 32 loaded words per lane are held at once.  GUARD: some slots
// of the trip lie past the end of the buffer (read as 0).
constexpr int kPeerGroup = 8;
template <int W, int M>
constexpr int peer_group() {
  constexpr int G = kPeerGroup;
  return 32 / (W * M) >= G ? G : (32 / (W * M) >= 1 ? 32 / (W * M) : 1);
}

// The number of peers: NPC when it is fixed at compile time (NPC > 0), else
// the run-time count.  With a fixed count the peer loop is straight-line code:
// the peers' pointers come from the kernel arguments in one batch of scalar
// loads and all of the group's vector loads issue back to back.
template <int NPC>
__device__ __forceinline__ int peer_count(const ReduceArgs& a) {
  return NPC > 0 ? NPC : a.npeers;
}

// Loads of peers g .. g+G-1 (those below the peer count) for the W slots of
// a trip.  The pointers of all G peers are read first (the argument block
// holds kMaxPeers entries and g + G <= kMaxPeers), so that their scalar loads
// are not each waited for between the vector loads of two peers.
template <int IN_BITS, int BITS, int R, int W, int G, bool GUARD, int NPC, bool STREAM>
__device__ __forceinline__ void load_peer_group(const ReduceArgs& a, int g, const int64_t* wt,
                                                const int64_t* kt, const uint32_t* wl,
                                                const uint32_t* kl, const bool* in,
                                                uint32_t (*w)[W][in_words<IN_BITS, BITS>()],
                                                uint32_t (*sc)[W]) {
  constexpr int M = in_words<IN_BITS, BITS>();
  static_assert(kMaxPeers % G == 0, "peer groups tile the argument block");
  const int np = peer_count<NPC>(a);
  const int64_t nwin = (a.n * IN_BITS + 31) / 32;       // input words per peer
  (void)nwin;
  const uint32_t* cps[G];
  const uint16_t* sps[G];
#pragma unroll
  for (int q = 0; q < G; ++q) {
    cps[q] = a.codes[g + q];
    sps[q] = a.scales[g + q];
  }
#pragma unroll
  for (int q = 0; q < G; ++q) {
    if (g + q < np) {                                   // wave-uniform
      const uint32_t* cp = cps[q];
      const uint16_t* sp = sps[q];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        if (GUARD) {
          // word by word: the last output word's input words may end early
          const int64_t w0 = wt[i / R] + (int64_t)wl[i] * M;
#pragma unroll
          for (int m = 0; m < M; ++m) w[q][i][m] = (in[i] && w0 + m < nwin) ? cp[w0 + m] : 0u;
          sc[q][i] = in[i] ? (sp + kt[i / R])[kl[i]] : 0u;
        } else {
          load_words<M, STREAM>(cp + wt[i / R] + wl[i] * M, w[q][i]);
          sc[q][i] = (sp + kt[i / R])[kl[i]];
        }
      }
    }
  }
}

// Decode loaded peers g .. g+G-1 into acc, in peer order (peer 0 starts the
// sums).
template <int IN_BITS, int BITS, int W, int G, int NPC>
__device__ __forceinline__ void decode_peer_group(const ReduceArgs& a, int g,
                                                  const uint32_t (*w)[W][in_words<IN_BITS, BITS>()],
                                                  const uint32_t (*sc)[W],
                                                  float (*acc)[Grid<BITS>::E]) {
  constexpr int M = in_words<IN_BITS, BITS>();
  constexpr int EIN = Grid<IN_BITS>::E;
  const int np = peer_count<NPC>(a);
#pragma unroll
  for (int q = 0; q < G; ++q) {
    if (g + q < np) {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        const float s = f16_bits_to_f32(sc[q][i]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          if (q == 0 && g == 0) accumulate_word<IN_BITS, true>(w[q][i][m], s, acc[i] + m * EIN);
          else accumulate_word<IN_BITS, false>(w[q][i][m], s, acc[i] + m * EIN);
        }
      }
    }
  }
}

// Slot addressing of a trip of NT output tiles from `tile0`: slot i = (tile
// u, row r); the tile's first input word and input block are wave-uniform,
// the lane's output word and input block within the tile are 32-bit.  A tile
// either lies inside one input block or starts on a block boundary, so
// block(t0 + off) = block(t0) + (off >> in_log2b).
template <int IN_BITS, int BITS, int LOG2B, int NT, bool GUARD>
__device__ __forceinline__ void trip_slots(const ReduceArgs& a, int64_t tile0, int64_t* wt,
                                           int64_t* kt, uint32_t* wl, uint32_t* kl, bool* in) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R;
  constexpr int M = in_words<IN_BITS, BITS>();
  const int lane = lane_id();
  const int64_t nwords = (a.n + E - 1) / E;           // output words
  const int lbi = a.in_log2b;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int64_t t0 = (tile0 + u) * S::TILE;
    wt[u] = (t0 / E) * M;
    kt[u] = t0 >> lbi;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t w = (uint32_t)(r * kWave + lane);
      wl[u * R + r] = w;
      kl[u * R + r] = (w * E) >> lbi;
      in[u * R + r] = !GUARD || t0 / E + w < nwords;
    }
  }
}

// The stage-2 residual of the lane's elements of NT tiles from `tile0`.
template <int BITS, int LOG2B, int NT, bool GUARD>
__device__ __forceinline__ void load_residual(
    const ReduceArgs& a, int64_t tile0,
    float (*e)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E]) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R;
  const int lane = lane_id();
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int64_t t0 = (tile0 + u) * S::TILE;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t off = (uint32_t)(r * kWave + lane) * E;
      if (!GUARD || t0 + S::TILE <= a.n) load_vec<kF32, E>(a.resid, t0, off, e[u][r]);
      else load_tail<kF32, E>(a.resid, t0, off, a.n - t0, e[u][r]);
    }
  }
}

// From the peer sums of NT tiles (scaled by 2^acc_shift<IN_BITS>): zero the
// positions past the end, write the optional sum, add the residual (EF),
// requantize, and write the new residual (EF).
template <int IN_BITS, int BITS, int LOG2B, bool SR, bool EF, int NT, bool GUARD>
__device__ __forceinline__ void requant_tiles(
    const ReduceArgs& a, int64_t tile0,
    float (*acc)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E],
    const float (*e)[TileShape<BITS, LOG2B>::R][Grid<BITS>::E]) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R;
  constexpr int K = acc_shift<IN_BITS>();
  constexpr float UNSCALE = 1.0f / (float)(1 << K);              // exact
  // the statistic can absorb the 2^K of the sums unless it is the 1-bit mean
  // or a residual is added first
  constexpr bool UNSCALE_FIRST = EF || (BITS == 1 && K > 0);
  const int lane = lane_id();
  const int64_t n = a.n;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int64_t t0 = (tile0 + u) * S::TILE;
    const bool full = !GUARD || t0 + S::TILE <= n;
    if (!full) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < E; ++j)
          if (t0 + (int64_t)(r * kWave + lane) * E + j >= n) acc[u][r][j] = 0.0f;
    }
    if (a.out_sum) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t off = (uint32_t)(r * kWave + lane) * E;
        float sum[E];
#pragma unroll
        for (int j = 0; j < E; ++j) sum[j] = acc[u][r][j] * UNSCALE;
        if (full) store_vec_f32<E>(a.out_sum, t0, off, sum);
        else store_tail_f32<E>(a.out_sum, t0, off, n - t0, sum);
      }
    }
    float deq[R][E];
    if constexpr (UNSCALE_FIRST) {
      // a = fl(sum + e): positions past the end stay +0 (e reads 0 there)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < E; ++j) {
          acc[u][r][j] = acc[u][r][j] * UNSCALE;
          if constexpr (EF) acc[u][r][j] = acc[u][r][j] + e[u][r][j];
        }
      quantize_tile<BITS, LOG2B, SR, EF, 0>(acc[u], t0, n, full, a.out, deq);
    } else {
      quantize_tile<BITS, LOG2B, SR, false, K>(acc[u], t0, n, full, a.out, deq);
    }
    if constexpr (EF) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t off = (uint32_t)(r * kWave + lane) * E;
        float en[E];
#pragma unroll
        for (int j = 0; j < E; ++j) en[j] = acc[u][r][j] - deq[r][j];   // e = a - deq
        if (full) store_vec_f32<E>(a.resid, t0, off, en);
        else store_tail_f32<E>(a.resid, t0, off, n - t0, en);
      }
    }
    (void)deq;
  }
  (void)e;
}

// ------------------------------------------------------------ exact sums --
// Eight peers of 4- or 8-bit codes whose block scales lie within a factor
// 2^D of each other (D = 5 at 4 bits, 3 at 8 bits): the peer-ordered binary32
// sum then never rounds.  With u = 2^(Emin - 25) the unit of the smallest
// nonzero scale (Emin its binary16 exponent field, 1 for a subnormal), every
// scale is s_p = M_p * u with M_p = significand * 2^(E_p - Emin) an integer
// below 2^16, every term q_p * s_p is an integer multiple of u, and every
// partial sum is at most qmax * sum_p M_p < 2^24 units in magnitude, so each
// binary32 addition is exact and the sum is S * u, S = sum_p q_p * M_p.  S is
// formed exactly in 32-bit integers, two peers per v_dot2_u32_u16 on the
// offset codes (S = sum_p c_p * M_p - 2^(b-1) * sum_p M_p), and float(S) * u
// (both exact) is bit-identical to the rounded peer-ordered sum.  A wave in
// which any block misses the condition takes the binary32 path.
template <int BITS>
constexpr uint32_t exact_spread() { return BITS == 4 ? 5u : 3u; }

template <int IN_BITS, int BITS, int LOG2B, int NPC>
constexpr bool exact_path() {
  return NPC == 8 && IN_BITS == BITS && (BITS == 4 || BITS == 8) &&
         TileShape<BITS, LOG2B>::L >= 8;
}

// Reductions of unsigned values over aligned groups of 8 lanes (every lane of
// a group ends with the result), and the value of lane Q of the lane's group.
__device__ __forceinline__ uint32_t group8_min(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(v));     // quad_perm [1,0,3,2]
  v = min(v, dpp_u32<0x4E>(v));     // quad_perm [2,3,0,1]
  return min(v, dpp_u32<0x141>(v)); // row_half_mirror: the other quad
}
__device__ __forceinline__ uint32_t group8_max(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  return max(v, dpp_u32<0x141>(v));
}
__device__ __forceinline__ uint32_t group8_add(uint32_t v) {
  v += dpp_u32<0xB1>(v);
  v += dpp_u32<0x4E>(v);
  return v + dpp_u32<0x141>(v);
}
template <int Q>
__device__ __forceinline__ uint32_t group8_lane(uint32_t v) {
  // ds_swizzle bit mode: lane (id & 0x18) | Q within each 32 lanes
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x18 | (Q << 5));
}

// 2^x as a binary32 value (x a normal exponent)
__device__ __forceinline__ float pow2_f32(int x) { return __uint_as_float((uint32_t)(x + 127) << 23); }

// Loads and peer sums of one trip of NT full tiles for exactly eight peers
// (exact_path): acc as decode_peer_group leaves it, i.e. 2^acc_shift<BITS>()
// times the peer-ordered binary32 sums.
// The scale array of peer p = lane & 7, the peer whose scales this lane
// loads (a block spans at least 8 lanes, so each aligned group of 8 lanes
// holds all eight).  The eight pointers are made wave-uniform first, so that
// they are read with the scalar loads of the argument block and selected per
// lane in registers; a per-lane choice among argument-block slots would
// otherwise become a vector load of the pointer, which the code word loads
// then wait behind.
__device__ __forceinline__ global_ptr<uint16_t> peer_scale_ptr(const ReduceArgs& a) {
  const int p = lane_id() & 7;
  global_ptr<uint16_t> sq[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) sq[q] = uniform_ptr(a.scales[q]);
  const global_ptr<uint16_t> s01 = (p & 1) ? sq[1] : sq[0];
  const global_ptr<uint16_t> s23 = (p & 1) ? sq[3] : sq[2];
  const global_ptr<uint16_t> s45 = (p & 1) ? sq[5] : sq[4];
  const global_ptr<uint16_t> s67 = (p & 1) ? sq[7] : sq[6];
  const global_ptr<uint16_t> s03 = (p & 2) ? s23 : s01;
  const global_ptr<uint16_t> s47 = (p & 2) ? s67 : s45;
  return (p & 4) ? s47 : s03;
}

// Loads of one trip of NT full tiles for exactly eight peers: the code words
// of every peer and slot, and per slot the scale of peer lane & 7 (sp).
template <int BITS, int LOG2B, int NT, bool STREAM>
__device__ __forceinline__ void reduce8_load(
    const ReduceArgs& a, global_ptr<uint16_t> sp, const int64_t* wt, const int64_t* kt,
    const uint32_t* wl, const uint32_t* kl,
    uint32_t (*w)[TileShape<BITS, LOG2B>::R * NT][1], uint32_t* s16) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int R = S::R, W = NT * R;
  // the code words of all eight peers (pointers read in one batch)
  const uint32_t* cps[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) cps[q] = a.codes[q];
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int i = 0; i < W; ++i) w[q][i][0] = load_once<STREAM>(cps[q] + wt[i / R] + wl[i]);
#pragma unroll
  for (int i = 0; i < W; ++i) s16[i] = (sp + kt[i / R])[kl[i]];
}

// Peer sums of a loaded trip (reduce8_load): acc as decode_peer_group leaves
// it, i.e. 2^acc_shift<BITS>() times the peer-ordered binary32 sums.
template <int BITS, int LOG2B, int NT>
__device__ __forceinline__ void reduce8_sums_loaded(
    const ReduceArgs& a, const uint32_t (*w)[TileShape<BITS, LOG2B>::R * NT][1],
    const uint32_t* s16, float (*acc)[Grid<BITS>::E]) {
  using S = TileShape<BITS, LOG2B>;
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  constexpr int E = S::E, R = S::R, W = NT * R;
  constexpr int K = acc_shift<BITS>();
  constexpr uint32_t HALF = Grid<BITS>::HALF;
  (void)R;
  // per slot: exponent range of the group's nonzero scales
  uint32_t lo[W];
  bool ok = true;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t e = (s16[i] >> 10) & 31u;
    const uint32_t ep = e != 0 ? e : 1u;
    const bool nz = s16[i] != 0;
    lo[i] = group8_min(nz ? ep : 31u);
    const uint32_t hi = group8_max(nz ? ep : 0u);
    ok = ok && (hi == 0 || hi <= lo[i] + exact_spread<BITS>());
  }
  if (__all(ok)) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const uint32_t e = (s16[i] >> 10) & 31u;
      const uint32_t ep = e != 0 ? e : 1u;
      const uint32_t m = (s16[i] & 0x3FFu) | (e != 0 ? 0x400u : 0u);
      const uint32_t M = s16[i] != 0 ? m << (ep - lo[i]) : 0u;    // < 2^16
      const uint32_t sumM = group8_add(M);
      const uint32_t pair = M | (dpp_u32<0xB1>(M) << 16);          // peers p, p ^ 1
      const u16x2 mp[4] = {__builtin_bit_cast(u16x2, group8_lane<0>(pair)),
                           __builtin_bit_cast(u16x2, group8_lane<2>(pair)),
                           __builtin_bit_cast(u16x2, group8_lane<4>(pair)),
                           __builtin_bit_cast(u16x2, group8_lane<6>(pair))};
      // 8 bits: sum[k] = sum_p M_p (c_pk - HALF), codes c as unsigned bytes.
      // 4 bits: byte k of a word holds elements 2k (low nibble l) and 2k + 1
      // (high nibble h); sum[2k + 1] = sum_p M_p 16 (h - 8) from the high
      // nibbles in place, and sum[2k] first takes the whole bytes,
      // sum_p M_p (l + 16 h) - 136 sum M, from which sum[2k + 1] is taken
      // away at the end: sum_p M_p (l - 8).  (Modulo 2^32 throughout; each
      // result is below 2^23 in magnitude, so it is exact as int32.)
      uint32_t sum[E];
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const uint32_t f = BITS == 4 ? ((j & 1) ? 16u * HALF : 17u * HALF) : HALF;
        sum[j] = 0u - f * sumM;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t we = w[2 * j][i][0], wo = w[2 * j + 1][i][0];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // bytes k of the two peers' words in the two 16-bit halves
          const uint32_t sel = (uint32_t)k | (0x0Cu << 8) | ((4u + k) << 16) | (0x0Cu << 24);
          const uint32_t b2 = __builtin_amdgcn_perm(wo, we, sel);
          if constexpr (BITS == 4) {
            sum[2 * k] = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, b2), mp[j], sum[2 * k],
                                                false);
            sum[2 * k + 1] = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, b2 & 0x00F000F0u),
                                                    mp[j], sum[2 * k + 1], false);
          } else {
            sum[k] = __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2, b2), mp[j], sum[k], false);
          }
        }
      }
      if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) sum[2 * k] -= sum[2 * k + 1];
      }
      // binary32 sums, scaled like the binary32 path's: 2^K * S * u
      const int x = (int)(lo[i] < 30u ? lo[i] : 30u) - 25 + K;
      const float unit = pow2_f32(x), unit16 = pow2_f32(x - 4);
#pragma unroll
      for (int j = 0; j < E; ++j)
        acc[i][j] = (float)(int)sum[j] * ((BITS == 4 && (j & 1)) ? unit16 : unit);
    }
  } else {
    // the binary32 path, with every peer's scale from the lane's group
    uint32_t sc[8][W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      sc[0][i] = group8_lane<0>(s16[i]);
      sc[1][i] = group8_lane<1>(s16[i]);
      sc[2][i] = group8_lane<2>(s16[i]);
      sc[3][i] = group8_lane<3>(s16[i]);
      sc[4][i] = group8_lane<4>(s16[i]);
      sc[5][i] = group8_lane<5>(s16[i]);
      sc[6][i] = group8_lane<6>(s16[i]);
      sc[7][i] = group8_lane<7>(s16[i]);
    }
    decode_peer_group<BITS, BITS, W, 8, 8>(a, 0, w, sc, acc);
  }
}

// Loads and peer sums of one trip of NT full tiles for exactly eight peers
// (exact_path).
template <int BITS, int LOG2B, int NT, bool STREAM>
__device__ __forceinline__ void reduce8_sums(const ReduceArgs& a, const int64_t* wt,
                                             const int64_t* kt, const uint32_t* wl,
                                             const uint32_t* kl, float (*acc)[Grid<BITS>::E]) {
  constexpr int W = NT * TileShape<BITS, LOG2B>::R;
  uint32_t w[8][W][1], s16[W];
  reduce8_load<BITS, LOG2B, NT, STREAM>(a, peer_scale_ptr(a), wt, kt, wl, kl, w, s16);
  reduce8_sums_loaded<BITS, LOG2B, NT>(a, w, s16, acc);
}

// Reduce and requantize NT consecutive output tiles starting at tile `tile0`,
// any number of peers (groups of G: all loads of a group are issued before
// any of its peers is decoded; NPC > 0: exactly NPC peers).  GUARD: the tiles
// may reach past the end of the buffer (only in the tail kernel): loads past
// the end read 0 and those positions are +0 for the statistic.  EF: stage-2
// error feedback with the residual a.resid.
template <int IN_BITS, int BITS, int LOG2B, bool SR, bool EF, int NT, bool GUARD, int NPC = 0,
          bool STREAM = false>
__device__ __forceinline__ void reduce_tiles(const ReduceArgs& a, int64_t tile0) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R, W = NT * R;
  constexpr int M = in_words<IN_BITS, BITS>();
  constexpr int G = peer_group<W, M>();
  int64_t wt[NT], kt[NT];
  uint32_t wl[W], kl[W];
  bool in[W];
  trip_slots<IN_BITS, BITS, LOG2B, NT, GUARD>(a, tile0, wt, kt, wl, kl, in);
  // stage-2 residual of the lane's elements, in flight with the first peers
  float e[NT][R][E];
  if constexpr (EF) load_residual<BITS, LOG2B, NT, GUARD>(a, tile0, e);
  float acc[NT][R][E];
  if constexpr (!GUARD && exact_path<IN_BITS, BITS, LOG2B, NPC>()) {
    reduce8_sums<BITS, LOG2B, NT, STREAM>(a, wt, kt, wl, kl, &acc[0][0]);
  } else if constexpr (NPC > 0) {
#pragma unroll
    for (int g = 0; g < NPC; g += G) {
      uint32_t w[G][W][M], sc[G][W];
      load_peer_group<IN_BITS, BITS, R, W, G, GUARD, NPC, STREAM>(a, g, wt, kt, wl, kl, in, w,
                                                                  sc);
      decode_peer_group<IN_BITS, BITS, W, G, NPC>(a, g, w, sc, &acc[0][0]);
    }
  } else {
#pragma unroll 1
    for (int g = 0; g < a.npeers; g += G) {
      uint32_t w[G][W][M], sc[G][W];
      load_peer_group<IN_BITS, BITS, R, W, G, GUARD, 0, STREAM>(a, g, wt, kt, wl, kl, in, w, sc);
      decode_peer_group<IN_BITS, BITS, W, G, 0>(a, g, w, sc, &acc[0][0]);
    }
  }
  requant_tiles<IN_BITS, BITS, LOG2B, SR, EF, NT, GUARD>(a, tile0, acc, e);
}

// Main kernel (TAIL = false): each wave takes one trip of U full tiles; the
// grid covers the complete trips of full tiles only (`first` = number of full
// tiles).  Tail kernel (TAIL = true, one wave): tiles from `first` on.
// (Measured: a grid of a few workgroups per CU whose waves walk several trips
// and issue the next trip's loads before decoding the current one is 30 %
// slower on 8 x 32 Mi peers than one trip per wave.)
// Waves per SIMD the register allocation must allow (1: no bound) for the
// same-width main kernels of blocks up to 1024 elements: measured on 8 x 32 Mi
// peers, b4 B128, 84 VGPRs (5 waves) 32.1 us in one receive buffer, 68 VGPRs
// (7 waves) 30.1 us, with no scratch; the step's 8-bit reduce of 8 Mi
// shares (B256, nearest) 21.5 -> 20.8 us at 5 waves.  The bound is chosen per
// kernel so that none spills (1 bit: 91 VGPRs, 5 waves; 2 bits: 57-60, 8
// waves; 4 bits: 67-71, 7 waves; 8 bits with nearest rounding and blocks up
// to 512: 96, 5 waves); the 8-bit stochastic-rounding kernels and the mixed
// widths would spill (or measured no faster: 8 -> 4 bits at 6 waves).
template <int IN_BITS, int BITS, int LOG2B, bool SR, bool EF, bool TAIL>
constexpr int reduce_min_waves() {
  if (TAIL || EF || LOG2B > 10 || IN_BITS != BITS) return 1;
  if (BITS == 8) return (!SR && LOG2B <= 9) ? 5 : 1;
  return BITS == 2 ? 8 : BITS == 4 ? 7 : 5;
}

// STREAM: the peers' code words are read non-temporally (main kernel only).
template <int IN_BITS, int BITS, int LOG2B, bool SR, bool EF, bool TAIL, bool STREAM = false>
__global__ __launch_bounds__(kBlockThreads) __attribute__((
    amdgpu_waves_per_eu(reduce_min_waves<IN_BITS, BITS, LOG2B, SR, EF, TAIL>()))) void
reduce_kernel(ReduceArgs a, int64_t first) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int U = reduce_tiles_per_trip<S::R * S::E>();
  if constexpr (TAIL) {
    if (global_wave_id() != 0) return;
    const int64_t ntiles = (a.n + S::TILE - 1) / S::TILE;
    for (int64_t tile = first; tile < ntiles; ++tile)
      reduce_tiles<IN_BITS, BITS, LOG2B, SR, EF, 1, true>(a, tile);
  } else {
    const int64_t ntrips = first / U;
    const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
    const int64_t trip = global_wave_id();
    // eight peers (one per GPU of an 8-GPU node): the straight-line form.
    // The grid gives every wave one trip; the loop only runs where the grid
    // was capped (more than 2^32 work-items), so the first trip is kept out
    // of it and its addresses are not carried from trip to trip.  (Waves
    // that take two trips and issue the second trip's loads before the first
    // trip's sums measured no faster: 8 x 32 Mi b4 in one receive buffer
    // 33.6 against 31.9 us.)
    if (a.npeers == 8) {
      if (trip < ntrips)
        reduce_tiles<IN_BITS, BITS, LOG2B, SR, EF, U, false, 8, STREAM>(a, trip * U);
    } else {
      if (trip < ntrips)
        reduce_tiles<IN_BITS, BITS, LOG2B, SR, EF, U, false, 0, STREAM>(a, trip * U);
    }
    for (int64_t t = trip + nwaves; t < ntrips; t += nwaves)
      reduce_tiles<IN_BITS, BITS, LOG2B, SR, EF, U, false, 0, STREAM>(a, t * U);
  }
}

}  // namespace lowbit
