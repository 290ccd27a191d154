// reduce.hpp -- local reduce + requantize kernel: the middle stage of a
// low-bit all-reduce.  Up to 16 peer chunks of the same element range are
// decoded, summed in binary32 in peer order and compressed again, in one pass
// over HBM.  Same tile layout as the compress kernel: lane l owns word
// r*64 + l of the tile in every peer chunk and in the output.
//
// The peer loop is not unrolled (the 32 peer pointers stay in the kernel
// argument block and are fetched with scalar loads); the next peer's words
// and scales are loaded while the current peer is decoded.
#pragma once

#include "quantize.hpp"

namespace lowbit {

#ifndef LOWBIT_REDUCE_ELEMS_PER_TRIP
#define LOWBIT_REDUCE_ELEMS_PER_TRIP 16
#endif

template <int PER_LANE>
constexpr int reduce_tiles_per_trip() {
  return PER_LANE >= LOWBIT_REDUCE_ELEMS_PER_TRIP ? 1 : LOWBIT_REDUCE_ELEMS_PER_TRIP / PER_LANE;
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

// Peer loop of one trip: W packed words per lane per peer.  Peers are taken
// in groups of kPeerGroup; all loads of a group are issued before any of its
// peers is decoded, so a whole group's reads are in flight together (the
// group's peer pointers come from the kernel-argument block by scalar loads).
// GUARD: some slots of the trip lie past the end of the buffer (read as 0).
constexpr int kPeerGroup = 8;

template <int BITS, int R, int W, bool GUARD>
__device__ __forceinline__ void reduce_peers(const ReduceArgs& a, const int64_t* wt,
                                             const int64_t* kt, const uint32_t* wl,
                                             const uint32_t* kl, const bool* in,
                                             float (*acc)[Grid<BITS>::E]) {
  const int np = a.npeers;
#pragma unroll 1
  for (int g = 0; g < np; g += kPeerGroup) {
    uint32_t w[kPeerGroup][W], sc[kPeerGroup][W];
#pragma unroll
    for (int q = 0; q < kPeerGroup; ++q) {
      if (g + q < np) {                                   // wave-uniform
        const uint32_t* cp = a.codes[g + q];
        const uint16_t* sp = a.scales[g + q];
#pragma unroll
        for (int i = 0; i < W; ++i) {
          if (GUARD) {
            w[q][i] = 0;
            sc[q][i] = 0;
            if (in[i]) {
              w[q][i] = (cp + wt[i / R])[wl[i]];
              sc[q][i] = (sp + kt[i / R])[kl[i]];
            }
          } else {
            w[q][i] = (cp + wt[i / R])[wl[i]];
            sc[q][i] = (sp + kt[i / R])[kl[i]];
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kPeerGroup; ++q) {
      if (g + q < np) {
#pragma unroll
        for (int i = 0; i < W; ++i) {
          const float s = f16_bits_to_f32(sc[q][i]);
          if (q == 0 && g == 0) accumulate_word<BITS, true>(w[q][i], s, acc[i]);
          else accumulate_word<BITS, false>(w[q][i], s, acc[i]);
        }
      }
    }
  }
}

// Reduce and requantize NT consecutive tiles starting at tile `tile0`.
// GUARD: the tiles may reach past the end of the buffer (only in the tail
// kernel): loads past the end read 0 and those positions are +0 for the
// statistic.
template <int BITS, int LOG2B, bool SR, int NT, bool GUARD>
__device__ __forceinline__ void reduce_tiles(const ReduceArgs& a, int64_t tile0) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R, W = NT * R;
  const int lane = lane_id();
  const int64_t n = a.n;
  const int64_t nwords = (n + E - 1) / E;

  // slot i = (tile u, row r): the tile's first word and block are
  // wave-uniform; the lane's word and block within the tile are 32-bit
  int64_t wt[NT], kt[NT];
  uint32_t wl[W], kl[W];
  bool in[W];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    wt[u] = (tile0 + u) * (S::TILE / E);
    kt[u] = ((tile0 + u) * S::TILE) >> LOG2B;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t w = (uint32_t)(r * kWave + lane);
      wl[u * R + r] = w;
      kl[u * R + r] = (w * E) >> LOG2B;
      in[u * R + r] = !GUARD || wt[u] + w < nwords;
    }
  }

  float acc[NT][R][E];
  reduce_peers<BITS, R, W, GUARD>(a, wt, kt, wl, kl, in, &acc[0][0]);

#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int64_t t0 = (tile0 + u) * S::TILE;
    const bool full = !GUARD || t0 + S::TILE <= n;
    if (!full) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < E; ++j)
          if ((wt[u] + wl[u * R + r]) * E + j >= n) acc[u][r][j] = 0.0f;
    }
    if (a.out_sum) {
      constexpr float UNSCALE = 1.0f / (float)(1 << acc_shift<BITS>());   // exact
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
    float unused[R][E];
    quantize_tile<BITS, LOG2B, SR, false, acc_shift<BITS>()>(acc[u], t0, n, full, a.out, unused);
    (void)unused;
  }
}

// Main kernel (TAIL = false): each wave takes one trip of U full tiles; the
// grid covers the complete trips of full tiles only (`first` = number of full
// tiles).  Tail kernel (TAIL = true, one wave): tiles from `first` on.
template <int BITS, int LOG2B, bool SR, bool TAIL>
__global__ __launch_bounds__(kBlockThreads) void reduce_kernel(ReduceArgs a, int64_t first) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int U = reduce_tiles_per_trip<S::R * S::E>();
  if constexpr (TAIL) {
    if (global_wave_id() != 0) return;
    const int64_t ntiles = (a.n + S::TILE - 1) / S::TILE;
    for (int64_t tile = first; tile < ntiles; ++tile) reduce_tiles<BITS, LOG2B, SR, 1, true>(a, tile);
  } else {
    const int64_t ntrips = first / U;
    const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
    for (int64_t trip = global_wave_id(); trip < ntrips; trip += nwaves)
      reduce_tiles<BITS, LOG2B, SR, U, false>(a, trip * U);
  }
}

}  // namespace lowbit
