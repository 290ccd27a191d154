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

// acc[j] (+)= q_j * s for the E codes of one packed word.  Each code is moved
// to the top of a byte so that the convert reads a sign-extended byte; the
// byte holds 2^(8-b) * q, and the scale is pre-divided by the same power of
// two (exact), so every product is exactly q * s and the fused add rounds
// exactly like acc + q * s.  FIRST: acc[j] = q_j * s.
template <int BITS, bool FIRST>
__device__ __forceinline__ void accumulate_word(uint32_t word, float s, float* acc) {
  using G = Grid<BITS>;
  if constexpr (BITS == 1) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float d = ((word >> j) & 1u) ? s : -s;     // set: +s, clear: -s
      acc[j] = FIRST ? d : acc[j] + d;
    }
  } else {
    constexpr int PER_BYTE = 8 / BITS;
    constexpr uint32_t TOP = (uint32_t)((0xFFu << (8 - BITS)) & 0xFFu) * 0x01010101u;
    const float sb = s * (1.0f / (float)(1 << (8 - BITS)));      // exact power-of-two scaling
    const uint32_t tw = word ^ G::FLIP;                          // two's-complement fields
#pragma unroll
    for (int p = 0; p < PER_BYTE; ++p) {
      const uint32_t t = (tw << (8 - BITS * (p + 1))) & TOP;     // field p of each byte on top
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float qb = (float)(signed char)(t >> (8 * k));    // 2^(8-b) * q
        const int j = PER_BYTE * k + p;
        acc[j] = FIRST ? qb * sb : __builtin_fmaf(qb, sb, acc[j]);
      }
    }
  }
}

template <int BITS, int LOG2B, bool SR>
__global__ __launch_bounds__(kBlockThreads) void reduce_kernel(ReduceArgs a) {
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R;
  constexpr int U = reduce_tiles_per_trip<R * E>();
  constexpr int W = U * R;                       // words per lane per peer per trip

  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * (kBlockThreads / kWave) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t n = a.n;
  const int64_t ntiles = (n + S::TILE - 1) / S::TILE;
  const int64_t nwords = (n + E - 1) / E;
  const int np = a.npeers;

  for (int64_t base = wave * U; base < ntiles; base += nwaves * U) {
    // word and block index of every (tile, row) slot of this lane
    int64_t widx[W], kidx[W];
    bool in[W];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t w0 = (base + u) * (S::TILE / E) + r * kWave + lane;
        widx[u * R + r] = w0;
        kidx[u * R + r] = (w0 * E) >> LOG2B;
        in[u * R + r] = base + u < ntiles && w0 < nwords;
      }

    uint32_t cw[W], cs[W], nw[W], ns[W];
    auto load_peer = [&](int p, uint32_t* w, uint32_t* sc) {
      const uint32_t* cp = a.codes[p];
      const uint16_t* sp = a.scales[p];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        w[i] = 0;
        sc[i] = 0;
        if (in[i]) {
          w[i] = cp[widx[i]];
          sc[i] = sp[kidx[i]];
        }
      }
    };

    float acc[U][R][E];
    load_peer(0, cw, cs);
    if (np > 1) load_peer(1, nw, ns);
#pragma unroll
    for (int i = 0; i < W; ++i)
      accumulate_word<BITS, true>(cw[i], f16_bits_to_f32(cs[i]), acc[i / R][i % R]);
#pragma unroll 1
    for (int p = 1; p < np; ++p) {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        cw[i] = nw[i];
        cs[i] = ns[i];
      }
      if (p + 1 < np) load_peer(p + 1, nw, ns);
#pragma unroll
      for (int i = 0; i < W; ++i)
        accumulate_word<BITS, false>(cw[i], f16_bits_to_f32(cs[i]), acc[i / R][i % R]);
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t0 = (base + u) * S::TILE;
      if (base + u >= ntiles) break;                 // wave-uniform
      const bool full = t0 + S::TILE <= n;
      if (!full) {
        // positions at or past n are +0 for the statistic
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int j = 0; j < E; ++j)
            if (widx[u * R + r] * E + j >= n) acc[u][r][j] = 0.0f;
      }
      if (a.out_sum) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t i0 = t0 + (int64_t)(r * kWave + lane) * E;
          if (full) store_vec_f32<E>(a.out_sum, i0, acc[u][r]);
          else store_tail_f32<E>(a.out_sum, i0, n, acc[u][r]);
        }
      }
      float unused[R][E];
      quantize_tile<BITS, LOG2B, SR, false>(acc[u], t0, n, full, a.out, unused);
      (void)unused;
    }
  }
}

}  // namespace lowbit
