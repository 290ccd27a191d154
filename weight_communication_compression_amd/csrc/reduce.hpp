// reduce.hpp -- local reduce + requantize kernel: the middle stage of a
// low-bit all-reduce.  Up to 16 peer chunks of the same element range are
// decoded, summed in binary32 in peer order and compressed again, in one pass
// over HBM.  Same tile layout as the compress kernel: lane l owns word
// r*64 + l of the tile in every peer chunk and in the output.
#pragma once

#include "quantize.hpp"

namespace lowbit {

template <int BITS, int LOG2B, bool SR>
__global__ __launch_bounds__(kBlockThreads) void reduce_kernel(ReduceArgs a) {
  using G = Grid<BITS>;
  using S = TileShape<BITS, LOG2B>;
  constexpr int E = S::E, R = S::R;

  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * (kBlockThreads / kWave) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int64_t n = a.n;
  const int64_t ntiles = (n + S::TILE - 1) / S::TILE;
  const int64_t nwords = (n + E - 1) / E;
  const int np = a.npeers;

  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t t0 = tile * S::TILE;
    const bool full = t0 + S::TILE <= n;

    float acc[R][E];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t w0 = t0 / E + r * kWave + lane;
      const int64_t kb = (w0 * E) >> LOG2B;
      const bool in = w0 < nwords;
      // issue every peer's loads before decoding any of them
      uint32_t cw[kMaxPeers];
      uint32_t sw[kMaxPeers];
#pragma unroll
      for (int p = 0; p < kMaxPeers; ++p) {
        cw[p] = 0;
        sw[p] = 0;
        if (p < np && in) {
          cw[p] = a.codes[p][w0];
          sw[p] = a.scales[p][kb];
        }
      }
#pragma unroll
      for (int p = 0; p < kMaxPeers; ++p) {
        if (p < np) {
          const float s = f16_bits_to_f32(sw[p]);
          if constexpr (BITS == 1) {
#pragma unroll
            for (int j = 0; j < E; ++j) {
              const float d = ((cw[p] >> j) & 1u) ? s : -s;
              acc[r][j] = (p == 0) ? d : acc[r][j] + d;
            }
          } else {
            const uint32_t tw = cw[p] ^ G::FLIP;        // fields become two's complement q
#pragma unroll
            for (int j = 0; j < E; ++j) {
              const int q = (int)(tw << (32 - BITS * (j + 1))) >> (32 - BITS);
              // q * s is exact, so fma(q, s, acc) rounds exactly like acc + q*s
              acc[r][j] = (p == 0) ? (float)q * s : __builtin_fmaf((float)q, s, acc[r][j]);
            }
          }
        }
      }
      if (!full) {
        // positions at or past n are +0 for the statistic
#pragma unroll
        for (int j = 0; j < E; ++j)
          if (w0 * E + j >= n) acc[r][j] = 0.0f;
      }
    }

    if (a.out_sum) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t i0 = t0 + (int64_t)(r * kWave + lane) * E;
        if (full) store_vec_f32<E>(a.out_sum, i0, acc[r]);
        else store_tail_f32<E>(a.out_sum, i0, n, acc[r]);
      }
    }

    float unused[R][E];
    quantize_tile<BITS, LOG2B, SR, false>(acc, t0, n, full, a.out, unused);
    (void)unused;
  }
}

}  // namespace lowbit
