// local reduce + requantize kernels: peers and output of the same width; the
// reduce-pattern bandwidth reference
#include "reduce_tu.hpp"

namespace lowbit {

lowbit_status launch_reduce_same(int bits, int log2b, bool sr, bool stream_input,
                                 const ReduceArgs& a, hipStream_t s) {
  switch (bits) {
    case 1: return launch_r_b<1, 1, false>(log2b, sr, stream_input, a, s);
    case 2: return launch_r_b<2, 2, false>(log2b, sr, stream_input, a, s);
    case 4: return launch_r_b<4, 4, false>(log2b, sr, stream_input, a, s);
    case 8: return launch_r_b<8, 8, false>(log2b, sr, stream_input, a, s);
  }
  return LOWBIT_EUNSUPPORTED;
}

// Measurement aid, not a step of the method: out[w] = XOR over the streams
// of word w.  It has the same-width reduce's access pattern at 4 bits
// (each wave takes 64 consecutive words of every stream, one 4-byte word per
// lane read non-temporally, the loads of up to eight streams in flight before
// any is combined, one output word per lane) and none of its arithmetic, so
// it shows what HBM delivers for that pattern.  (8 x 16 MiB streams: 64 words
// per wave 29.5 us, 128 words 31.3 us, 256 words 29.7 us.)
__global__ __launch_bounds__(kBlockThreads) void xor_streams_kernel(XorArgs a) {
  constexpr int W = 1, G = 8;
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const uint32_t lane = (uint32_t)lane_id();
  for (int64_t base = global_wave_id() * (W * kWave); base < a.nwords;
       base += nwaves * (W * kWave)) {                      // wave-uniform
    const bool full = base + W * kWave <= a.nwords;
    uint32_t acc[W] = {};
#pragma unroll 1
    for (int g = 0; g < a.nstreams; g += G) {
      uint32_t v[G][W];
#pragma unroll
      for (int q = 0; q < G; ++q)
#pragma unroll
        for (int i = 0; i < W; ++i) {
          const uint32_t off = (uint32_t)i * kWave + lane;
          v[q][i] = (g + q < a.nstreams && (full || base + off < a.nwords))
                        ? __builtin_nontemporal_load(a.streams[g + q] + base + off) : 0u;
        }
#pragma unroll
      for (int q = 0; q < G; ++q)
#pragma unroll
        for (int i = 0; i < W; ++i) acc[i] ^= v[q][i];
    }
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const uint32_t off = (uint32_t)i * kWave + lane;
      if (full || base + off < a.nwords) store_stream(a.out + base + off, acc[i]);
    }
  }
}

lowbit_status launch_xor_streams(const XorArgs& a, hipStream_t s) {
  const int64_t waves = (a.nwords + kWave - 1) / kWave;
  return launch(&xor_streams_kernel, grid_for_tiles(waves), kBlockThreads, s, a);
}

}  // namespace lowbit
