// measure.hip -- the memory-system probe kernel (measurement aid, not a step
// of the method): one pass of 32-bit word reads, writes or copies, either one
// trip per wave over the whole buffer or a fixed persistent grid that loops,
// with plain or non-temporal stores.  It backs the launch shapes and store
// policies the codec kernels use.
#include "launch.hpp"

namespace lowbit {

// A trip is 1024 words: four coalesced 16-byte pieces per lane (piece k of
// lane l holds words 4 (64 k + l) .. + 3 of the trip).
constexpr int kProbeTripWords = 1024;

template <int OP, bool NT>
__global__ __launch_bounds__(kBlockThreads) void stream_probe_kernel(ProbeArgs a, int64_t ntrips) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t nwaves = (int64_t)gridDim.x * (kBlockThreads / kWave);
  const int lane = lane_id();
  for (int64_t trip = global_wave_id(); trip < ntrips; trip += nwaves) {   // wave-uniform
    const int64_t w0 = trip * kProbeTripWords;
    if constexpr (OP == kProbeRead || OP == kProbeCopy) {
      const u32x4* src = reinterpret_cast<const u32x4*>(a.src + w0);
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = src[k * kWave + lane];
      if constexpr (OP == kProbeCopy) {
        u32x4* dst = reinterpret_cast<u32x4*>(a.dst + w0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (NT) __builtin_nontemporal_store(v[k], dst + k * kWave + lane);
          else dst[k * kWave + lane] = v[k];
        }
      } else {
        // dst[trip] = XOR of the trip's words
        uint32_t x = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) x ^= (uint32_t)__shfl_xor((int)x, d);
        if (lane == 0) {
          if constexpr (NT) __builtin_nontemporal_store(x, a.dst + trip);
          else a.dst[trip] = x;
        }
      }
    } else {
      // dst[i] = i ^ value (the low 32 bits of the word index)
      u32x4* dst = reinterpret_cast<u32x4*>(a.dst + w0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t i = (uint32_t)w0 + (uint32_t)(4 * (k * kWave + lane));
        const u32x4 v = {i ^ a.value, (i + 1) ^ a.value, (i + 2) ^ a.value, (i + 3) ^ a.value};
        if constexpr (NT) __builtin_nontemporal_store(v, dst + k * kWave + lane);
        else dst[k * kWave + lane] = v;
      }
    }
  }
}

template <int OP>
static lowbit_status launch_probe_op(const ProbeArgs& a, bool nt, int64_t blocks, int64_t ntrips,
                                     hipStream_t s) {
  return nt ? launch(&stream_probe_kernel<OP, true>, blocks, kBlockThreads, s, a, ntrips)
            : launch(&stream_probe_kernel<OP, false>, blocks, kBlockThreads, s, a, ntrips);
}

lowbit_status launch_stream_probe(int op, const ProbeArgs& a, int64_t nwords, int64_t waves,
                                  bool nt, hipStream_t s) {
  const int64_t ntrips = nwords / kProbeTripWords;
  constexpr int64_t kWavesPerBlock = kBlockThreads / kWave;
  // one trip per wave (the grid capped as for the codec kernels), or the
  // given number of waves looping over the trips
  const int64_t blocks = waves > 0 ? (waves + kWavesPerBlock - 1) / kWavesPerBlock
                                   : grid_for_tiles(ntrips);
  switch (op) {
    case kProbeRead: return launch_probe_op<kProbeRead>(a, nt, blocks, ntrips, s);
    case kProbeWrite: return launch_probe_op<kProbeWrite>(a, nt, blocks, ntrips, s);
    case kProbeCopy: return launch_probe_op<kProbeCopy>(a, nt, blocks, ntrips, s);
  }
  return LOWBIT_EINVAL;
}

}  // namespace lowbit
