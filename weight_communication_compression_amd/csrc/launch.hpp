// launch.hpp -- host-side launch helpers shared by the kernel translation
// units and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lowbit.h"
#include <type_traits>

#include "args.hpp"
#include "device.hpp"
#include "grid.hpp"

namespace lowbit {

// Workgroups for a kernel in which each wave takes one trip of work (one wave
// per trip); the kernels loop over whatever the cap of grid_blocks leaves.
// (On MI355X a grid that walks memory once, in order, sustains more HBM
// bandwidth than a persistent grid-stride loop: with lowbit_stream_probe_u32
// on 4 GiB, 6.2 vs 5.2-5.8 TB/s reads, 6.0 vs 5.0-5.1 TB/s writes, 5.7 vs
// 4.9-5.4 TB/s copy for persistent grids of 2048 and 8192 waves.)
template <int THREADS = kBlockThreads>
inline int64_t grid_for_tiles(int64_t ntrips) {
  return grid_blocks(ntrips, THREADS);
}

// Launch `kernel` on `s` and return the status of this launch alone: the
// value hipLaunchKernel returns for it.  (An error left on the thread by
// earlier, unrelated work is neither reported nor cleared.)
template <typename... P>
inline lowbit_status launch(void (*kernel)(P...), int64_t blocks, int threads, hipStream_t s,
                            typename std::common_type<P>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel),
                                       dim3((uint32_t)blocks), dim3((uint32_t)threads), argv, 0, s);
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_EDEVICE;
}

// mode: 0 plain, 1 error feedback, 2 weight difference, 3 EF21, 4 Hadamard;
// stream_input: read x non-temporally where the kernel can (see
// stream_capable; the other modes ignore it)
lowbit_status launch_quantize_plain(int bits, int log2b, bool sr, int dt, bool stream_input,
                                    const QuantArgs& a, hipStream_t s);
lowbit_status launch_quantize_ef(int bits, int log2b, bool sr, int dt, bool stream_input,
                                 const QuantArgs& a, hipStream_t s);
lowbit_status launch_quantize_wdiff(int bits, int log2b, bool sr, int dt, bool stream_input,
                                    const QuantArgs& a, hipStream_t s);
lowbit_status launch_quantize_ef21(int bits, int log2b, bool sr, int dt, bool stream_input,
                                   const QuantArgs& a, hipStream_t s);
lowbit_status launch_quantize_hadamard(int bits, int log2b, bool sr, int dt, bool stream_input,
                                       const QuantArgs& a, hipStream_t s);
// local reduce: same width in and out, without / with a stage-2 residual;
// mixed widths (in_bits > bits) for the pairs 8->4, 8->2, 4->2.
// stream_input: read the peers' code words non-temporally.
lowbit_status launch_reduce_same(int bits, int log2b, bool sr, bool stream_input,
                                 const ReduceArgs& a, hipStream_t s);
lowbit_status launch_reduce_same_ef(int bits, int log2b, bool sr, bool stream_input,
                                    const ReduceArgs& a, hipStream_t s);
lowbit_status launch_reduce_mixed(int in_bits, int bits, int log2b, bool sr, bool ef,
                                  bool stream_input, const ReduceArgs& a, hipStream_t s);
lowbit_status launch_dequant(int bits, bool apply, int dt, const DequantArgs& a, hipStream_t s);
// decompress + inverse Hadamard, blocks of 32 .. 4096
lowbit_status launch_hadamard_dequant(int bits, const DequantArgs& a, hipStream_t s);
lowbit_status launch_copy(const float* x, float* y, int64_t n, hipStream_t s);
lowbit_status launch_add_inplace(const float* x, float* y, int64_t n, hipStream_t s);
lowbit_status launch_xor_streams(const XorArgs& a, hipStream_t s);
lowbit_status launch_fold(const float* x, int64_t n, int bits, uint32_t* out, hipStream_t s);
// memory-system probe: op (ProbeOp) over nwords words (a multiple of 1024);
// waves = 0: one trip per wave, else that many waves looping; nt: streaming
// stores
lowbit_status launch_stream_probe(int op, const ProbeArgs& a, int64_t nwords, int64_t waves,
                                  bool nt, hipStream_t s);

}  // namespace lowbit

// Expand F(LOG2B) for every supported block size 2^5 .. 2^12.
#define LOWBIT_FOR_EACH_LOG2B(F) F(5) F(6) F(7) F(8) F(9) F(10) F(11) F(12)
