// launch.hpp -- host-side launch helpers shared by the kernel translation
// units and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lowbit.h"
#include "args.hpp"
#include "device.hpp"

// Optional cap on the grid, in workgroups per CU (0: no cap).  Without a cap
// every wave makes one trip through its kernel's loop: on MI355X a grid that
// walks memory once, in order, sustains far more HBM bandwidth than a
// persistent grid-stride loop (measured: 6.8 vs 5-6 TB/s reads, 6.9 vs
// 4.3-5.1 TB/s writes).
#ifndef LOWBIT_BLOCKS_PER_CU
#define LOWBIT_BLOCKS_PER_CU 0
#endif

namespace lowbit {


// Number of compute units of the current device (cached per device id).
int device_cu_count();

// Grid for a kernel where each wave takes `ntrips` trips' worth of work: one
// wave per trip (4 per workgroup); the kernels loop over whatever a cap
// leaves.  The grid stays below 2^31 workgroups.
template <int THREADS = kBlockThreads>
inline int grid_for_tiles(int64_t ntrips) {
  const int64_t waves_per_block = THREADS / kWave;
  int64_t blocks = (ntrips + waves_per_block - 1) / waves_per_block;
  int64_t cap = (int64_t)1 << 30;
  if (LOWBIT_BLOCKS_PER_CU > 0) cap = (int64_t)device_cu_count() * LOWBIT_BLOCKS_PER_CU;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

inline lowbit_status launch_status() {
  return hipGetLastError() == hipSuccess ? LOWBIT_OK : LOWBIT_EDEVICE;
}

// mode: 0 plain, 1 error feedback, 2 weight difference, 3 EF21, 4 Hadamard
lowbit_status launch_quantize_plain(int bits, int log2b, bool sr, int dt, const QuantArgs& a,
                                    hipStream_t s);
lowbit_status launch_quantize_ef(int bits, int log2b, bool sr, int dt, const QuantArgs& a,
                                 hipStream_t s);
lowbit_status launch_quantize_wdiff(int bits, int log2b, bool sr, int dt, const QuantArgs& a,
                                    hipStream_t s);
lowbit_status launch_quantize_ef21(int bits, int log2b, bool sr, int dt, const QuantArgs& a,
                                   hipStream_t s);
lowbit_status launch_quantize_hadamard(int bits, int log2b, bool sr, int dt, const QuantArgs& a,
                                       hipStream_t s);
// local reduce: same width in and out, without / with a stage-2 residual;
// mixed widths (in_bits > bits) for the pairs 8->4, 8->2, 4->2
lowbit_status launch_reduce_same(int bits, int log2b, bool sr, const ReduceArgs& a,
                                 hipStream_t s);
lowbit_status launch_reduce_same_ef(int bits, int log2b, bool sr, const ReduceArgs& a,
                                    hipStream_t s);
lowbit_status launch_reduce_mixed(int in_bits, int bits, int log2b, bool sr, bool ef,
                                  const ReduceArgs& a, hipStream_t s);
lowbit_status launch_dequant(int bits, bool apply, int dt, const DequantArgs& a, hipStream_t s);
// decompress + inverse Hadamard, blocks of 32 .. 4096
lowbit_status launch_hadamard_dequant(int bits, const DequantArgs& a, hipStream_t s);
lowbit_status launch_copy(const float* x, float* y, int64_t n, hipStream_t s);
lowbit_status launch_add_inplace(const float* x, float* y, int64_t n, hipStream_t s);
lowbit_status launch_xor_streams(const XorArgs& a, hipStream_t s);
lowbit_status launch_fold(const float* x, int64_t n, int bits, uint32_t* out, hipStream_t s);

}  // namespace lowbit

// Expand F(LOG2B) for every supported block size 2^5 .. 2^12.
#define LOWBIT_FOR_EACH_LOG2B(F) F(5) F(6) F(7) F(8) F(9) F(10) F(11) F(12)
