// args.hpp -- kernel argument blocks (plain structs passed by value as kernel
// arguments), shared by the kernels and the C ABI.
#pragma once

#include <stdint.h>

namespace lowbit {

constexpr int kMaxPeers = 16;

// Output side of a compress: where codes and scales go and the SR counter.
struct TileOut {
  uint32_t* codes;
  uint16_t* scales;
  uint64_t index_offset;  // global index of element 0
  uint32_t key;           // K(seed)
};

struct QuantArgs {
  const void* x;          // plain: x;  error feedback: g;  weight diff: w_new
  const void* x2;         // weight diff: w_old
  float* resid;           // error feedback: residual / EF21: state, read and overwritten
  int64_t n;
  TileOut out;
};

struct ReduceArgs {
  const uint32_t* codes[kMaxPeers];
  const uint16_t* scales[kMaxPeers];
  int32_t npeers;
  int32_t in_log2b;        // log2 of the peers' block size
  int64_t n;
  float* out_sum;          // may be null
  float* resid;            // stage-2 error feedback: residual, read and overwritten
  TileOut out;
};

struct DequantArgs {
  const uint32_t* codes;
  const uint16_t* scales;
  int64_t n;
  int32_t log2b;
  float* y;                // decompress output (binary32)
  const void* w_old;       // apply: previous weights
  void* w_out;             // apply: output weights (may equal w_old)
};

// Reference kernel with the reduce's access pattern (measurement aid).
struct XorArgs {
  const uint32_t* streams[kMaxPeers];
  uint32_t* out;
  int64_t nwords;
  int32_t nstreams;
};

// Memory-system probe (measurement aid): operation codes and arguments.
enum ProbeOp : int { kProbeRead = 0, kProbeWrite = 1, kProbeCopy = 2 };
struct ProbeArgs {
  const uint32_t* src;
  uint32_t* dst;
  uint32_t value;
};

}  // namespace lowbit
