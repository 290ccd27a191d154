// local reduce + requantize kernels: peers packed with more bits than the
// output (8 -> 4, 8 -> 2, 4 -> 2), with or without stage-2 error feedback
#include "reduce_tu.hpp"

namespace lowbit {

template <bool EF>
static lowbit_status launch_mixed(int in_bits, int bits, int log2b, bool sr, bool si,
                                  const ReduceArgs& a, hipStream_t s) {
  if (in_bits == 8 && bits == 4) return launch_r_b<8, 4, EF>(log2b, sr, si, a, s);
  if (in_bits == 8 && bits == 2) return launch_r_b<8, 2, EF>(log2b, sr, si, a, s);
  if (in_bits == 4 && bits == 2) return launch_r_b<4, 2, EF>(log2b, sr, si, a, s);
  return LOWBIT_EUNSUPPORTED;
}

lowbit_status launch_reduce_mixed(int in_bits, int bits, int log2b, bool sr, bool ef,
                                  bool stream_input, const ReduceArgs& a, hipStream_t s) {
  return ef ? launch_mixed<true>(in_bits, bits, log2b, sr, stream_input, a, s)
            : launch_mixed<false>(in_bits, bits, log2b, sr, stream_input, a, s);
}

}  // namespace lowbit
