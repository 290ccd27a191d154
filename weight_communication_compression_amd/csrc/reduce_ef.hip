// local reduce + requantize kernels with stage-2 error feedback: peers and
// output of the same width
#include "reduce_tu.hpp"

namespace lowbit {

lowbit_status launch_reduce_same_ef(int bits, int log2b, bool sr, bool stream_input,
                                    const ReduceArgs& a, hipStream_t s) {
  switch (bits) {
    case 1: return launch_r_b<1, 1, true>(log2b, sr, stream_input, a, s);
    case 2: return launch_r_b<2, 2, true>(log2b, sr, stream_input, a, s);
    case 4: return launch_r_b<4, 4, true>(log2b, sr, stream_input, a, s);
    case 8: return launch_r_b<8, 8, true>(log2b, sr, stream_input, a, s);
  }
  return LOWBIT_EUNSUPPORTED;
}

}  // namespace lowbit
