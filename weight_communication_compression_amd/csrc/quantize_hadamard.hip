// compress kernels with Hadamard smoothing: blockwise Walsh-Hadamard
// transform in registers, then the plain compress
#define LOWBIT_TU_MODE kHadamard
#define LOWBIT_TU_LAUNCHER launch_quantize_hadamard
#include "quantize_tu.hpp"
