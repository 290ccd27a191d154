// compress kernels: weight-difference compress (d = w_new - w_old)
#define LOWBIT_TU_MODE kWeightDiff
#define LOWBIT_TU_LAUNCHER launch_quantize_wdiff
#include "quantize_tu.hpp"
