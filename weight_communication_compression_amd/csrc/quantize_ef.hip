// compress kernels: error-feedback compress (a = g + e, e <- a - deq)
#define LOWBIT_TU_MODE kErrorFeedback
#define LOWBIT_TU_LAUNCHER launch_quantize_ef
#include "quantize_tu.hpp"
