// compress kernels: EF21 compress (d = g - h, h <- h + deq)
#define LOWBIT_TU_MODE kEF21
#define LOWBIT_TU_LAUNCHER launch_quantize_ef21
#include "quantize_tu.hpp"
