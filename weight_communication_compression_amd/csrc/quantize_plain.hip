// compress kernels: plain blockwise quantize + pack
#define LOWBIT_TU_MODE kPlain
#define LOWBIT_TU_LAUNCHER launch_quantize_plain
#include "quantize_tu.hpp"
