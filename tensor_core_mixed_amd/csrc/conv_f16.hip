// Implicit-GEMM convolution kernel instances for f16 inputs.
#include "tile_instances.h"
TCM_CONV_TU(tcm::F16, f16)
