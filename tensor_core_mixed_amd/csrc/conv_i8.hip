// Implicit-GEMM convolution kernel instances for i8 inputs.
#include "tile_instances.h"
TCM_CONV_TU(tcm::I8, i8)
