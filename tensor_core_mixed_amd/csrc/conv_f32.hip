// Implicit-GEMM convolution kernel instances for f32 inputs.
#include "tile_instances.h"
TCM_CONV_TU(tcm::F32, f32)
