// Implicit-GEMM convolution kernel instances for bf16 inputs.
#include "tile_instances.h"
TCM_CONV_TU(tcm::BF16, bf16)
