// Grouped GEMM kernel instances for f16 inputs.
#include "tile_instances.h"
TCM_GROUP_TU(tcm::F16, f16)
