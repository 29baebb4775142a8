// Grouped GEMM kernel instances for f32 inputs.
#include "tile_instances.h"
TCM_GROUP_TU(tcm::F32, f32)
