// Grouped GEMM kernel instances for i8 inputs.
#include "tile_instances.h"
TCM_GROUP_TU(tcm::I8, i8)
