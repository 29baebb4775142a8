// Grouped GEMM kernel instances for bf16 inputs.
#include "tile_instances.h"
TCM_GROUP_TU(tcm::BF16, bf16)
