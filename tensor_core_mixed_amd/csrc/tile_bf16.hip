// Tiled-kernel instances for bf16 inputs.
#include "tile_instances.h"
TCM_TILE_TU(tcm::BF16, bf16)
