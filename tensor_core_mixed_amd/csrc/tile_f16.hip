// Tiled-kernel instances for f16 inputs.
#include "tile_instances.h"
TCM_TILE_TU(tcm::F16, f16)
