// Tiled-kernel instances for f16 inputs with A column-major (m contiguous).
#include "tile_instances.h"
TCM_TILE_ACOL_TU(tcm::F16, f16)
