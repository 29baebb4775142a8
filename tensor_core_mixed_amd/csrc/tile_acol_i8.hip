// Tiled-kernel instances for i8 inputs with A column-major (m contiguous).
#include "tile_instances.h"
TCM_TILE_ACOL_TU(tcm::I8, i8)
