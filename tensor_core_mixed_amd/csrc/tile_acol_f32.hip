// Tiled-kernel instances for f32 inputs with A column-major (m contiguous).
#include "tile_instances.h"
TCM_TILE_ACOL_TU(tcm::F32, f32)
