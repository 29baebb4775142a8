// Tiled-kernel instances for bf16 inputs with A column-major (m contiguous).
#include "tile_instances.h"
TCM_TILE_ACOL_TU(tcm::BF16, bf16)
