// Instantiates the tiled kernel for every (tile config, B layout) of one
// element type, its grouped form likewise, and the implicit-GEMM convolution
// kernel for every tile config; each (kernel, element type) is compiled in
// its own translation unit.
#pragma once
#include "tile_kernel.h"

namespace tcm {

template <int DT>
TileLauncher pick_tile(int config, bool b_kmajor) {
    switch (config) {
    case 0: return b_kmajor ? &launch_tile<DT, 0, true> : &launch_tile<DT, 0, false>;
    case 1: return b_kmajor ? &launch_tile<DT, 1, true> : &launch_tile<DT, 1, false>;
    case 2: return b_kmajor ? &launch_tile<DT, 2, true> : &launch_tile<DT, 2, false>;
    case 3: return b_kmajor ? &launch_tile<DT, 3, true> : &launch_tile<DT, 3, false>;
    case 4: return b_kmajor ? &launch_tile<DT, 4, true> : &launch_tile<DT, 4, false>;
    case 5: return b_kmajor ? &launch_tile<DT, 5, true> : &launch_tile<DT, 5, false>;
    case 6: return b_kmajor ? &launch_tile<DT, 6, true> : &launch_tile<DT, 6, false>;
    default: return nullptr;
    }
}

template <int DT>
int pick_sk_occupancy(int config, bool b_kmajor) {
    switch (config) {
    case 0: return b_kmajor ? sk_occupancy<DT, 0, true>() : sk_occupancy<DT, 0, false>();
    case 1: return b_kmajor ? sk_occupancy<DT, 1, true>() : sk_occupancy<DT, 1, false>();
    case 2: return b_kmajor ? sk_occupancy<DT, 2, true>() : sk_occupancy<DT, 2, false>();
    case 3: return b_kmajor ? sk_occupancy<DT, 3, true>() : sk_occupancy<DT, 3, false>();
    case 4: return b_kmajor ? sk_occupancy<DT, 4, true>() : sk_occupancy<DT, 4, false>();
    case 5: return b_kmajor ? sk_occupancy<DT, 5, true>() : sk_occupancy<DT, 5, false>();
    case 6: return b_kmajor ? sk_occupancy<DT, 6, true>() : sk_occupancy<DT, 6, false>();
    default: return 0;
    }
}

// column-major A: the configs of at least 64 rows (the transposing reads of
// an m-contiguous tile are laid out for 4 to 64 chunks a k row)
template <int DT>
TileLauncher pick_tile_acol(int config, bool b_kmajor) {
    switch (config) {
    case 0: return b_kmajor ? &launch_tile_acol<DT, 0, true> : &launch_tile_acol<DT, 0, false>;
    case 1: return b_kmajor ? &launch_tile_acol<DT, 1, true> : &launch_tile_acol<DT, 1, false>;
    case 3: return b_kmajor ? &launch_tile_acol<DT, 3, true> : &launch_tile_acol<DT, 3, false>;
    case 4: return b_kmajor ? &launch_tile_acol<DT, 4, true> : &launch_tile_acol<DT, 4, false>;
    case 5: return b_kmajor ? &launch_tile_acol<DT, 5, true> : &launch_tile_acol<DT, 5, false>;
    default: return nullptr;
    }
}

template <int DT>
TileLauncher pick_conv(int config) {
    switch (config) {
    case 0: return &launch_conv<DT, 0>;
    case 1: return &launch_conv<DT, 1>;
    case 2: return &launch_conv<DT, 2>;
    case 3: return &launch_conv<DT, 3>;
    case 4: return &launch_conv<DT, 4>;
    case 5: return &launch_conv<DT, 5>;
    case 6: return &launch_conv<DT, 6>;
    default: return nullptr;
    }
}

template <int DT>
int pick_conv_occupancy(int config) {
    switch (config) {
    case 0: return conv_occupancy<DT, 0>();
    case 1: return conv_occupancy<DT, 1>();
    case 2: return conv_occupancy<DT, 2>();
    case 3: return conv_occupancy<DT, 3>();
    case 4: return conv_occupancy<DT, 4>();
    case 5: return conv_occupancy<DT, 5>();
    case 6: return conv_occupancy<DT, 6>();
    default: return 0;
    }
}

template <int DT>
GroupLauncher pick_group(int config, bool b_kmajor) {
    switch (config) {
    case 0: return b_kmajor ? &launch_group<DT, 0, true> : &launch_group<DT, 0, false>;
    case 1: return b_kmajor ? &launch_group<DT, 1, true> : &launch_group<DT, 1, false>;
    case 2: return b_kmajor ? &launch_group<DT, 2, true> : &launch_group<DT, 2, false>;
    case 3: return b_kmajor ? &launch_group<DT, 3, true> : &launch_group<DT, 3, false>;
    case 4: return b_kmajor ? &launch_group<DT, 4, true> : &launch_group<DT, 4, false>;
    case 5: return b_kmajor ? &launch_group<DT, 5, true> : &launch_group<DT, 5, false>;
    case 6: return b_kmajor ? &launch_group<DT, 6, true> : &launch_group<DT, 6, false>;
    default: return nullptr;
    }
}

}  // namespace tcm

#define TCM_TILE_TU(DT, NAME)                                                                          \
    namespace tcm {                                                                                    \
    TileLauncher tile_launcher_##NAME(int config, bool b_kmajor) { return pick_tile<DT>(config, b_kmajor); } \
    int tile_sk_occupancy_##NAME(int config, bool b_kmajor) { return pick_sk_occupancy<DT>(config, b_kmajor); } \
    }

#define TCM_TILE_ACOL_TU(DT, NAME)                                                                          \
    namespace tcm {                                                                                         \
    TileLauncher tile_acol_launcher_##NAME(int config, bool b_kmajor) { return pick_tile_acol<DT>(config, b_kmajor); } \
    }

#define TCM_CONV_TU(DT, NAME)                                                                     \
    namespace tcm {                                                                               \
    TileLauncher conv_launcher_##NAME(int config) { return pick_conv<DT>(config); }               \
    int conv_sk_occupancy_##NAME(int config) { return pick_conv_occupancy<DT>(config); }          \
    }

#define TCM_GROUP_TU(DT, NAME)                                                                        \
    namespace tcm {                                                                                   \
    GroupLauncher group_launcher_##NAME(int config, bool b_kmajor) { return pick_group<DT>(config, b_kmajor); } \
    }
