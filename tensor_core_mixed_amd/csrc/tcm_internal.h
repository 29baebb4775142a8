// Internal declarations shared by the host side (planner, C ABI) and the
// kernels: the tile-config table, kernel argument blocks and launchers.
#pragma once
#include <cstdint>

namespace tcm {

enum DType : int { F16 = 0, BF16 = 1, F32 = 2, I8 = 3 };

inline int elem_bytes(int dt) { return dt == F32 ? 4 : (dt == I8 ? 1 : 2); }

// One K-step stages 128 bytes of every operand row/column: 64 f16/bf16,
// 32 f32 or 128 int8 elements.  Each 16-byte chunk is one MFMA operand
// fragment of one lane (8 f16, 16 int8) or four f32 k-values.
constexpr int kStepBytes = 128;
constexpr int kChunkBytes = 16;
inline int bk_elems(int dt) { return kStepBytes / elem_bytes(dt); }

// Tile-config table: macro tile BM x BN, waves arranged WM x WN (one wave
// tile of (BM/WM) x (BN/WN) outputs each), 2 LDS stages.
struct TileConfig {
    int bm, bn, wm, wn;
    const char* name;
};
constexpr int kNumConfigs = 4;
constexpr TileConfig kConfigs[kNumConfigs] = {
    {256, 256, 4, 2, "256x256 w4x2"},  // big square problems: 64x128 per wave, two waves per SIMD
    {128, 128, 2, 2, "128x128 w2x2"},  // mid sizes, 2 workgroups per CU
    {32, 256, 1, 4, "32x256 w1x4"},    // skinny M (M <= 32)
    {64, 256, 1, 4, "64x256 w1x4"},    // skinny M (M <= 64)
};
inline int lds_bytes(const TileConfig& c) { return 2 * (c.bm + c.bn) * kStepBytes; }

// Arguments of the tiled MFMA kernel.  Sizes are in elements, strides of the
// operands in elements.  The kernel runs `dp_tiles` tiles whole (tile t on
// workgroup t % grid), then splits the k-iterations of the next `sk_tiles`
// tiles evenly over the grid (Stream-K), fixing split tiles up through ws.
struct TileArgs {
    const void* A;
    const void* B;
    void* C;
    const void* bias;
    int M, N, K;          // the fast path takes sizes and strides below 2^31
    int lda, ldb, ldc;
    int relu;
    int has_bias;
    int tiles_m, tiles_n;
    int iters;            // k-iterations per tile = ceil(K / bk)
    int dp_tiles;
    int sk_tiles;
    int grid;
    int group_m;          // tile-order group height (L2 reuse)
    float* ws_partial;    // Stream-K partial tiles: 2 slots per workgroup, bm*bn 4-byte values each
    int* ws_counter;      // one arrival counter per split tile (zero between launches)
};

// Arguments of the generic (any alignment / layout) kernel.
struct GenericArgs {
    const void* A;
    const void* B;
    void* C;
    const void* bias;
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
    int a_col, b_col;
    int relu;
    int has_bias;
    int tiles_m, tiles_n;
};

// Launchers (defined next to the kernels).  Return hipError_t as int.
using TileLauncher = int (*)(const TileArgs&, void* stream);
// config index, dtype, B column-major (K-contiguous) -> launcher, or nullptr
TileLauncher tile_launcher(int config, int dtype, bool b_kmajor);
int launch_generic(int dtype, const GenericArgs& a, void* stream);
int launch_fill_zero(int* p, int64_t n, void* stream);

}  // namespace tcm
