// Internal declarations shared by the host side (planner, C ABI) and the
// kernels: the tile-config table, kernel argument blocks and launchers.
#pragma once
#include <cstdint>

namespace tcm {

enum DType : int { F16 = 0, BF16 = 1, F32 = 2, I8 = 3 };

inline int elem_bytes(int dt) { return dt == F32 ? 4 : (dt == I8 ? 1 : 2); }

// Storage of C: the accumulator type (f32, or int32 for int8), or a
// rounded-to-nearest-even 16-bit float.
enum CType : int { C_ACC = 0, C_F16 = 1, C_BF16 = 2 };
constexpr int c_elem_bytes(int c_type) { return c_type == C_ACC ? 4 : 2; }

// One K-step stages 128 bytes of every operand row/column: 64 f16/bf16,
// 32 f32 or 128 int8 elements.  Each 16-byte chunk is one MFMA operand
// fragment of one lane (8 f16, 16 int8) or four f32 k-values.
constexpr int kStepBytes = 128;
constexpr int kChunkBytes = 16;
inline int bk_elems(int dt) { return kStepBytes / elem_bytes(dt); }

// Tile-config table: macro tile BM x BN, waves arranged WM x WN (one wave
// tile of (BM/WM) x (BN/WN) outputs each), and the LDS stages of the
// Stream-K kernel (the data-parallel kernels use 2).  A short Stream-K
// segment is latency-bound: each stage is one more K-step of copies in
// flight per workgroup.
struct TileConfig {
    int bm, bn, wm, wn;
    int sk_stages;
    const char* name;
};
constexpr int kNumConfigs = 7;
// Equal shares of a tile (TileArgs::split): at most this many per tile.
constexpr int kMaxSplit = 8;
constexpr TileConfig kConfigs[kNumConfigs] = {
    {256, 256, 4, 2, 2, "256x256 w4x2"},     // big square problems: 64x128 per wave, two waves per SIMD
    {128, 128, 2, 2, 2, "128x128 w2x2"},     // mid sizes, 2 workgroups per CU
    {32, 256, 1, 4, 2, "32x256 w1x4"},       // skinny M (M <= 32)
    {64, 256, 1, 4, 2, "64x256 w1x4"},       // skinny M (M <= 64)
    {64, 64, 2, 2, 2, "64x64 w2x2"},         // Stream-K units for skinny / small problems (16 KiB partials)
    {64, 64, 2, 2, 4, "64x64 w2x2 deep"},    // the same with four Stream-K stages (two workgroups per CU):
                                             // short latency-bound segments, e.g. M <= 64 with a few K-steps each
    {32, 64, 1, 2, 6, "32x64 w1x2 deep"},    // skinny M (M <= 32): six Stream-K stages of 12 KiB, two workgroups
                                             // per CU, most of a short segment's copies in flight at once
};
// Configs whose Stream-K plans run as equal shares of every tile on the
// data-parallel loop (TileArgs::split): the eight-wave tile, whose
// persistent Stream-K kernel has no registers for the partial-tile sum.
constexpr bool split_config(int ci) { return kConfigs[ci].wm * kConfigs[ci].wn > 4; }
inline int lds_bytes(const TileConfig& c, bool sk = false) { return (sk ? c.sk_stages : 2) * (c.bm + c.bn) * kStepBytes; }

// Arguments of the tiled MFMA kernel.  Sizes are in elements, strides of the
// operands in elements.  The kernel runs `dp_tiles` tiles whole (tile t on
// workgroup t % grid), then splits the k-iterations of the next `sk_tiles`
// tiles evenly over the grid (Stream-K), fixing split tiles up through ws.
// Tiles are counted over all `batch` entries.
struct TileArgs {
    const void* A;
    const void* B;
    void* C;
    const void* bias;
    int M, N, K;          // the fast path takes sizes and strides below 2^31
    int lda, ldb, ldc;
    int relu;
    int has_bias;
    int accum;            // C's contents seed the accumulator (read before written)
    int c_type;           // C storage: 0 the accumulator type (f32 / int32), 1 f16, 2 bf16
    int batch;            // entries of a strided batch (1: a single product)
    int64_t stride_a, stride_b, stride_c, stride_bias;  // element strides between entries
    int tiles_m, tiles_n; // tiles of one entry
    int iters;            // k-iterations per tile = ceil(K / bk)
    int dp_tiles;
    int sk_tiles;
    int grid;
    int group_m;          // tile order: rows per group inside a super-tile
    int super_m, super_n; // tile order: super-tile (one XCD's share) in tiles
    float* ws_partial;    // Stream-K partial tiles: 2 slots per workgroup, bm*bn 4-byte values each
    int* ws_counter;      // one arrival counter per split tile (zero between launches)
    int sk_fixup_kernel;  // 1: split tiles are summed by a second kernel, not by their last arrival
    // Equal shares (eight-wave config): > 1 cuts every one of the sk_tiles
    // tiles into `split` k ranges of equal length, one per workgroup of a
    // grid of sk_tiles * split, each run on the data-parallel loop and stored
    // as a partial tile (slot s * sk_tiles + t); a second kernel sums them.
    int split;
    // Implicit-GEMM convolution (kernels built with CONV only): A is the
    // im2col view of an NHWC input x: row m = output pixel (n, p, q), column
    // k = (r*S + s)*C + c.  C is a multiple of the K-step, so every K-step
    // covers one filter tap (r, s).
    int cv_H, cv_W, cv_C, cv_P, cv_Q, cv_S;
    int cv_pad_h, cv_pad_w, cv_stride_h, cv_stride_w, cv_dil_h, cv_dil_w;
    int cv_x_bytes;       // bytes of x (below 2^30)
};

// Tile t -> (tm, tn) for a grid of tiles_m x tiles_n tiles.  Workgroups are
// dealt to the 8 XCDs round-robin by id, and each XCD has its own L2, so:
//  1. renumber ids so that XCD x (ids x, x+8, x+16, ...) owns one contiguous
//     run of the tile order;
//  2. walk the grid in super-tiles of super_m x super_n tiles (bands of
//     super_m rows, super-tiles left to right), sized so one run covers about
//     one near-square super-tile -- an XCD then reads the A rows and B
//     columns of that block only;
//  3. inside a super-tile, walk groups of group_m rows column by column, so
//     the 32 tiles an XCD runs at once form a group_m x (32/group_m) block.
// Every step is a bijection on [0, tiles_m * tiles_n).  A batch of
// matrices shares one tile space: step 1 runs over all of it, then each
// position splits into (entry, tile within the entry) before steps 2-3.
#if defined(__HIPCC__)
__host__ __device__
#endif
inline int xcd_order(int t, int T) {
    const int q = T >> 3, r = T & 7, x = t & 7, local = t >> 3;
    return x * q + (x < r ? x : r) + local;
}
#if defined(__HIPCC__)
__host__ __device__
#endif
inline void super_order(int nt, int tiles_m, int tiles_n, int group_m, int super_m, int super_n, int* tm, int* tn) {
    const int band = nt / (super_m * tiles_n);
    const int o = nt - band * super_m * tiles_n;
    const int h = tiles_m - band * super_m < super_m ? tiles_m - band * super_m : super_m;
    const int J = o / (h * super_n);
    const int o2 = o - J * h * super_n;
    const int w = tiles_n - J * super_n < super_n ? tiles_n - J * super_n : super_n;
    const int g = o2 / (group_m * w);
    const int gh = h - g * group_m < group_m ? h - g * group_m : group_m;
    const int inner = o2 - g * group_m * w;
    *tm = band * super_m + g * group_m + inner % gh;
    *tn = J * super_n + inner / gh;
}
#if defined(__HIPCC__)
__host__ __device__
#endif
inline void tile_coords(int t, int tiles_m, int tiles_n, int group_m, int super_m, int super_n, int* tm, int* tn) {
    super_order(xcd_order(t, tiles_m * tiles_n), tiles_m, tiles_n, group_m, super_m, super_n, tm, tn);
}
// Position n of the locality walk over a batch of tiles_m x tiles_n grids
// (steps 2-3 above, entry by entry) -> (entry, tm, tn).  Step 1 is the
// caller's: tile t of the work list (data-parallel tiles first, then the
// Stream-K tiles in the order of the split) sits at n = xcd_order(t, tiles).
// (Renumbering the Stream-K workgroups by XCD instead, so that each XCD
// walks one contiguous run of the split, measured slower on a long-K
// problem.)
#if defined(__HIPCC__)
__host__ __device__
#endif
inline void walk_coords(int n, int tiles_m, int tiles_n, int group_m, int super_m, int super_n, int* b, int* tm,
                        int* tn) {
    const int per = tiles_m * tiles_n;
    *b = n / per;
    super_order(n - *b * per, tiles_m, tiles_n, group_m, super_m, super_n, tm, tn);
}

// Super-tile shape for a tiles_m x tiles_n grid: about T/8 tiles, near square.
inline void tile_order_shape(int tiles_m, int tiles_n, int group_m, int* super_m, int* super_n) {
    const long long T = (long long)tiles_m * tiles_n;
    const long long share = (T + 7) / 8;
    int sm = group_m;
    while ((long long)(2 * sm) * (2 * sm) <= share && 2 * sm <= tiles_m) sm *= 2;
    if (sm > tiles_m) sm = tiles_m;
    long long sn = (share + sm - 1) / sm;
    if (sn > tiles_n) sn = tiles_n;
    if (sn < 1) sn = 1;
    *super_m = sm;
    *super_n = (int)sn;
}

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
    int accum;
    int c_type;
    int bytewise;  // some pointer is not aligned to its element: single-byte accesses
    int batch;
    int64_t stride_a, stride_b, stride_c, stride_bias;
    int tiles_m, tiles_n;
    // convolution: A is the im2col view of NHWC x (see TileArgs)
    int conv;
    int64_t cv_H, cv_W, cv_C, cv_P, cv_Q, cv_R, cv_S;
    int64_t cv_pad_h, cv_pad_w, cv_stride_h, cv_stride_w, cv_dil_h, cv_dil_w;
};

// A group of products that share K, the element type and the epilogue but
// not their shapes or operands (tcm_gemm_grouped).  The tiles of all entries
// form one work list, entry after entry; the table travels in the kernel
// arguments, so a group holds at most kMaxGroup entries.
constexpr int kMaxGroup = 32;
struct GroupEntry {
    const void* A;
    const void* B;
    void* C;
    const void* bias;
    int M, N;
    int lda, ldb, ldc;
    int tiles_m, tiles_n;   // of this entry
    int super_m, super_n;   // its tile walk
    int tile0;              // its first tile in the work list
};
struct GroupArgs {
    TileArgs t;             // what the entries share: K, epilogue, C type, schedule, workspace
    int count;              // entries, 1 .. kMaxGroup
    GroupEntry e[kMaxGroup];
};

// Launchers (defined next to the kernels).  Return hipError_t as int.
using TileLauncher = int (*)(const TileArgs&, void* stream);
using GroupLauncher = int (*)(const GroupArgs&, void* stream);
// the grouped kernels: config index, dtype, B column-major -> launcher
GroupLauncher group_launcher(int config, int dtype, bool b_kmajor);
// config index, dtype, B column-major (K-contiguous), A column-major (M-contiguous) -> launcher, or nullptr
TileLauncher tile_launcher(int config, int dtype, bool b_kmajor, bool a_mmajor);
// the implicit-GEMM convolution kernels (B = the KRSC filter, k-contiguous)
TileLauncher conv_launcher(int config, int dtype);
// Stream-K workgroups of a config that fit on one CU, from the compiled
// kernel's resources (0 if the runtime cannot tell).
int tile_sk_occupancy(int config, int dtype, bool b_kmajor);
int launch_generic(int dtype, const GenericArgs& a, void* stream);
int launch_fill_zero(int* p, int64_t n, void* stream);

}  // namespace tcm
