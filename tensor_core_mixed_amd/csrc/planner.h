// Planner: which kernel, which tile config, data-parallel or Stream-K, and
// the launch geometry for one GEMM call.  Pure host code (no HIP calls), so
// the C ABI can expose it for CPU-side tests.
#pragma once
#include <cstdint>

#include "gemv.h"
#include "tcm_internal.h"

namespace tcm {

struct Options {
    int force_mode = 0;     // 0 auto, 1 data-parallel, 2 Stream-K
    int force_config = -1;  // -1 auto, else tile-table index
    int sk_grid = 0;        // 0 auto, else persistent grid size
    int generic = 0;        // 1: always the generic kernel
    int sk_fixup = 0;       // 0 planner decides, 1 last arrival sums a split tile, 2 a second kernel does
    // Stream-K grid policy (tunable; sk_grid, an absolute size, wins):
    // grid_per_cu8 > 0: grid_per_cu8 / 8 workgroups per CU; grid_shares > 0:
    // exactly tiles x grid_shares workgroups (every split tile in equal shares)
    int grid_per_cu8 = 0;
    int grid_shares = 0;
    int group_m = 0;        // tile-order group rows (0: the planner's 4)
    int gemv = 0;           // split-k GEMV for products of at most 16 rows: 0 planner decides, 1 never, 2 whenever eligible
    int gemv_splits = 0;    // its k ranges (0: the planner's)
    int gemv_wide = 0;      // row-major B: the 16x16x32 GEMV kernel (up to 64 rows): 0 planner decides, 1 never, 2 whenever eligible
    int sk_occ[kNumConfigs] = {0};  // Stream-K workgroups per CU by config (0: static estimate)
};

struct Problem {
    int64_t M, N, K, lda, ldb, ldc;
    int dtype;     // element type (low byte of the ABI dtype)
    bool a_col, b_col;
    int epilogue;
    int c_type;    // CType
    int64_t batch = 1;  // entries of a strided batch
    bool aligned;  // every pointer 16-byte aligned
    // implicit-GEMM convolution: A is the im2col view of an NHWC input of
    // conv_x_bytes bytes and conv_c channels (lda is nominal)
    bool conv = false;
    int64_t conv_c = 0, conv_x_bytes = 0;
    // a group of products sharing K (its M is the entries' total, N their
    // largest): the work list's exact tile count and the tiled kernel's
    // eligibility, per config, computed over the entries
    bool group = false;
    int64_t group_tiles[kNumConfigs] = {0};
    bool group_ok[kNumConfigs] = {false};
    // a group's bytes summed over its entries: each operand once, and the
    // bytes split tiles read (an entry's A once per tile column, its B once
    // per tile row) per config
    double group_a_bytes = 0, group_b_bytes = 0, group_c_bytes = 0;
    double group_a_reads[kNumConfigs] = {0}, group_b_reads[kNumConfigs] = {0};
};

struct Plan {
    int kernel = 0;   // 0 none (empty problem), 1 generic, 2 tiled, 3 split-k GEMV (bm = rows bucket,
                      // bn = columns per workgroup, bk = k per workgroup, iters = k ranges)
    bool gemv_wide = false;  // GEMV on row-major B: the 16x16x32 kernel (else the 4x4x4 one)
    int config = -1;
    int bm = 0, bn = 0, bk = 0;
    int mode = 1;     // 1 data-parallel, 2 Stream-K (+ data-parallel tiles)
    int grid = 0;     // Stream-K persistent grid (mode 2) or data-parallel workgroups
    int64_t tiles = 0, iters = 0, dp_tiles = 0, sk_tiles = 0;
    int64_t ws_partial_bytes = 0, ws_counters = 0;
    int group_m = 4;
    bool fixup_kernel = false;  // Stream-K split tiles summed by a second kernel
    int split = 0;    // > 1: Stream-K as that many equal shares of every tile on the data-parallel loop
    double est_cycles = 0;  // the cost model's estimate (for logs)
};

// Number of CUs the cost model assumes when no device is queried.
constexpr int kDefaultCUs = 256;

// Tile kernel eligibility for a config (alignment, strides, 32-bit offsets).
bool tile_eligible(const Problem& p, const TileConfig& c);
// Workgroups of a config that fit on one CU (LDS- and register-limited
// estimate), for the data-parallel and the Stream-K kernel.
int tile_wg_per_cu(const TileConfig& c);
int tile_sk_wg_per_cu(const TileConfig& c);
// Split-k GEMV eligibility: f16 / bf16, row-major A, a single product,
// 16-byte aligned pointers and rows of A, offsets below 2 GiB, and either
// (4x4x4 kernel) B row-major, 1 <= M <= 16, N a multiple of 4, 8-byte
// aligned rows of B; or (16x16x32 kernel) B row-major, 1 <= M <= 64,
// 16-byte aligned rows of B; or B column-major, 1 <= M <= 16, K and ldb
// multiples of 8.
bool gemv_eligible(const Problem& p);
// The 16x16x32 row-major-B kernel's part of that, and the other kernels'.
bool gemv_wide_eligible(const Problem& p);
bool gemv_narrow_eligible(const Problem& p);
// Whether the planner (no option forcing a tile config or mode) takes the
// GEMV for an eligible p.
bool gemv_preferred(const Problem& p, const Options& o);
// Fill `out` for problem p.  Returns false if p is invalid.
bool make_plan(const Problem& p, const Options& o, int cus, Plan* out);
// Stream-K share [begin, end) of workgroup wg (same split the kernel uses).
void streamk_range(int64_t sk_tiles, int64_t iters, int grid, int wg, int64_t* begin, int64_t* end);

}  // namespace tcm
