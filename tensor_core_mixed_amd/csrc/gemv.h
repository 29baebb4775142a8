// The split-k GEMV kernel's arguments and launcher, shared by the host side
// (planner, C ABI) and the kernel.
#pragma once
#include <cstdint>

namespace tcm {

// Arguments of the split-k GEMV kernels (products of at most 16 rows, f16 /
// bf16, row-major A; B row-major, or column-major with b_col; with `wide`, a
// row-major B and at most 64 rows on 16x16x32 MFMAs).  Workgroup
// (x, y) computes a block of columns of every row over the k range
// [kw y, kw y + kw) and, with splits > 1, stores that partial sum to
// partial[y][m][n]; a second kernel adds the splits in order and runs the
// epilogue.  With splits == 1 the first kernel runs the epilogue itself.
constexpr int kGemvMaxRows = 16;
constexpr int kGemvCols = 256;   // row-major B: columns per workgroup (64 lanes x 4)
constexpr int kGemvKAlign = 64;  // row-major B: kw is a multiple of this (4 waves x 16-row chunks)
constexpr int kGemvTCols = 128;  // column-major B: columns per workgroup (4 waves x 2 groups of 16)
constexpr int kGemvTSteps = 8;   // column-major B: 32-k steps per wave in flight at once
constexpr int kGemvTKAlign = 32 * kGemvTSteps;  // column-major B: kw is a multiple of this
constexpr int kGemvWideRows = 64;  // row-major B on 16x16x32 MFMAs: rows at most
constexpr int kGemvWCols = 128;    // its columns per workgroup (16 lanes x 8)
constexpr int kGemvWKAlign = 128;  // its kw is a multiple of this (4 waves x 32-k steps)
struct GemvArgs {
    const void* A;
    const void* B;
    void* C;
    const void* bias;
    int M, N, K;
    int lda, ldb, ldc;
    int relu;
    int has_bias;
    int accum;
    int c_type;
    int splits;          // k ranges (gridDim.y)
    int kw;              // k per range, a multiple of kGemvKAlign
    float* partial;      // splits x M x N partial sums (splits > 1)
    int64_t b_bytes;     // extent of B in bytes (its buffer range)
    int b_col;           // 1: B column-major (k contiguous, ldb >= K)
    int64_t a_bytes;     // extent of A in bytes (its buffer range; column-major B and `wide`)
    int wide;            // row-major B: 1 = the 16x16x32 kernel (M <= 64), 0 = the 4x4x4 one (M <= 16)
};
// rows bucket (1, 2, 4, 8 or 16) of an M <= 16
inline int gemv_rows_bucket(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }
// rows bucket (16, 32 or 64) of the 16x16x32 row-major kernel
inline int gemv_wide_rows_bucket(int64_t M) { return M <= 16 ? 16 : M <= 32 ? 32 : 64; }
int launch_gemv(int dtype, const GemvArgs& a, void* stream);

}  // namespace tcm
