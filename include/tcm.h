/*
 * tcm.h -- C ABI of the MI355X (gfx950) dense GEMM engine.
 *
 * One operation: the matrix product with a fused bias / ReLU epilogue,
 *
 *     C[i][j] = epi( [C_in[i][j] +] bias[j] + sum_k a(i,k) * b(k,j) ),
 *
 * the product-plus-bias whose bias is the initial value of the reduction
 * (kimm240.github.io/tvm, FuseReductionEpilogue posts 1 and 2; post 2 also
 * generalises the initial value to a per-element tensor, the optional C_in,
 * which is C's own contents before the call), followed by
 * the ReLU of the Conv2d + Bias + ReLU pattern (same page, Conv2d-Reshape-
 * Add-ReLU fusion post), computed on the matrix cores with low-precision
 * inputs and a wide accumulator (je-d.tistory.com/entry/tvm, Tensor Core
 * notes: mixed-precision multiply-accumulate).  Large problems are tiled and
 * staged through LDS (kimm240.github.io/tvm, GEMM optimisation Steps 2-6);
 * shapes whose tile count fills the GPU badly are split along k across
 * workgroups (leiblog.wang, the Stream-K reproduction post).  The same
 * tiled product also serves a strided batch of products (tcm_gemm_batched)
 * and the Conv2d + bias + ReLU pattern as an implicit GEMM (tcm_conv2d).
 *
 * All pointers are DEVICE pointers (any allocation the HIP runtime can read
 * on the current device).  The caller owns A, B, C and bias; the library
 * never frees them.  Calls are asynchronous on `stream` (a hipStream_t passed
 * as void*, NULL = the null stream) and never synchronise; results are
 * ready when the stream reaches the call.  Calls on one stream run in order.
 * The library's state is a cached split-k workspace per (device, stream),
 * so concurrent calls on different streams are independent, plus the
 * process-wide switches and tuning table below (mutex-protected).  The
 * workspace grows on demand (hipMalloc, plus a zero-fill kernel for its
 * counters), never synchronising; an outgrown buffer is kept, not freed,
 * until tcm_release_workspace, because kernels or graphs enqueued earlier may
 * still use it.  A call whose plan fits the stream's existing workspace
 * allocates nothing and issues only kernel launches, so it can be captured
 * into a HIP graph after one warm-up call of the same shape on that stream; a
 * call that would grow the workspace while its stream is capturing returns
 * TCM_ERR_NOT_SUPPORTED.  A captured graph uses the workspace of the stream
 * it was captured on: its replays must not run at the same time as other
 * calls (eager or replayed) on that stream's workspace, e.g. replay it on the
 * same stream.  tcm_gemm_noalloc needs no workspace at all.
 *
 * Errors are returned, never raised; argument checks run before any HIP call.
 */
#ifndef TCM_H
#define TCM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes --------------------------------------------------------- */
typedef enum {
    TCM_OK = 0,
    TCM_ERR_INVALID_VALUE = 1, /* a bad size, leading dimension, pointer, flag or option */
    TCM_ERR_NOT_SUPPORTED = 2, /* a valid request that cannot be served as asked: workspace
                                  growth while the stream is being captured into a graph, or
                                  a forced split-k plan beyond tcm_gemm_noalloc's scratch */
    TCM_ERR_HIP = 3,           /* a HIP runtime error (no device, launch failure, ...) */
    TCM_ERR_ALLOC = 4          /* the split-k workspace could not be allocated */
} tcm_status;

/* ---- element types (low byte of `dtype`) ---------------------------------- */
/*   TCM_F16_F32  : A, B IEEE binary16; accumulate and C in binary32; bias f32
 *   TCM_BF16_F32 : A, B bfloat16;      accumulate and C in binary32; bias f32
 *   TCM_F32_F32  : A, B binary32;      accumulate and C in binary32; bias f32
 *   TCM_I8_I32   : A, B int8;          accumulate and C in int32 (wrapping
 *                  two's complement on overflow); bias int32                */
enum { TCM_F16_F32 = 0, TCM_BF16_F32 = 1, TCM_F32_F32 = 2, TCM_I8_I32 = 3 };

/* ---- operand layout flags (or-ed into `dtype`) ---------------------------- */
/* Row-major unless flagged:
 *   a(i,k) = A[i*lda + k]   or, with TCM_A_COLMAJOR,  A[k*lda + i]
 *   b(k,j) = B[k*ldb + j]   or, with TCM_B_COLMAJOR,  B[j*ldb + k]
 *   C is always row-major: C[i*ldc + j].                                      */
#define TCM_A_COLMAJOR (1 << 8)
#define TCM_B_COLMAJOR (1 << 9)

/* ---- output type flags (or-ed into `dtype`; float element types only) ---- */
/* C (and C_in with TCM_EPI_ACCUM) stored as IEEE binary16 or as bfloat16
 * instead of binary32: the f32 accumulator is rounded to nearest-even at the
 * store (the mixed-precision output of the Tensor Core notes,
 * je-d.tistory.com/entry/tvm: narrow inputs and outputs, wide accumulation).
 * At most one of the two; TCM_ERR_INVALID_VALUE with int8.                   */
#define TCM_C_F16 (1 << 10)
#define TCM_C_BF16 (1 << 11)

/* ---- epilogue flags -------------------------------------------------------- */
/* TCM_EPI_BIAS:  bias[j] (length N, f32 or int32 per dtype) seeds the
 *                accumulator of column j before any product is added.
 * TCM_EPI_RELU:  C = x > 0 ? x : 0 after the sum (NaN and -0 become +0).
 * TCM_EPI_ACCUM: C's contents before the call (C_in, in C's own type) also
 *                seed the accumulator: C = epi(C_in + bias + A.B) in place.
 *                Every element of C is read once before it is written.     */
enum { TCM_EPI_NONE = 0, TCM_EPI_BIAS = 1, TCM_EPI_RELU = 2, TCM_EPI_BIAS_RELU = 3, TCM_EPI_ACCUM = 4 };

/*
 * tcm_gemm -- C = epi(bias + A.B) with M x K A, K x N B, M x N C.
 *
 *   M, N, K      sizes, >= 0.  M == 0 or N == 0: nothing to do, TCM_OK.
 *                K == 0: C = epi(bias or 0).
 *   A, lda       A and its leading dimension in elements:
 *                lda >= K (row-major) or lda >= M (TCM_A_COLMAJOR), lda >= 1.
 *   B, ldb       likewise: ldb >= N (row-major) or ldb >= K (TCM_B_COLMAJOR).
 *   C, ldc       output (input too with TCM_EPI_ACCUM), ldc >= N; f32 for
 *                float types unless TCM_C_F16 / TCM_C_BF16, int32 for int8.
 *                C must not overlap A, B or bias.
 *   dtype        one element type above, optionally or-ed with layout and
 *                output type flags.
 *   bias         device vector of N elements, read only with TCM_EPI_BIAS.
 *   epilogue     TCM_EPI_* flags (any combination).
 *   stream       hipStream_t as void* (NULL: null stream).
 *
 * Any alignment and any leading dimension is served (je-d.tistory.com, the
 * auto-tensorcore note: code off the matrix-core fast path is slower but
 * functionally equal): 16-byte aligned pointers with 16-byte multiple
 * layouts take the tiled fast path, in either layout of A and of B (K, lda
 * and ldb whole numbers of 16-byte pieces; N too with row-major B, M too
 * with column-major A, which runs on tiles of at least 64 rows); anything
 * else runs on the generic kernel, which reads and writes single bytes when
 * a pointer is not a multiple of its element size.
 * Products of few rows in f16 or bf16 with row-major A run on a split-k
 * GEMV instead of the tiles when lda is a multiple of 8, every pointer
 * 16-byte aligned, and A and B lie below 2 GiB: at most 32 rows with
 * row-major B and ldb a multiple of 8, else at most 8 rows, with row-major
 * B N and ldb multiples of 4, with column-major B (k contiguous) K and ldb
 * multiples of 8 (up to 64 / 16 rows with option "gemv" = 2).  B streams
 * from HBM once over an even split of the k range (the Stream-K
 * reproduction post on leiblog.wang).  Row-major B: 128 columns per
 * workgroup, each lane transposing the 8 x 8 blocks of B it loads in
 * registers into operands of the matrix cores' 16x16x32 blocks (with ldb
 * not a multiple of 8: 256 columns per workgroup in 4x4x4 blocks);
 * column-major B: 128 columns per workgroup in 16x16x32 blocks fed straight
 * from memory.  The k ranges' partial sums (ranges x M
 * x N floats of workspace) are added in range order by a second kernel on
 * the stream, which runs the epilogue.
 * Returns TCM_OK once the work is enqueued; TCM_ERR_INVALID_VALUE for
 * negative sizes, too-small leading dimensions, a NULL operand with a
 * non-empty extent, unknown dtype/flags/epilogue, both output type flags or
 * an output type flag with int8, TCM_EPI_BIAS with a NULL bias, or C
 * overlapping an input; TCM_ERR_ALLOC if the split-k workspace cannot be
 * allocated; TCM_ERR_NOT_SUPPORTED if it would have to grow while the stream
 * is capturing; TCM_ERR_HIP on a launch error.
 */
int tcm_gemm(int64_t M, int64_t N, int64_t K,
             const void* A, int64_t lda,
             const void* B, int64_t ldb,
             void* C, int64_t ldc,
             int dtype, const void* bias, int epilogue,
             void* stream);

/*
 * tcm_gemm_noalloc -- tcm_gemm for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, hosts
 * that forbid hipMalloc.  Same arguments, results and errors as tcm_gemm; it
 * never allocates (no hipMalloc, hipFree or allocating library call).  Its
 * split-k (Stream-K) plans keep their partial tiles and arrival counters in
 * one fixed array of tcm_noalloc_scratch_bytes() bytes per device (64 MiB of
 * partial tiles plus 65536 counters), part of the library's device image and
 * held until the process ends, instead of the per-stream workspace.
 *   * The split-k GEMV keeps its partial sums in the same array; one that
 *     needs more runs on the tiles instead.
 *   * A planned split-k launch that needs more than that array runs as
 *     data-parallel tiles instead (no scratch); when split-k is forced
 *     (tcm_set_option "force_mode" 2) such a call returns
 *     TCM_ERR_NOT_SUPPORTED and launches nothing.
 *   * Every call on a device shares that device's array, which keeps the last
 *     call's contents: the counters a call uses are cleared by a fill kernel
 *     on its stream first.  Calls that overlap in time on one device (other
 *     streams, or graph replays) race on the array: order them.
 */
int tcm_gemm_noalloc(int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda,
                     const void* B, int64_t ldb,
                     void* C, int64_t ldc,
                     int dtype, const void* bias, int epilogue,
                     void* stream);
/* Bytes of tcm_gemm_noalloc's fixed scratch array on each device. */
int64_t tcm_noalloc_scratch_bytes(void);

/*
 * tcm_gemm_batched -- `batch` independent products of one shape,
 *
 *     C_e = epi( [C_e,in +] bias_e + A_e . B_e ),   e = 0 .. batch-1,
 *
 * with entry e of each operand at a fixed element stride from the first:
 * A_e = A + e*stride_a, B_e = B + e*stride_b, C_e = C + e*stride_c,
 * bias_e = bias + e*stride_bias (pointer arithmetic in elements of each
 * operand's own type).  All entries share M, N, K, the leading dimensions,
 * dtype and epilogue.  The tiles of all entries form one work list, so
 * split-k (Stream-K) spreads the k-iterations of every entry's tiles over
 * one persistent grid: many skinny products fill the GPU together, the
 * contiguous-batching case that motivates Stream-K (leiblog.wang, the
 * Stream-K reproduction post).
 *
 *   batch        >= 0 (0: nothing to do).  batch < 2^31.
 *   stride_*     >= 0 and < 2^40 elements.  0 shares one operand (or bias)
 *                across the batch.  The entries of C are written, so with
 *                batch > 1 stride_c must be at least the extent of one C
 *                ((M-1)*ldc + N elements): C entries never overlap.
 *   the rest     as tcm_gemm, per entry; the overlap check covers the
 *                whole span of each operand over the batch.
 * Returns as tcm_gemm; TCM_ERR_INVALID_VALUE also for a negative batch or
 * stride, or overlapping C entries.  tcm_gemm(...) is tcm_gemm_batched with
 * batch 1.
 */
int tcm_gemm_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda, int64_t stride_a,
                     const void* B, int64_t ldb, int64_t stride_b,
                     void* C, int64_t ldc, int64_t stride_c,
                     int dtype, const void* bias, int64_t stride_bias, int epilogue,
                     void* stream);

/*
 * tcm_gemm_grouped -- `count` independent products that share K, dtype and
 * epilogue but not their shapes or operands,
 *
 *     C_e = epi( [C_e,in +] bias_e + A_e . B_e ),   A_e: M_e x K, B_e: K x N_e,
 *
 * e.g. the experts of a mixture, each with its own rows.  The tiles of all
 * entries form one work list (entry after entry), so split-k (Stream-K)
 * spreads the k-iterations of every entry's tiles over one persistent grid,
 * the contiguous-batching case that motivates Stream-K (leiblog.wang, the
 * Stream-K reproduction post), here with a different M (and N) per entry.
 *
 *   count        0 .. TCM_MAX_GROUP entries (0: nothing to do).
 *   entries      HOST array of `count` descriptors, read during the call
 *                only: M, N (>= 0; an entry with M or N == 0 is skipped),
 *                A, lda, B, ldb, C, ldc, bias as for tcm_gemm (device
 *                pointers; bias read only with TCM_EPI_BIAS).
 *   K, dtype, epilogue, stream   as tcm_gemm, shared by every entry.
 * Every C must not overlap any entry's A, B, bias or another entry's C.
 * When no tile config can take every entry (odd layouts, unaligned
 * pointers), the entries run one by one as tcm_gemm calls.
 * Returns as tcm_gemm; TCM_ERR_INVALID_VALUE also for count outside
 * [0, TCM_MAX_GROUP], a NULL `entries` with count > 0, or overlapping C.
 */
#define TCM_MAX_GROUP 32
typedef struct {
    int64_t M, N;
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    void* C;
    int64_t ldc;
    const void* bias;
} tcm_group_entry;

int tcm_gemm_grouped(int64_t count, const tcm_group_entry* entries, int64_t K,
                     int dtype, int epilogue, void* stream);

/*
 * tcm_conv2d -- 2-D convolution with the fused bias + ReLU epilogue (the
 * Conv2d + bias + ReLU pattern of kimm240.github.io/tvm, post "Implement and
 * enable Conv2d-Reshape-Add-ReLU fusion"), computed as an implicit GEMM on
 * the same matrix-core main loop and epilogue as tcm_gemm:
 *
 *     y[n,p,q,k] = epi( bias[k] + sum_{r,s,c} x[n,h,w,c] * f[k,r,s,c] ),
 *     h = p*stride_h - pad_h + r*dil_h,   w = q*stride_w - pad_w + s*dil_w,
 *
 * taps with h or w outside the input add nothing (zero padding).  As a GEMM:
 * M = N*P*Q output pixels, N = K output channels, K = R*S*C; A is the im2col
 * view of x (never built in memory: the kernel gathers it tap by tap), B is
 * the filter with k contiguous, C is y row-major with ldc = K.
 *
 *   N, H, W, C   batch, input height, width, channels; >= 0, < 2^31.
 *   K, R, S      output channels, filter height, width; K >= 0, R, S >= 1.
 *   pad_*        zero padding on both sides, >= 0.  stride_*, dil_* >= 1.
 *                P = (H + 2*pad_h - dil_h*(R-1) - 1) / stride_h + 1, Q likewise;
 *                a dilated filter larger than the padded input is an error.
 *   x            device, NHWC dense (channels fastest), N*H*W*C elements.
 *   f            device, KRSC dense, K*R*S*C elements.
 *   y            device, NPQK dense, N*P*Q*K elements of C's type; written
 *                only; must not overlap x, f or bias.
 *   dtype        TCM_F16 / TCM_BF16 / TCM_F32 / TCM_I8, optionally with
 *                TCM_C_F16 or TCM_C_BF16 (float inputs) for a 16-bit y.  The
 *                layout flags are errors: the layouts above are fixed.
 *   bias, epilogue  as tcm_gemm, except that TCM_EPI_ACCUM is an error.
 *   stream       hipStream_t or NULL.
 * The tiled kernel takes C a multiple of the K-step (64 for f16/bf16, 32
 * for f32, 128 for int8), 16-byte aligned pointers and inputs below 1 GiB;
 * any other valid call runs on the generic kernel with the same result.
 * Accumulation is f32 (int32 for int8, exact).  Returns as tcm_gemm;
 * TCM_OK with nothing launched when N*P*Q or K is 0.  Allocates only the
 * shared Stream-K workspace, as tcm_gemm.
 */
int tcm_conv2d(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
               int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w,
               int64_t dil_h, int64_t dil_w,
               const void* x, const void* f, void* y,
               int dtype, const void* bias, int epilogue, void* stream);

/* Text of a status code (static storage; never NULL). */
const char* tcm_status_string(int status);

/*
 * tcm_set_option / tcm_get_option -- process-wide tuning switches, for
 * experiments and tests.  Keys:
 *   "force_mode"   0 = planner decides, 1 = data-parallel tiles only,
 *                  2 = split-k (Stream-K) over a persistent grid; on the
 *                  eight-wave 256x256 config (tile-table row 0), unless
 *                  "sk_grid" or "grid_per_cu8" is given, as equal shares:
 *                  every tile cut into at most 8 k ranges of equal length,
 *                  one workgroup each, summed by a second kernel.
 *   "force_config" -1 = planner decides, else an index into the tile table
 *                  (tcm_config_count()); a config that cannot serve the call
 *                  is ignored.
 *   "sk_grid"      0 = planner decides, else the persistent grid size for
 *                  split-k (clamped to the number of co-resident workgroups).
 *   "generic"      1 = route every call to the generic (any-alignment) kernel.
 *   "sk_fixup"     how a split-k tile cut between workgroups is summed:
 *                  0 = planner decides (a second kernel when the tile has five
 *                  or more segments), 1 = its last-arriving workgroup sums
 *                  the partials, 2 = a second kernel launched on the same
 *                  stream sums them.  Both add the partials in the same
 *                  order: the results are bit-identical.  Equal shares are
 *                  always summed by the second kernel.
 *   "group_m"      0 = planner decides (4), else the rows of tiles per group
 *                  of the tile order (1..16).
 *   "grid_per_cu8" 0 = planner decides, else a split-k grid of value/8
 *                  workgroups per CU (1..64).
 *   "grid_shares"  0 = planner decides, else a split-k grid of value
 *                  workgroups per tile (1..64): every split tile in equal
 *                  shares that start at the same k (the equal shares of the
 *                  eight-wave config: at most 8, at most as many as fill the
 *                  CUs once, each at least one K-step).
 *   "tuned"        1 (default) = use the tuning table (tcm_tune) for problems
 *                  whose class it holds; 0 = ignore it.  force_config /
 *                  force_mode / sk_grid / gemv win.
 *   "gemv"         the split-k GEMV (tcm_gemm): 0 = planner decides (calls
 *                  it can serve with at most 32 rows on the 16x16x32
 *                  row-major-B kernel, else 8, or the tuning table's
 *                  choice), 1 = never, 2 = every call it can serve (at most
 *                  64 / 16 rows) unless a tile config or mode is forced.
 *   "gemv_wide"    which GEMV kernel serves row-major B: 0 or 2 = the
 *                  16x16x32 kernel where eligible, 1 = never it (the 4x4x4
 *                  kernel, at most 16 rows).
 *   "gemv_splits"  0 = planner decides (4x4x4 kernel: about two workgroups
 *                  per CU, the partial sums kept within an eighth of B's
 *                  bytes; 16x16x32 row-major kernel: one workgroup per CU,
 *                  ranges of a multiple of 512 rows (256 above 16 rows)
 *                  where K allows; column-major B: ranges of 256 rows), else
 *                  the number of k ranges, rounded to ranges of a multiple
 *                  of 64 rows, at most 1024 each (4x4x4 kernel), of 128
 *                  rows (16x16x32 row-major kernel) or of 256 rows
 *                  (column-major B) (1..4096).
 * Unknown keys or out-of-range values: TCM_ERR_INVALID_VALUE.
 * tcm_get_option returns the value, or -2 for an unknown key.
 */
int tcm_set_option(const char* key, int64_t value);
int64_t tcm_get_option(const char* key);

/* ---- planning and introspection ------------------------------------------ */
typedef struct {
    int32_t kernel;        /* 0 = generic kernel, 1 = tiled MFMA kernel, 2 = split-k GEMV */
    int32_t config;        /* tile-table index (tiled kernel) or -1 */
    int32_t bm, bn, bk;    /* macro tile; bk in elements.  GEMV: the rows it
                              computes (1, 2, 4, 8, 16; 16, 32, 64 on the
                              16x16x32 row-major-B kernel), the columns per
                              workgroup (256 on the 4x4x4 kernel, else 128), k
                              rows per range; iters_per_tile = the k ranges,
                              tiles = the column blocks */
    int32_t mode;          /* 1 = data-parallel, 2 = Stream-K (+ data-parallel tiles) */
    int32_t grid;          /* workgroups launched */
    int64_t tiles;         /* ceil(M/bm) * ceil(N/bn) */
    int64_t iters_per_tile;/* ceil(K/bk) */
    int64_t dp_tiles;      /* tiles done whole by one workgroup */
    int64_t sk_tiles;      /* tiles whose k range is split over workgroups */
    int64_t workspace_bytes; /* split-k workspace the call needs */
    int32_t fixup_kernel;  /* 1 = split tiles are summed by a second kernel on the stream */
    int32_t split;         /* > 1: Stream-K as equal shares, every split tile cut
                              into this many k ranges of equal length, one
                              workgroup each (grid = sk_tiles * split); else 0 */
} tcm_plan_info;

/*
 * tcm_plan -- the plan tcm_gemm would use for this problem (same arguments
 * minus the pointers; `aligned` says whether A, B, C, bias would be 16-byte
 * aligned).  Launches nothing and allocates nothing.  With a device present
 * it plans for the current device exactly as tcm_gemm does (its CU count and
 * the workgroups per CU the runtime reports for the split-k kernels); with
 * none it plans for 256 CUs with a static occupancy estimate.
 * Returns TCM_OK or TCM_ERR_INVALID_VALUE.
 */
int tcm_plan(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
             int dtype, int epilogue, int aligned, tcm_plan_info* out);

/*
 * tcm_plan_batched -- the plan tcm_gemm_batched would use for `batch`
 * products of this shape (1 <= batch < 2^31; the strides do not enter the
 * plan, only whether every entry is 16-byte aligned, `aligned`).  `tiles`
 * counts the tiles of all entries, which share one work list.  tcm_plan is
 * tcm_plan_batched with batch 1.  Returns TCM_OK or TCM_ERR_INVALID_VALUE.
 */
int tcm_plan_batched(int64_t batch, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                     int64_t ldc, int dtype, int epilogue, int aligned, tcm_plan_info* out);

/* Number of rows of the tile table, and row i as (bm, bn, bk, waves).  Two
 * rows may share a shape and differ in the depth of their split-k (Stream-K)
 * pipeline: LDS stages of copies in flight per workgroup, traded against
 * workgroups per CU.  Returns TCM_OK or TCM_ERR_INVALID_VALUE (bad index or
 * dtype). */
int tcm_config_count(void);
int tcm_config_info(int index, int dtype, int32_t* bm, int32_t* bn, int32_t* bk, int32_t* waves);

/*
 * tcm_streamk_range -- the k-iteration range [begin, end) that workgroup
 * `wg` of a Stream-K grid of `grid` workgroups owns over `sk_tiles` tiles of
 * `iters_per_tile` iterations (even split of the total).  Host mirror of the
 * device partition, for tests.
 */
int tcm_streamk_range(int64_t sk_tiles, int64_t iters_per_tile, int32_t grid, int32_t wg,
                      int64_t* begin, int64_t* end);

/*
 * tcm_tile_order -- the output tile (tm, tn) that workgroup t of a
 * data-parallel launch computes on a tiles_m x tiles_n grid: each XCD's
 * workgroups get one near-square block of tiles so they share A rows and B
 * columns in that XCD's L2 (the cache-blocking idea of the tiling step,
 * kimm240.github.io/tvm, GEMM optimisation Step 2, applied to whole tiles).
 * Host mirror of the device order, for tests.  TCM_ERR_INVALID_VALUE for
 * t outside [0, tiles_m * tiles_n) or a grid of 2^31 tiles or more.
 */
int tcm_tile_order(int32_t t, int32_t tiles_m, int32_t tiles_n, int32_t* tm, int32_t* tn);

/* ---- auto-tuning ----------------------------------------------------------- */
/*
 * The tuning table holds, per shape class, the plan parameters that measured
 * fastest (the schedule search of the pages: Fireiron is built for
 * auto-scheduling and auto-tuning, je-d.tistory.com/entry/tvm; the GEMM
 * schedule exploration of kimm240.github.io/tvm, Steps 2-6).
 *
 * A shape class is: element type, A and B layout flags, output type,
 * epilogue flags, whether every pointer is 16-byte aligned, whether the call
 * is a batch, and the half octave of each of M, N and K (floor(2*log2(x)):
 * e.g. every M in [4096, 5792] shares class 24).  An entry gives the tile
 * config and mode (or a split-k GEMV kernel: config 100 in the text for the
 * 4x4x4 row-major-B or the column-major-B kernel, 101 for the 16x16x32
 * row-major-B one), the split-k grid policy (the planner's; g/8 workgroups
 * per CU; or s workgroups per tile, every tile split into s equal shares),
 * the way split tiles are summed (the planner's, last arrival, fix-up
 * kernel) and the tile-order group rows (the planner's, or 1..16).
 * tcm_gemm and tcm_plan use the entry of the call's class, or, when the
 * table holds none, the entry of the nearest class that differs only in
 * the size classes, by at most one half octave in each (option "tuned");
 * explicit force_config / force_mode / sk_grid switches win, and switches the
 * caller set keep their values.  A tile config that cannot serve the call is
 * ignored as with force_config.
 *
 * The library ships a table (tuned/mi355x.txt beside the directory of
 * libtcm.so, or the file named by the environment variable TCM_TUNE_FILE;
 * an empty TCM_TUNE_FILE ships none), loaded before the first plan; entries
 * tuned or loaded before that keep precedence.
 */

/*
 * tcm_tune -- search the tuning space on this problem and record the
 * fastest point for its shape class.  Stage 1 times every tile config in
 * both modes (data-parallel, split-k) with the planner's other parameters,
 * and the split-k GEMV kernels where they can serve the call;
 * stage 2 varies, around the three fastest tile plans, the tile-order group rows and,
 * for split-k, the grid (0.5 to 2 workgroups per CU, 1 to 4 equal shares per
 * tile) and the fix-up.  Each candidate is timed twice and keeps its better
 * time; a stage-2 variant is recorded only if it beats the best stage-1 point
 * by 2% (otherwise the planner's own parameters, which adapt to the other
 * shapes of the class).
 *
 * Same arguments as tcm_gemm plus `iters` (timed calls per candidate,
 * 1..10000) and `best` (optional: the plan now chosen).  Runs on `stream`
 * with the caller's buffers and BLOCKS until timing is done; C is written by
 * every candidate, so its contents afterwards are one correct result, except
 * with TCM_EPI_ACCUM, where C has been accumulated into repeatedly.  A call
 * the generic kernel serves records nothing.  Returns as tcm_gemm.
 */
int tcm_tune(int64_t M, int64_t N, int64_t K,
             const void* A, int64_t lda, const void* B, int64_t ldb,
             void* C, int64_t ldc, int dtype, const void* bias, int epilogue,
             int iters, void* stream, tcm_plan_info* best);

/*
 * tcm_tune_table -- the tuning table as text, one class per line:
 *   "tcm-tune-2 dtype a_col b_col c_type epilogue aligned batched mclass
 *    nclass kclass config mode grid_kind grid_param fixup group_m
 *    microseconds M N K"
 * (c_type 0 = the accumulator type, 1 = f16, 2 = bf16; config 100 / 101 =
 * the split-k GEMV kernels, with mode 1 and zeros after it; grid_kind 0 = the
 * planner's, 1 = grid_param/8 workgroups per CU, 2 = grid_param per tile;
 * fixup and group_m 0 = the planner's; M N K = the shape it was tuned on).
 * Writes it NUL-terminated into buf (truncated to len) and returns its full
 * length.  tcm_tune_load parses such text (blank lines and lines starting
 * with '#' are skipped) and adds or replaces its entries (all-or-nothing:
 * TCM_ERR_INVALID_VALUE and no change on a malformed line).  tcm_tune_clear
 * empties the table (the shipped entries too).  All three are host-only.
 */
int tcm_tune_table(char* buf, int64_t len);
int tcm_tune_load(const char* text);
void tcm_tune_clear(void);

/* Describe the last plan tcm_gemm launched on this thread into buf (NUL-
 * terminated, truncated to len).  Returns the full length. */
int tcm_last_plan(char* buf, int64_t len);

/* Free every cached split-k workspace, outgrown ones included (waits for
 * every device holding one to finish its work first).  No call may run or be
 * replayed concurrently. */
void tcm_release_workspace(void);

/* Library version string. */
const char* tcm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TCM_H */
