// Planner: tile config + data-parallel / Stream-K choice from a small cost
// model of one MI355X CU.
//
// Work unit: one K-step (128 bytes of every operand row) of one macro tile.
// A CU spends max(matrix-core time, LDS time, L2 time) on it.  Data-parallel
// time is the number of full "waves" of tiles times a tile's K-steps; the
// last, partial wave costs as much as a full one, which is the waste that
// Stream-K removes by splitting the total K-steps evenly over a persistent
// grid (leiblog.wang, Stream-K reproduction post: even k split across SMs
// against wave waste at small shapes), at the price of writing and summing
// partial tiles.  Problems with tiny M are bound by reading B from HBM; the
// model floors every estimate at the HBM time of the unique bytes.
#include "planner.h"

#include <algorithm>
#include <cmath>

namespace tcm {
namespace {

constexpr int64_t kOffsetLimit = 0x40000000LL;  // buffer-descriptor range used by the kernels
// Cost-model constants, fitted to measured MI355X runs of every tile config
// in both modes on the workload set (lone-workgroup step time, fix-up
// round trips) and to the MFMA rate the kernels reach on N(0,1) inputs
// (the matrix cores are power-limited: their rate falls with operand entropy).
constexpr double kLdsBytesPerClk = 200.0;       // measured ds_read_b128 rate per CU
constexpr double kL2BytesPerClk = 64.0;         // per-CU share of L2 bandwidth
constexpr double kHbmBytesPerClk = 8.0e12 / 2.4e9;  // whole chip
constexpr double kStepOverhead = 96.0;          // barrier + wait per K-step
constexpr double kStepLatency = 500.0;          // lone workgroup: fixed part of a K-step ...
constexpr double kStepBytesPerClk = 16.0;       // ... plus its copies at this rate
constexpr double kFixupLatency = 1500.0;        // one device-coherent round trip per partial tile read back
// Stream-K workgroups start their segments at different k, so tiles that
// share an operand panel no longer read it from L2 at the same time.  For
// 128x128 tiles (two workgroups per CU) a split K-step then streams its
// operands at about the CU's share of MALL / HBM bandwidth, ~9 TB/s over
// 256 CUs (measured on 3840^2 x 4096 and the 3x3 convolutions: split
// K-steps took twice as long as data-parallel ones).  The 64x64 units keep
// the fitted per-step cost: their K-steps are a quarter of the bytes.
constexpr double kStaggerBytesPerClk = 14.6;
// Split tiles also lose the L2 reuse of their operand panels across the
// grid: each tile row re-reads B and each tile column re-reads A, served
// from MALL (the 256 MiB last-level cache) at ~16 TB/s (fitted to
// 1536^2 x 16384 with 64x64 and 128x128 units and to M = 256).  An operand
// re-read by split tiles stays in the MALL only while it takes at most half
// of it (the other operand, C and the partial tiles share the cache); a
// larger one is re-read from HBM (seven 4096 x 4096 f16 weights of a group,
// 235 MB: Stream-K 74 us against 49 us data-parallel).
// A launch that splits tiles pays about 4 us the model above does not see:
// every workgroup's first segment fills its pipeline from HBM, and split
// tiles wait on the partial-tile round trips.  Fitted to the 130 shapes of
// the tuning set: with it the data-parallel / Stream-K choice agrees with
// the measured winner on 118 of them, without it on 110 (the misses were
// short-K products such as 768^3 .. 1536^3, where split segments are a few
// K-steps long).
constexpr double kSplitFixed = 9600.0;
// Equal shares of the eight-wave tile: the sum kernel's launch and its one
// memory round trip.
constexpr double kSplitSum = 6000.0;
constexpr int kEpiAccumBit = 4;  // the epilogue flag that reads C_in (C read as well as written)
constexpr double kMallBytesPerClk = 16.0e12 / 2.4e9;
constexpr double kMallBytes = 128.0 * 1024 * 1024;

double flops_per_clk(int dt) {
    switch (dt) {
    case F16:
    case BF16: return 4096.0 * 0.47;
    case I8: return 8192.0 * 0.40;
    default: return 256.0 * 0.82;
    }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int tile_wg_per_cu(const TileConfig& c) {
    int by_lds = (160 * 1024) / lds_bytes(c);
    // registers: a 128x128 wave tile (256 accumulators) or eight-wave
    // workgroups leave one workgroup per CU; 64x64 wave tiles two; 32x32 four
    const int wave_tile = (c.bm / c.wm) * (c.bn / c.wn);
    int by_regs = (wave_tile >= 128 * 128 || c.wm * c.wn > 4) ? 1 : (wave_tile >= 64 * 64 ? 2 : 4);
    return std::max(1, std::min(by_lds, by_regs));
}

int tile_sk_wg_per_cu(const TileConfig& c) {
    // the Stream-K kernels carry the partial-tile fix-up on top: the
    // 32x32-per-wave config, and the 128x128 one compiled for it, hold two
    // workgroups per CU; the others one
    const int wave_tile = (c.bm / c.wm) * (c.bn / c.wn);
    const bool two = wave_tile <= 32 * 32 || (c.wm * c.wn == 4 && c.bm == 128 && c.bn == 128);
    return two ? std::max(1, std::min(2, (160 * 1024) / (lds_bytes(c, true) + 16))) : 1;
}

bool tile_eligible(const Problem& p, const TileConfig& c) {
    const int es = elem_bytes(p.dtype);
    const int ce = kChunkBytes / es;
    if (!p.aligned) return false;
    // column-major A (m contiguous): the GEMM kernels (not the grouped or
    // convolution ones) of tiles of at least 64 rows, M a whole number of
    // 16-byte pieces, as for the columns of a row-major B
    if (p.a_col && (p.conv || p.group || c.bm < 64 || p.M % ce)) return false;
    if (p.K <= 0 || p.M <= 0 || p.N <= 0) return false;
    if (p.M >= (1LL << 31) || p.N >= (1LL << 31) || p.K >= (1LL << 31)) return false;
    if (p.lda >= (1LL << 31) || p.ldb >= (1LL << 31) || p.ldc >= (1LL << 31)) return false;
    if (p.K % ce || p.lda % ce) return false;
    if (p.b_col) {
        if (p.ldb % ce) return false;
    } else {
        if (p.N % ce || p.ldb % ce) return false;
    }
    // every per-tile byte offset must stay inside the descriptor range
    if (p.conv) {
        // one K-step is one filter tap; the gather addresses x from its base
        // with 32-bit element offsets, and row indices past M stay in int
        if (p.conv_c % bk_elems(p.dtype)) return false;
        if (p.conv_x_bytes >= kOffsetLimit) return false;
        if (p.M + c.bm >= (1LL << 31)) return false;
    } else if (p.a_col) {
        if ((int64_t)bk_elems(p.dtype) * p.lda * es + (int64_t)c.bm * es >= kOffsetLimit) return false;
    } else if ((int64_t)c.bm * p.lda * es + kStepBytes >= kOffsetLimit) {
        return false;
    }
    if (p.b_col) {
        if ((int64_t)c.bn * p.ldb * es + kStepBytes >= kOffsetLimit) return false;
    } else {
        if ((int64_t)bk_elems(p.dtype) * p.ldb * es + (int64_t)c.bn * es >= kOffsetLimit) return false;
    }
    const int cs = c_elem_bytes(p.c_type);
    if ((int64_t)c.bm * p.ldc * cs + (int64_t)c.bn * cs >= kOffsetLimit) return false;
    const int64_t tiles = cdiv(p.M, c.bm) * cdiv(p.N, c.bn) * std::max<int64_t>(p.batch, 1);
    if (tiles >= (1LL << 31)) return false;
    return true;
}

void streamk_range(int64_t sk_tiles, int64_t iters, int grid, int wg, int64_t* begin, int64_t* end) {
    const int64_t W = sk_tiles * iters;
    *begin = (int64_t)wg * W / grid;
    *end = (int64_t)(wg + 1) * W / grid;
}

namespace {

struct Estimate {
    double cycles;
    int mode;
    int grid;
    int64_t dp_tiles, sk_tiles;
    int split = 0;  // equal shares of every tile (the eight-wave config's Stream-K)
};

// Tiles of the work list for config ci.
int64_t tile_count(const Problem& p, int ci) {
    const TileConfig& c = kConfigs[ci];
    return p.group ? p.group_tiles[ci] : cdiv(p.M, c.bm) * cdiv(p.N, c.bn) * std::max<int64_t>(p.batch, 1);
}

Estimate estimate(const Problem& p, int ci, int cus, int force_mode, int sk_grid, int sk_occ_known, int grid_per_cu8 = 0,
                  int grid_shares = 0) {
    const TileConfig& c = kConfigs[ci];
    const int dt = p.dtype;
    const int bke = bk_elems(dt);
    const int64_t T = tile_count(p, ci);
    const int64_t I = cdiv(p.K, bke);
    const int occ = tile_wg_per_cu(c);
    const int64_t slots = (int64_t)cus * occ;

    const double mfma = 2.0 * c.bm * c.bn * bke / flops_per_clk(dt);
    const double lds = ((c.bm + c.bn) * (double)kStepBytes + (double)(c.bm * c.wn + c.bn * c.wm) * kStepBytes) / kLdsBytesPerClk;
    const double l2 = (c.bm + c.bn) * (double)kStepBytes / kL2BytesPerClk;
    const double step = std::max(mfma, std::max(lds, l2)) + kStepOverhead;  // per K-step, CU to itself
    const double lone_step = kStepLatency + (c.bm + c.bn) * (double)kStepBytes / kStepBytesPerClk;
    const double tile_store = (double)c.bm * c.bn * 4 / kL2BytesPerClk;
    // unique bytes: a convolution's A is its input x, read once however many
    // taps reuse it; a group's bytes are summed over its entries, each with
    // its own B
    const double nb = (double)std::max<int64_t>(p.batch, 1);
    const double a_bytes = p.conv ? (double)p.conv_x_bytes : (double)p.M * p.K * elem_bytes(dt);
    double a_uniq = nb * a_bytes, b_uniq = nb * (double)p.K * p.N * elem_bytes(dt), c_uniq = nb * (double)p.M * p.N * 4;
    double a_reads = a_uniq * cdiv(p.N, c.bn), b_reads = b_uniq * cdiv(p.M, c.bm);
    if (p.group) {
        a_uniq = p.group_a_bytes;
        b_uniq = p.group_b_bytes;
        c_uniq = p.group_c_bytes;
        a_reads = p.group_a_reads[ci];
        b_reads = p.group_b_reads[ci];
    }
    const double hbm_floor = (a_uniq + b_uniq + c_uniq) / kHbmBytesPerClk;

    // data-parallel: waves of `slots` tiles, each wave takes I steps on a CU shared by `occ` workgroups
    Estimate dp{0, 1, (int)std::min<int64_t>(T, 1LL << 30), T, 0};
    {
        const int64_t waves = cdiv(T, slots);
        const int64_t busy = std::min<int64_t>(T, slots);
        const double share = (double)std::min<int64_t>(occ, cdiv(busy, cus));  // workgroups per busy CU
        dp.cycles = std::max(waves * (I * std::max(step * share, lone_step) + tile_store * share), hbm_floor);
    }
    // Stream-K: hybrid of (full waves - 1) data-parallel waves, then an even
    // split of the remaining tiles' K-steps over the grid
    Estimate sk{0, 2, 0, 0, 0};
    {
        // every workgroup of the grid must own at least one K-step: the
        // kernel counts a split tile's arrivals as the number of workgroups
        // between its first and last owner
        const int sk_occ = sk_occ_known > 0 ? sk_occ_known : tile_sk_wg_per_cu(c);
        int64_t grid = sk_grid > 0 ? sk_grid : (int64_t)cus * sk_occ;
        if (sk_grid <= 0 && grid_per_cu8 > 0) grid = std::max<int64_t>(1, (int64_t)cus * grid_per_cu8 / 8);
        // equal shares per tile, as many as fit the co-resident grid (at least one)
        if (sk_grid <= 0 && grid_shares > 0) grid = T * std::max<int64_t>(1, std::min<int64_t>(grid_shares, grid / std::max<int64_t>(T, 1)));
        const bool chosen = sk_grid > 0 || grid_per_cu8 > 0 || grid_shares > 0;  // the grid is given: no alignment
        // Aligned split: when the tiles fit the co-resident grid S >= 2 times
        // over, a grid of exactly T * S workgroups (if it keeps 3/4 of the
        // slots busy) gives every tile S shares that start at the same k.
        // Tiles that share an operand panel then stream it through L2
        // together, as data-parallel tiles do (1536^2 x 16384 on 128x128
        // units: 107.5 us at 432 = 144 x 3 workgroups, 116.3 us at 512).
        // Tiles of different entries of a batch or group share no operand
        // panel, so only single products are aligned (an aligned 128x128 plan
        // for eight 16-row products took 54.6 us against 48.7 us on 64x64
        // Stream-K units).
        bool aligned = sk_grid <= 0 && grid_shares > 0;  // equal shares of every tile start at the same k
        if (!chosen && T < grid && !p.group && p.batch <= 1) {
            const int64_t S = grid / T;
            if (S >= 2 && 4 * T * S >= 3 * grid) {
                grid = T * S;
                aligned = true;
            }
        }
        grid = std::max<int64_t>(1, std::min(grid, T * I));
        const int64_t full = T / grid, rem = T % grid;
        int64_t dp_tiles = full >= 1 ? (full - 1) * grid : 0;
        (void)rem;
        const int64_t sk_tiles = T - dp_tiles;
        const int64_t W = sk_tiles * I;
        const int64_t per_wg = cdiv(W, grid);
        const double share = (double)std::min<int64_t>(sk_occ, cdiv(std::min<int64_t>(grid, W), cus));
        const int64_t dp_waves = dp_tiles / grid;
        // a split tile: every segment stores its partial (agent-coherent
        // stores), the last arrival reads all of them back
        const double partial = (double)c.bm * c.bn * 4;
        const int64_t nseg = per_wg >= I ? 2 : cdiv(I, per_wg) + 1;
        const bool splits = (W % grid != 0) || (I % per_wg != 0) || per_wg < I;
        // only rows below M travel (skinny problems move a sliver of each partial)
        const double rows_frac = std::min(1.0, (double)std::max<int64_t>(p.M, 1) / c.bm);
        // the last arrival's reads are latency-bound: about one memory round
        // trip per segment (the next partial's loads overlap the current add).
        // A fix-up kernel (six or more segments) costs about as much: its
        // launch and one read of the partials; the model keeps one estimate.
        const double fixup = splits ? rows_frac * partial / kL2BytesPerClk + nseg * (kFixupLatency + rows_frac * partial / kL2BytesPerClk) : 0.0;
        // a lone Stream-K workgroup keeps sk_stages - 1 K-steps of copies in
        // flight, which divides the latency part of its step
        const double sk_lone = kStepLatency / (c.sk_stages - 1) + (c.bm + c.bn) * (double)kStepBytes / kStepBytesPerClk;
        const double wg_step = std::max(step * share, lone_step);
        const double sk_wg_step = std::max(step * share, sk_lone);
        const double split_step = !aligned && c.bm * c.bn >= 128 * 128
                                      ? std::max(sk_wg_step, share * (c.bm + c.bn) * (double)kStepBytes / kStaggerBytesPerClk)
                                      : sk_wg_step;
        const double sk_frac = (double)sk_tiles / (double)T;
        const double rereads = aligned ? 0.0
                                       : sk_frac * (a_reads / (a_uniq <= kMallBytes ? kMallBytesPerClk : kHbmBytesPerClk) +
                                                    b_reads / (b_uniq <= kMallBytes ? kMallBytesPerClk : kHbmBytesPerClk));
        sk.cycles = std::max(dp_waves * (I * wg_step + tile_store * share) + per_wg * split_step + tile_store * share + fixup +
                                 (splits ? kSplitFixed : 0.0),
                             std::max(hbm_floor, rereads));
        sk.grid = (int)grid;
        sk.dp_tiles = dp_tiles;
        sk.sk_tiles = sk_tiles;
    }
    // Equal shares (the eight-wave config): its persistent Stream-K kernel
    // runs out of registers (the partial-tile sum on top of 128 accumulators
    // a wave) and spills inside the main loop, so its Stream-K is the split
    // aligned to whole tiles: each of the T tiles in S equal k shares, one
    // workgroup each, on the data-parallel loop, every share storing its
    // partial tile and a second kernel summing them.  S fills the co-resident
    // slots (at most kMaxSplit shares, each at least one K-step) unless the
    // equal-shares option gives a smaller S; a forced grid keeps the
    // persistent kernel.
    // All shares store their partials at once at the end, and the sum reads
    // them back: both at HBM rate.  A batch's tiles form one list (shares of
    // neighbouring tiles of one entry share operand panels, as in a single
    // product); groups and convolutions keep their own kernels.
    Estimate sp{1e300, 2, 0, 0, 0};
    if (split_config(ci) && !p.group && !p.conv && sk_grid <= 0 && grid_per_cu8 <= 0) {
        // (a second wave of shares costs a whole second round of K-steps:
        // 1536^2 x 16384 at 8 shares, 288 workgroups, ran 1.45x slower than
        // at 7; a tuned share count carried to a shape with more tiles is
        // capped the same way)
        const int64_t fit = slots / std::max<int64_t>(T, 1);
        int64_t S = grid_shares > 0 ? std::min<int64_t>(grid_shares, fit) : fit;
        S = std::min<int64_t>(std::min<int64_t>(S, kMaxSplit), I);
        if (S >= 2) {
            const int64_t per = cdiv(I, S);
            const int64_t busy = std::min<int64_t>(T * S, slots);
            const double share = (double)std::min<int64_t>(occ, cdiv(busy, cus));
            const double partials = (double)T * S * c.bm * c.bn * 4;
            const double c_bytes = (double)p.M * p.N * c_elem_bytes(p.c_type) * ((p.epilogue & kEpiAccumBit) ? 2 : 1);
            sp.cycles = std::max(cdiv(T * S, slots) * per * std::max(step * share, lone_step) +
                                     (2 * partials + c_bytes) / kHbmBytesPerClk + kSplitSum,
                                 hbm_floor);
            sp.grid = (int)(T * S);
            sp.dp_tiles = 0;
            sp.sk_tiles = T;
            sp.split = (int)S;
        }
    }
    if (force_mode == 1) return dp;
    if (force_mode == 2) return sp.split ? sp : sk;
    if (split_config(ci)) return sp.cycles < 0.97 * dp.cycles ? sp : dp;
    // the 32-row deep unit exists for its Stream-K pipeline (as data-parallel
    // tiles it is no faster than 64x64 ones on the products it may serve)
    if (c.bm < 64 && c.sk_stages > 2) return sk;
    return sk.cycles < 0.97 * dp.cycles ? sk : dp;
}

}  // namespace

bool gemv_wide_eligible(const Problem& p) {
    return (p.dtype == F16 || p.dtype == BF16) && !p.a_col && !p.b_col && !p.conv && !p.group && p.batch <= 1 &&
           p.M >= 1 && p.M <= kGemvWideRows && p.N >= 1 && p.K >= 1 && p.K <= (1LL << 22) && p.lda % 8 == 0 &&
           p.ldb % 8 == 0 && p.aligned && p.ldc < (1LL << 31) && p.M * p.lda * 2 < (1LL << 31) &&
           p.K * p.ldb * 2 < (1LL << 31);
}

bool gemv_narrow_eligible(const Problem& p) {
    const bool common = (p.dtype == F16 || p.dtype == BF16) && !p.a_col && !p.conv && !p.group && p.batch <= 1 &&
                        p.M >= 1 && p.M <= kGemvMaxRows && p.K >= 1 && p.K <= (1LL << 22) && p.lda % 8 == 0 &&
                        p.aligned && p.ldc < (1LL << 31) && p.lda < (1LL << 31);
    if (!common) return false;
    if (p.b_col)  // 16-byte pieces of k along every row of A and column of B; both below 2 GiB
        return p.K % 8 == 0 && p.ldb % 8 == 0 && p.N >= 1 && ((p.M - 1) * p.lda + p.K) * 2 < (1LL << 31) &&
               ((p.N - 1) * p.ldb + p.K) * 2 < (1LL << 31);
    return p.N >= 4 && p.N % 4 == 0 && p.ldb % 4 == 0 && (p.K - 1) * p.ldb * 2 + p.N * 2 < (1LL << 31);
}

namespace {
// a GEMV kernel can serve p under options o (gemv_wide = 1 leaves out the 16x16x32 kernel)
bool gemv_ok(const Problem& p, const Options& o) {
    return gemv_narrow_eligible(p) || (o.gemv_wide != 1 && gemv_wide_eligible(p));
}
// Row-major B: the 16x16x32 kernel wherever it can serve, unless option
// gemv_wide says never; the 4x4x4 one is left for rows of B that are not
// 16-byte aligned.  On N = K = 4096 (f16, block of calls) the 4x4x4 kernel
// takes 7.4 / 10.3 / 14.5 us at M = 1 / 8 / 16, the 16x16x32 one 6.6 / 8.6 /
// 8.6 us.
bool gemv_pick_wide(const Problem& p, const Options& o) {
    return gemv_wide_eligible(p) && o.gemv_wide != 1;
}
}  // namespace

bool gemv_eligible(const Problem& p) { return gemv_wide_eligible(p) || gemv_narrow_eligible(p); }

// The GEMV beats the tiled kernel's Stream-K plans on N = K = 4096 (f16,
// row-major B) up to 32 rows: 6.6 / 8.6 / 8.6 / 10.7 / 11.3 us at M = 1 / 8 /
// 16 / 24 / 32 against 10.9 / 11.0 / 11.4 / 11.8 / 12.5 us; at 48 rows it
// is slower (14.5 against 13.3 us).  Without the 16x16x32 kernel (column-
// major B, rows of B not 16-byte aligned) it stops at 8 rows.
constexpr int64_t kGemvAutoRows = 8, kGemvWideAutoRows = 32;
bool gemv_preferred(const Problem& p, const Options& o) {
    if (o.generic || o.gemv == 1 || o.force_config >= 0 || o.force_mode != 0 || o.sk_grid != 0) return false;
    if (!gemv_ok(p, o)) return false;
    return o.gemv == 2 || p.M <= kGemvAutoRows || (p.M <= kGemvWideAutoRows && gemv_pick_wide(p, o));
}

namespace {

// k ranges of the GEMV: about two workgroups per CU (the 16-row kernel's
// LDS and register budget), but the partial sums (splits x M x N x 4 bytes)
// kept within an eighth of B's bytes, and at most kGemvKMax rows a range.
constexpr int64_t kGemvKMax = 1024;
void gemv_plan(const Problem& p, const Options& o, int cus, Plan* pl) {
    pl->kernel = 3;
    pl->config = -1;
    pl->mode = 1;
    if (gemv_pick_wide(p, o)) {
        // 16x16x32 kernel: one workgroup per CU (at N = K = 4096 and 8 to 32
        // rows 8 k ranges beat 16 by 1.1-2.5 us: fewer partial sums), each k
        // range a multiple of a group of in-flight steps for all four waves
        // (4 x 4 x 32 k at 16 rows, 4 x 2 x 32 above) where K allows; an
        // asked-for count on the 128-row grid
        const int bucket = gemv_wide_rows_bucket(p.M);
        const int64_t nb = cdiv(p.N, kGemvWCols);
        int64_t kw;
        if (o.gemv_splits > 0) {
            kw = cdiv(cdiv(p.K, o.gemv_splits), kGemvWKAlign) * kGemvWKAlign;
        } else {
            const int64_t align = kGemvWKAlign * (bucket == 16 ? 4 : 2);
            kw = cdiv(cdiv(p.K, std::max<int64_t>(1, cus / nb)), align) * align;
        }
        const int64_t splits = cdiv(p.K, kw);
        pl->gemv_wide = true;
        pl->bm = bucket;
        pl->bn = kGemvWCols;
        pl->bk = (int)kw;
        pl->iters = splits;
        pl->tiles = nb;
        pl->grid = (int)(nb * splits);
        pl->dp_tiles = nb;
        pl->ws_partial_bytes = splits > 1 ? splits * p.M * p.N * 4 : 0;
        pl->fixup_kernel = splits > 1;
        return;
    }
    if (p.b_col) {
        // column-major B: every wave keeps its whole k range in flight, so a
        // range is one group of kGemvTSteps 32-k steps (256 rows) unless
        // more are asked for; many workgroups hide each other's latency
        const int64_t nb = cdiv(p.N, kGemvTCols);
        int64_t kw = kGemvTKAlign;
        if (o.gemv_splits > 0) kw = std::max<int64_t>(1, cdiv(cdiv(p.K, o.gemv_splits), kGemvTKAlign)) * kGemvTKAlign;
        const int64_t splits = cdiv(p.K, kw);
        pl->bm = 16;
        pl->bn = kGemvTCols;
        pl->bk = (int)kw;
        pl->iters = splits;
        pl->tiles = nb;
        pl->grid = (int)(nb * splits);
        pl->dp_tiles = nb;
        pl->ws_partial_bytes = splits > 1 ? splits * p.M * p.N * 4 : 0;
        pl->fixup_kernel = splits > 1;
        return;
    }
    const int64_t nb = cdiv(p.N, kGemvCols);
    int64_t splits = o.gemv_splits;
    if (splits <= 0) {
        splits = std::max<int64_t>(1, 2 * cus / nb);
        splits = std::min<int64_t>(splits, std::max<int64_t>(1, p.K / (16 * p.M)));
    }
    splits = std::max<int64_t>(1, std::min(splits, cdiv(p.K, kGemvKAlign)));
    int64_t kw = cdiv(cdiv(p.K, splits), kGemvKAlign) * kGemvKAlign;
    if (kw > kGemvKMax) kw = kGemvKMax;
    splits = cdiv(p.K, kw);
    pl->bm = gemv_rows_bucket(p.M);
    pl->bn = kGemvCols;
    pl->bk = (int)kw;
    pl->iters = splits;
    pl->tiles = nb;
    pl->grid = (int)(nb * splits);
    pl->dp_tiles = nb;
    pl->ws_partial_bytes = splits > 1 ? splits * p.M * p.N * 4 : 0;
    pl->fixup_kernel = splits > 1;
}

}  // namespace

bool make_plan(const Problem& p, const Options& o, int cus, Plan* out) {
    Plan pl;
    if (p.M < 0 || p.N < 0 || p.K < 0) return false;
    if (p.M == 0 || p.N == 0) {
        pl.kernel = 0;
        *out = pl;
        return true;
    }
    if (cus <= 0) cus = kDefaultCUs;
    if (gemv_ok(p, o) && (gemv_preferred(p, o) || (o.gemv == 2 && !o.generic && o.force_config < 0))) {
        gemv_plan(p, o, cus, &pl);
        *out = pl;
        return true;
    }
    int best = -1;
    Estimate best_e{1e300, 1, 0, 0, 0};
    if (!o.generic) {
        for (int c = 0; c < kNumConfigs; ++c) {
            if (o.force_config >= 0 && c != o.force_config) continue;
            // the 32-row deep unit is planned for products of one tile row
            // (M <= 32; a group counts all its rows) unless it is forced
            if (o.force_config < 0 && kConfigs[c].bm < 64 && kConfigs[c].sk_stages > 2 && p.M > kConfigs[c].bm) continue;
            if (p.group ? !p.group_ok[c] : !tile_eligible(p, kConfigs[c])) continue;
            Estimate e = estimate(p, c, cus, o.force_mode, o.sk_grid, o.sk_occ[c], o.grid_per_cu8, o.grid_shares);
            // the eight-wave config's Stream-K is its equal shares; where they
            // cannot serve (tiles filling more than half the CUs, a group, a
            // given grid) it would run the persistent kernel, which spills
            // registers: a forced Stream-K then picks among the other configs
            // unless that config is forced too
            if (o.force_mode == 2 && o.force_config < 0 && split_config(c) && e.split == 0) continue;
            // configs run from large tiles to small: a smaller tile must be
            // clearly cheaper, since the model underrates its extra operand
            // traffic (2560 x 4096 x 4096: 64x64 tiles estimated 0.7% below
            // 256x256 ones, measured 140.9 against 96.7 us)
            if (e.cycles < best_e.cycles * 0.97) {
                best = c;
                best_e = e;
            }
        }
        // a forced config that cannot serve the call falls back to the planner's choice
        if (best < 0 && o.force_config >= 0) {
            Options o2 = o;
            o2.force_config = -1;
            return make_plan(p, o2, cus, out);
        }
    }
    if (best < 0) {
        pl.kernel = 1;
        pl.bm = pl.bn = 64;
        pl.bk = 64 / elem_bytes(p.dtype);
        pl.tiles = cdiv(p.M, 64) * cdiv(p.N, 64) * std::max<int64_t>(p.batch, 1);
        pl.iters = cdiv(p.K, pl.bk);
        pl.mode = 1;
        pl.grid = (int)std::min<int64_t>(pl.tiles, (1LL << 31) - 1);
        pl.dp_tiles = pl.tiles;
        if (pl.tiles >= (1LL << 31)) return false;
        *out = pl;
        return true;
    }
    const TileConfig& c = kConfigs[best];
    pl.kernel = 2;
    pl.config = best;
    pl.bm = c.bm;
    pl.bn = c.bn;
    pl.bk = bk_elems(p.dtype);
    pl.tiles = tile_count(p, best);
    pl.iters = cdiv(p.K, pl.bk);
    pl.mode = best_e.mode;
    pl.est_cycles = best_e.cycles;
    if (pl.mode == 1) {
        pl.grid = (int)pl.tiles;
        pl.dp_tiles = pl.tiles;
        pl.sk_tiles = 0;
    } else {
        pl.grid = best_e.grid;
        pl.dp_tiles = best_e.dp_tiles;
        pl.sk_tiles = best_e.sk_tiles;
        pl.ws_partial_bytes = 2LL * pl.grid * c.bm * c.bn * 4;
        pl.ws_counters = pl.sk_tiles;
        if (best_e.split > 1) {  // equal shares: one partial a workgroup, summed by the second kernel
            pl.split = best_e.split;
            pl.ws_partial_bytes = (int64_t)pl.grid * c.bm * c.bn * 4;
            pl.ws_counters = 0;
            pl.fixup_kernel = true;
            pl.group_m = o.group_m > 0 ? o.group_m : 4;
            *out = pl;
            return true;
        }
        // Split tiles cut into many short segments are summed by a second
        // kernel: the segments then store their partials and end, instead
        // of waiting for the stores, counting their arrival and having the
        // last arrival read the others back (M = 1 / 16 / 64 with N = K =
        // 4096 on 64x64 units, eight segments a tile: 13.2 / 13.4 / 15.8 us
        // in the kernel, 12.2 / 12.5 / 14.0 us with the second kernel;
        // 1280^2 x 5120 on 128x128 units in five aligned shares: 39.3 us by
        // the last arrival, 35.2 us with the second kernel; at three or four
        // segments a tile the launch costs more than it saves).
        const int64_t per_wg = (pl.sk_tiles * pl.iters + pl.grid - 1) / pl.grid;
        pl.fixup_kernel = o.sk_fixup == 2 || (o.sk_fixup == 0 && pl.iters >= 5 * per_wg);
    }
    pl.group_m = o.group_m > 0 ? o.group_m : 4;
    *out = pl;
    return true;
}

}  // namespace tcm
