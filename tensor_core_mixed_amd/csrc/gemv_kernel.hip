// Split-k GEMV kernels for products of at most 16 rows: C = epi(A B + bias)
// with A (M x K, M <= 16) row-major and B (K x N) row-major or, in the
// second kernel below, column-major; f16 or bf16.
//
// Such a product is bound by streaming B once from HBM: it moves K*N
// operand elements for 2*M*K*N flops, far below the MFMA ridge.  The tiled
// kernel serves it with a 32- or 64-row MFMA tile (at M = 1, 31 of 32 rows
// are padding), stages every K-step of B through LDS to transpose it into
// k-contiguous fragments, and sums Stream-K partial tiles.  Here B never
// goes through LDS: every wave-wide load is one 512-byte run of one row of B
// (64 lanes x 4 columns of 2 bytes), and the lane multiplies the 4 x 4
// block it holds after four such rows on the matrix cores'
// v_mfma_f32_4x4x4_16b, whose 16 independent 4x4x4 blocks let each lane
// bring its own columns (see mul_rows_mfma).  Measured on N = K = 4096:
// that instruction issues in about 4 ns per SIMD (1024 multiply-adds), the
// VALU v_dot2_f32_f16 in about 1.9 ns (128), so an earlier dot-product
// inner loop was 4-30% slower from M = 4 on.
//
// Work split (the even k-split of the Stream-K reproduction post on
// leiblog.wang, applied across workgroups of one column block): workgroup
// (x, y) owns 256 columns and the k range [kw y, kw y + kw); its four waves
// take a quarter of that range each, 16 rows per chunk, the loads of chunk
// c+1 in flight while chunk c is multiplied.  The four waves' sums meet in
// LDS and are added in wave order; with more than one k range the sum is a
// partial stored to the workspace, and a second kernel adds the ranges in
// order and runs the epilogue, so the result does not depend on timing.
// (Letting the last workgroup of a column block add the ranges instead,
// after an arrival counter, was slower at every M: 9.0 against 7.3 us at
// M = 1, 27 against 15 us at M = 16.)
//
// Rows of B at or past K read as zeros (buffer range check); the A columns
// past K are zero in LDS, so no padding value reaches a sum.  Columns at or
// past N are neither loaded nor stored (N is a multiple of 4).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemv.h"
#include "tcm_internal.h"

namespace tcm {
namespace gemv {

typedef unsigned u2_t __attribute__((ext_vector_type(2)));
typedef unsigned u4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef short s4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;                 // four waves
constexpr int kChunk = 16;                    // rows of B per wave per pipeline step
constexpr unsigned kOOB = 0x80000000u;        // beyond every buffer range used here: loads read zeros
constexpr int kRsrcWord3 = 0x00020000;

template <int DT>
__device__ __forceinline__ float to_f32(unsigned short h) {
    if constexpr (DT == F16) return (float)__builtin_bit_cast(_Float16, h);
    else return __builtin_bit_cast(float, (unsigned)h << 16);
}

// Partial sums: splits x M x N floats.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const GemvArgs& g) {
    const int64_t bytes = (int64_t)g.splits * g.M * g.N * 4;
    return __builtin_amdgcn_make_buffer_rsrc(g.partial, (short)0, bytes < (int64_t)kOOB ? (int)bytes : (int)kOOB, kRsrcWord3);
}
// sum over y = 0, 1, .. of the partial at byte offset off + y * mn * 4, in
// that order: the loads of up to 32 k ranges are issued before any is added
__device__ __forceinline__ float sum_splits(const GemvArgs& g, __amdgpu_buffer_rsrc_t rp, unsigned off, int64_t mn) {
    const unsigned step = (unsigned)(mn * 4);
    float s = 0.f;
    for (int y0 = 0; y0 < g.splits; y0 += 32) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j)
            v[j] = y0 + j < g.splits
                       ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, off + (unsigned)(y0 + j) * step, 0, 0))
                       : 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j)
            if (y0 + j < g.splits) s += v[j];
    }
    return s;
}

// C[m][n] = epi(init + s): init = C_in (with accum) + bias, in binary32;
// ReLU; stored in C's type (16-bit types rounded to nearest even).
__device__ __forceinline__ void finish(const GemvArgs& g, int m, int n, float s) {
    char* c = (char*)g.C;
    const int64_t idx = (int64_t)m * g.ldc + n;
    float init = 0.f;
    if (g.accum) {
        if (g.c_type == C_F16) init = to_f32<F16>(((const unsigned short*)c)[idx]);
        else if (g.c_type == C_BF16) init = to_f32<BF16>(((const unsigned short*)c)[idx]);
        else init = ((const float*)c)[idx];
    }
    if (g.has_bias) init = init + ((const float*)g.bias)[n];
    float v = init + s;
    if (g.relu) v = v > 0.f ? v : 0.f;
    if (g.c_type == C_F16) ((_Float16*)c)[idx] = (_Float16)v;
    else if (g.c_type == C_BF16) ((__bf16*)c)[idx] = (__bf16)v;
    else ((float*)c)[idx] = v;
}

template <int DT, int MB>
struct Gemv {
    static constexpr int D = 2;  // register sets of B chunks (four measured no faster)
    static constexpr int KW_MAX = 1024;  // k per workgroup the LDS copy of A holds (host keeps kw <= this)
    // A rows in LDS are kw + 8 elements apart: the four rows one 4x4x4 step
    // reads (lanes 4b+i read row i) then fall on different banks (kw alone
    // is a multiple of 128 bytes: a 4-way bank conflict)
    static constexpr int kRowPad = 8;

    // chunk of 16 rows of B for one lane: 4 columns (8 bytes) per row
    struct Rows {
        u2_t v[kChunk];
    };

    __device__ __forceinline__ static void load_rows(Rows& r, __amdgpu_buffer_rsrc_t rb, unsigned lane_off, int k, int K,
                                                     int ldb_bytes) {
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const unsigned off = (k + i < K && lane_off != kOOB) ? (unsigned)((k + i) * ldb_bytes) + lane_off : kOOB;
            r.v[i] = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(rb, off, 0, 0));
        }
    }

    // The product on the matrix cores: v_mfma_f32_4x4x4_16b runs 16
    // independent 4x4x4 blocks, lane 4b+i giving row i of block b's A (4 k
    // values), lane 4b+j column j of its B, and getting column j of its D
    // (4 rows).  Every block here takes the same A (4 rows of the product),
    // and lane l gives one of its own columns as B: one instruction covers 4
    // rows x 64 columns x 4 k.  The 4 x 4 block of B a lane loads (4 rows of
    // 4 columns) is transposed in registers, two v_perm per column.
    static constexpr int MG = MB < 4 ? 1 : MB / 4;  // row groups of 4
    __device__ __forceinline__ static void mul_rows_mfma(f4_t (&acc)[MG][4], const Rows& r, const unsigned short* sAh, int kw,
                                                         int kc, int lane) {
#pragma unroll
        for (int q = 0; q < kChunk / 4; ++q) {
            const u2_t r0 = r.v[4 * q], r1 = r.v[4 * q + 1], r2 = r.v[4 * q + 2], r3 = r.v[4 * q + 3];
            u2_t bc[4];  // column c of the block: (B[k][c], B[k+1][c]) (B[k+2][c], B[k+3][c])
            bc[0] = u2_t{__builtin_amdgcn_perm(r1[0], r0[0], 0x05040100u), __builtin_amdgcn_perm(r3[0], r2[0], 0x05040100u)};
            bc[1] = u2_t{__builtin_amdgcn_perm(r1[0], r0[0], 0x07060302u), __builtin_amdgcn_perm(r3[0], r2[0], 0x07060302u)};
            bc[2] = u2_t{__builtin_amdgcn_perm(r1[1], r0[1], 0x05040100u), __builtin_amdgcn_perm(r3[1], r2[1], 0x05040100u)};
            bc[3] = u2_t{__builtin_amdgcn_perm(r1[1], r0[1], 0x07060302u), __builtin_amdgcn_perm(r3[1], r2[1], 0x07060302u)};
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                const u2_t a = *(const u2_t*)(sAh + (4 * g + (lane & 3)) * (kw + kRowPad) + kc + 4 * q);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if constexpr (DT == F16)
                        acc[g][c] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4_t, a), __builtin_bit_cast(h4_t, bc[c]),
                                                                       acc[g][c], 0, 0, 0);
                    else
                        acc[g][c] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s4_t, a),
                                                                           __builtin_bit_cast(s4_t, bc[c]), acc[g][c], 0, 0, 0);
                }
            }
        }
    }

    // LDS: the A block (at least 4 rows) while the waves multiply, then their four sums
    static constexpr int MBA = MB < 4 ? 4 : MB;
    static constexpr int A_BYTES = MBA * (KW_MAX + kRowPad) * 2, RED_BYTES = 4 * MB * kGemvCols * 4;
    static constexpr int LDS_BYTES = A_BYTES > RED_BYTES ? A_BYTES : RED_BYTES;

    __device__ static void run(const GemvArgs& g) {
        __shared__ __attribute__((aligned(16))) unsigned lds[LDS_BYTES / 4];
        unsigned* sA = lds;
        float(*red)[MB][kGemvCols] = (float(*)[MB][kGemvCols])lds;
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int n0 = blockIdx.x * kGemvCols;
        const int kw = g.kw, k0 = blockIdx.y * kw;
        const int rw = kw / 4;  // rows per wave
        const int kb = k0 + wave * rw;

        // B: one buffer range over all of it, from column n0 on
        const int ldb_bytes = g.ldb * 2;
        const int64_t rb_bytes = g.b_bytes - (int64_t)n0 * 2;
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (char*)g.B + (int64_t)n0 * 2, (short)0, rb_bytes < (int64_t)kOOB ? (int)rb_bytes : (int)kOOB, kRsrcWord3);
        const unsigned lane_off = n0 + 4 * lane < g.N ? (unsigned)(8 * lane) : kOOB;

        // A block [MB][kw] into LDS, rows kw + kRowPad apart (rows past M and columns past K as zeros):
        // its loads are issued before the first chunk of B, so waiting for
        // them leaves B's in flight
        const unsigned short* A = (const unsigned short*)g.A;
        const int per_row = kw / 8;  // 16-byte pieces per row
        for (int i = tid; i < MBA * per_row; i += kThreads) {
            const int m = i / per_row, k = k0 + 8 * (i - m * per_row);
            u4_t v = {0u, 0u, 0u, 0u};
            if (m < g.M && k < g.K) {
                const unsigned short* src = A + (int64_t)m * g.lda + k;
                if (k + 8 <= g.K) {
                    v = *(const u4_t*)src;
                } else {
                    unsigned short e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = k + j < g.K ? src[j] : (unsigned short)0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = (unsigned)e[2 * j] | ((unsigned)e[2 * j + 1] << 16);
                }
            }
            *(u4_t*)(sA + (m * (kw + kRowPad) + 8 * (i - m * per_row)) / 2) = v;
        }

        // a ring of D register sets: the loads of chunks c+1 .. c+D-1 are in
        // flight while chunk c is multiplied (the counter of outstanding
        // loads, 63 at most, holds (D - 1) x 16 of them)
        static_assert((D - 1) * kChunk <= 63, "loads in flight within the vmcnt range");
        Rows ring[D];
        const int chunks = rw / kChunk;
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (j < chunks) load_rows(ring[j], rb, lane_off, kb + j * kChunk, g.K, ldb_bytes);
        __syncthreads();  // sA written
        const unsigned short* sAh = (const unsigned short*)sA;
        f4_t acc[MG][4];
#pragma unroll
        for (int q = 0; q < MG; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[q][c] = f4_t{0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < chunks; c += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if (c + j < chunks) {
                    mul_rows_mfma(acc, ring[j], sAh, kw, wave * rw + (c + j) * kChunk, lane);
                    if (c + j + D < chunks) load_rows(ring[j], rb, lane_off, kb + (c + j + D) * kChunk, g.K, ldb_bytes);
                }
            }
        }
        __syncthreads();  // the A block is dead
        // row 4q+i of the product, columns 4 lane .. 4 lane + 3
#pragma unroll
        for (int q = 0; q < MG; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * q + i < MB) *(f4_t*)&red[wave][4 * q + i][4 * lane] = f4_t{acc[q][0][i], acc[q][1][i], acc[q][2][i], acc[q][3][i]};
        // the four waves' sums, added in wave order
        __syncthreads();
        const int n = n0 + tid;
        const bool col = n < g.N;
        if (g.splits == 1) {
            if (!col) return;
#pragma unroll
            for (int m = 0; m < MB; ++m)
                if (m < g.M) finish(g, m, n, ((red[0][m][tid] + red[1][m][tid]) + red[2][m][tid]) + red[3][m][tid]);
            return;
        }
        // the k range's partial sums, added by the second kernel
        const int64_t mn = (int64_t)g.M * g.N;
        const __amdgpu_buffer_rsrc_t rp = partial_rsrc(g);
#pragma unroll
        for (int m = 0; m < MB; ++m)
            if (m < g.M && col)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(int, ((red[0][m][tid] + red[1][m][tid]) + red[2][m][tid]) + red[3][m][tid]), rp,
                    (unsigned)((blockIdx.y * mn + (int64_t)m * g.N + n) * 4), 0, 0);
    }
};

template <int DT, int MB>
__global__ __launch_bounds__(kThreads) void gemv_split_kernel(GemvArgs g) {
    Gemv<DT, MB>::run(g);
}

// Output (m, n) = epi(init + sum over splits y, in order, of partial[y][m][n]).
__global__ __launch_bounds__(kThreads) void gemv_reduce_kernel(GemvArgs g) {
    const int64_t mn = (int64_t)g.M * g.N;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= mn) return;
    const int m = (int)(i / g.N), n = (int)(i - (int64_t)m * g.N);
    finish(g, m, n, sum_splits(g, partial_rsrc(g), (unsigned)(i * 4), mn));
}

// ------------------------------------------------------ column-major B
// B stored column-major (k contiguous: a weight matrix kept as [N][K]).
// Here the memory layout is the matrix cores' operand layout: for
// v_mfma_f32_16x16x32, lane l (j = l & 15, g = l >> 4) gives 8 consecutive
// k (16 bytes) from k = 8g of row j of A and of column j of B.  So each lane
// loads 16 bytes of column n + j of B and 16 bytes of row j of A (rows past
// M read as zeros) and one instruction covers 16 rows x 16 columns x 32 k:
// no LDS, no transpose.  A wave owns 32 columns (two groups of 16) of the
// workgroup's 128 over the whole k range, with the loads of kGemvTSteps
// 32-k steps (three 16-byte loads each) in flight at once; waves share
// nothing.  Each load instruction reads 64 contiguous bytes of 16 columns;
// the next step reads the rest of those 128-byte lines.
template <int DT>
__global__ __launch_bounds__(kThreads) void gemv_t_kernel(GemvArgs g) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, grp = lane >> 4;
    const int n_wave = blockIdx.x * kGemvTCols + wave * 32;
    const int k0 = blockIdx.y * g.kw;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.A, (short)0, g.a_bytes < (int64_t)kOOB ? (int)g.a_bytes : (int)kOOB, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.B, (short)0, g.b_bytes < (int64_t)kOOB ? (int)g.b_bytes : (int)kOOB, kRsrcWord3);
    const unsigned a_row = j < g.M ? (unsigned)(j * g.lda) * 2u : kOOB;  // bytes to row j of A
    unsigned b_colp[2];                                                   // bytes to this lane's columns of B
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
        const int n = n_wave + 16 * cg + j;
        b_colp[cg] = n < g.N ? (unsigned)((int64_t)n * g.ldb * 2) : kOOB;
    }
    f4_t acc[2] = {f4_t{0.f, 0.f, 0.f, 0.f}, f4_t{0.f, 0.f, 0.f, 0.f}};
    const int steps = g.kw / 32;
    for (int s0 = 0; s0 < steps; s0 += kGemvTSteps) {
        u4_t av[kGemvTSteps], bv[kGemvTSteps][2];
#pragma unroll
        for (int i = 0; i < kGemvTSteps; ++i) {
            const int k = k0 + 32 * (s0 + i) + 8 * grp;  // K is a multiple of 8: a piece lies wholly below K or not
            const bool in = k < g.K;
            av[i] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                 ra, in && a_row != kOOB ? a_row + 2u * (unsigned)k : kOOB, 0, 0));
#pragma unroll
            for (int cg = 0; cg < 2; ++cg)
                bv[i][cg] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rb, in && b_colp[cg] != kOOB ? b_colp[cg] + 2u * (unsigned)k : kOOB, 0, 0));
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the group issued before the first multiply waits
#pragma unroll
        for (int i = 0; i < kGemvTSteps; ++i)
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) {
                if constexpr (DT == F16)
                    acc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, av[i]),
                                                                     __builtin_bit_cast(h8_t, bv[i][cg]), acc[cg], 0, 0, 0);
                else
                    acc[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, av[i]),
                                                                      __builtin_bit_cast(b8_t, bv[i][cg]), acc[cg], 0, 0, 0);
            }
    }
    // lane l holds rows 4g .. 4g+3 of columns n_wave + 16 cg + j
    const int64_t mn = (int64_t)g.M * g.N;
    const __amdgpu_buffer_rsrc_t rp = partial_rsrc(g);
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
        const int n = n_wave + 16 * cg + j;
        if (n >= g.N) continue;
        // the whole vector is cast, then indexed: hipcc miscompiles the bit
        // cast of one element of a vector (it yields element 0)
        const i4_t bits = __builtin_bit_cast(i4_t, acc[cg]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int m = 4 * grp + t;
            if (m >= g.M) break;
            if (g.splits > 1)
                __builtin_amdgcn_raw_buffer_store_b32(bits[t], rp, (unsigned)((blockIdx.y * mn + (int64_t)m * g.N + n) * 4),
                                                      0, 0);
            else
                finish(g, m, n, acc[cg][t]);
        }
    }
}

// ------------------------------------------- row-major B, up to 64 rows
// The layout of the first kernel (B n-contiguous) on the full-rate
// v_mfma_f32_16x16x32, whose B operand wants 8 consecutive k of one column
// per lane.  A lane loads 8 consecutive rows of B, 16 bytes (8 columns) of
// each, and transposes that 8 x 8 block in registers: column j's 8 k values,
// two per register, take 4 v_perm.  The 16 lanes of lane group g
// (16g .. 16g+15) hold the same 8 rows, k = 8g .. 8g+7 of the step, so they
// fill the instruction's 16 column slots and its k layout: issue j of a step
// multiplies columns n0 + 8c + j (c = lane & 15), and A's operand is one
// 16-byte load per 16-row block in its own layout (row c, k = 8g ..).  A
// wave covers 128 columns x 32 k per step with 8 loads of B and one of A per
// 16 rows; B never goes through LDS, and at 64 rows the matrix cores need
// about a quarter of the time B's bytes take.
//
// Work split as in the first kernel: workgroup (x, y) owns 128 columns and
// the k range [kw y, kw y + kw); wave w takes its 32-k steps w, w + 4, ...,
// the loads of wide_steps<MB>() of them in flight together.  The four waves'
// sums meet in LDS and are added in wave order, then stored as a partial
// (several k ranges) or through the epilogue (one).
//
// Rows of B at or past K read as zeros (buffer range check); A's k past K
// are zeroed in registers, so a padding value never reaches a sum.  Columns
// at or past N come from whatever the row holds there and are never stored.

// keep the first nv (1 .. 7) of the 8 halves of v
__device__ __forceinline__ u4_t keep_low_halves(u4_t v, int nv) {
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = 2 * d + 1 < nv ? v[d] : (2 * d < nv ? (v[d] & 0xffffu) : 0u);
    return v;
}

// 32-k steps per wave whose loads are in flight together: at 16 rows four
// (216 registers), at 32 two, so that the accumulators stay in the 256
// registers of two waves per SIMD (with four, or at 64 rows, the compiler
// moves them through the accumulation registers every step)
template <int MB>
constexpr int wide_steps() { return MB == 16 ? 4 : 2; }

// NS 32-k steps of one wave, from step s (then s + 4, ...): every load of
// the group issued before the first multiply waits for its data
template <int DT, int RB, int NS>
__device__ __forceinline__ void wide_group(f4_t (&acc)[RB][8], __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                           const unsigned (&a_row)[RB], unsigned b_lane, unsigned ldb_bytes, int kb, int K) {
    u4_t bv[NS][8], av[NS][RB];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int k = kb + 128 * i;  // this lane's 8 rows of B and 8 k of A
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const unsigned off = k + r < K && b_lane != kOOB ? (unsigned)(k + r) * ldb_bytes + b_lane : kOOB;
            bv[i][r] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
        }
#pragma unroll
        for (int q = 0; q < RB; ++q) {
            const unsigned off = k < K && a_row[q] != kOOB ? a_row[q] + 2u * (unsigned)k : kOOB;
            av[i][q] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int k = kb + 128 * i;
        if (k < K && k + 8 > K) {  // A's piece ends past K: zero those k (B's rows there read as zeros)
#pragma unroll
            for (int q = 0; q < RB; ++q) av[i][q] = keep_low_halves(av[i][q], K - k);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // column n0 + 8c + j at k .. k+7: (row 2p, row 2p+1) halves j of the lane's rows
            const int d = j >> 1;
            const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
            const u4_t bt = u4_t{__builtin_amdgcn_perm(bv[i][1][d], bv[i][0][d], sel),
                                 __builtin_amdgcn_perm(bv[i][3][d], bv[i][2][d], sel),
                                 __builtin_amdgcn_perm(bv[i][5][d], bv[i][4][d], sel),
                                 __builtin_amdgcn_perm(bv[i][7][d], bv[i][6][d], sel)};
#pragma unroll
            for (int q = 0; q < RB; ++q) {
                if constexpr (DT == F16)
                    acc[q][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, av[i][q]),
                                                                       __builtin_bit_cast(h8_t, bt), acc[q][j], 0, 0, 0);
                else
                    acc[q][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, av[i][q]),
                                                                        __builtin_bit_cast(b8_t, bt), acc[q][j], 0, 0, 0);
            }
        }
    }
}

template <int DT, int MB>
__global__ __launch_bounds__(kThreads, MB <= 32 ? 2 : 1) void gemv_r_kernel(GemvArgs g) {
    constexpr int RB = MB / 16;  // 16-row blocks
    constexpr int S = wide_steps<MB>();
    static_assert(S * (8 + RB) <= 63, "loads in flight within the vmcnt range");
    __shared__ __attribute__((aligned(16))) float red[4][MB][kGemvWCols];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, grp = lane >> 4;
    const int n0 = blockIdx.x * kGemvWCols;
    const int k0 = blockIdx.y * g.kw, K = g.K;
    // The ranges end at the 16-byte boundary past each operand's last
    // element: the range check zeroes a whole dword that crosses the end, and
    // the last piece of A's last row (K odd) or of B's last row (N not a
    // multiple of 8) holds elements that are used.  A, B and their rows are
    // 16-byte aligned, so that boundary lies in the same page as the
    // element; the bytes past it are masked (A) or feed only columns past N.
    const int64_t a_lim = (g.a_bytes + 15) & ~(int64_t)15, b_lim = (g.b_bytes + 15) & ~(int64_t)15;
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, a_lim < (int64_t)kOOB ? (int)a_lim : (int)kOOB, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)g.B, (short)0, b_lim < (int64_t)kOOB ? (int)b_lim : (int)kOOB, kRsrcWord3);
    const unsigned ldb_bytes = (unsigned)g.ldb * 2u;
    const unsigned b_lane = n0 + 8 * c < g.N ? (unsigned)(n0 + 8 * c) * 2u : kOOB;  // bytes to this lane's columns
    unsigned a_row[RB];                                                             // bytes to this lane's rows of A
#pragma unroll
    for (int q = 0; q < RB; ++q) a_row[q] = 16 * q + c < g.M ? (unsigned)((16 * q + c) * g.lda) * 2u : kOOB;
    f4_t acc[RB][8];
#pragma unroll
    for (int q = 0; q < RB; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[q][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    // groups of S steps, then the range's last steps one at a time (the
    // host makes kw a multiple of 4 S steps where K allows)
    const int steps = g.kw / 32;
    int s0 = wave;
    for (; s0 + 4 * (S - 1) < steps; s0 += 4 * S)
        wide_group<DT, RB, S>(acc, ra, rb, a_row, b_lane, ldb_bytes, k0 + 32 * s0 + 8 * grp, K);
    for (; s0 < steps; s0 += 4) wide_group<DT, RB, 1>(acc, ra, rb, a_row, b_lane, ldb_bytes, k0 + 32 * s0 + 8 * grp, K);
    // lane l holds rows 16q + 4g + t (t = 0 .. 3) of columns n0 + 8c + j
#pragma unroll
    for (int q = 0; q < RB; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int m = 16 * q + 4 * grp + t;
            if (m < g.M) {
                *(f4_t*)&red[wave][m][8 * c] = f4_t{acc[q][0][t], acc[q][1][t], acc[q][2][t], acc[q][3][t]};
                *(f4_t*)&red[wave][m][8 * c + 4] = f4_t{acc[q][4][t], acc[q][5][t], acc[q][6][t], acc[q][7][t]};
            }
        }
    __syncthreads();
    // the four waves' sums, added in wave order: thread t takes column t mod 128 of every other row
    const int col = tid & (kGemvWCols - 1), n = n0 + col;
    if (n >= g.N) return;
    const int64_t mn = (int64_t)g.M * g.N;
    for (int m = tid / kGemvWCols; m < MB && m < g.M; m += kThreads / kGemvWCols) {
        const float s = ((red[0][m][col] + red[1][m][col]) + red[2][m][col]) + red[3][m][col];
        if (g.splits == 1)
            finish(g, m, n, s);
        else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, s), partial_rsrc(g),
                                                  (unsigned)((blockIdx.y * mn + (int64_t)m * g.N + n) * 4), 0, 0);
    }
}

template <int DT>
int launch_dt(const GemvArgs& a, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (a.wide) {
        const dim3 grid_w((unsigned)((a.N + kGemvWCols - 1) / kGemvWCols), (unsigned)a.splits);
        switch (gemv_wide_rows_bucket(a.M)) {
        case 16: hipLaunchKernelGGL((gemv_r_kernel<DT, 16>), grid_w, dim3(kThreads), 0, s, a); break;
        case 32: hipLaunchKernelGGL((gemv_r_kernel<DT, 32>), grid_w, dim3(kThreads), 0, s, a); break;
        default: hipLaunchKernelGGL((gemv_r_kernel<DT, 64>), grid_w, dim3(kThreads), 0, s, a); break;
        }
        int st = (int)hipGetLastError();
        if (st != 0 || a.splits <= 1) return st;
        const int64_t mn = (int64_t)a.M * a.N;
        hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((mn + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
        return (int)hipGetLastError();
    }
    if (a.b_col) {
        const dim3 grid_t((unsigned)((a.N + kGemvTCols - 1) / kGemvTCols), (unsigned)a.splits);
        hipLaunchKernelGGL((gemv_t_kernel<DT>), grid_t, dim3(kThreads), 0, s, a);
        int st = (int)hipGetLastError();
        if (st != 0 || a.splits <= 1) return st;
        const int64_t mn = (int64_t)a.M * a.N;
        hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((mn + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
        return (int)hipGetLastError();
    }
    const dim3 grid((unsigned)((a.N + kGemvCols - 1) / kGemvCols), (unsigned)a.splits);
    switch (gemv_rows_bucket(a.M)) {
    case 1: hipLaunchKernelGGL((gemv_split_kernel<DT, 1>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemv_split_kernel<DT, 2>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemv_split_kernel<DT, 4>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((gemv_split_kernel<DT, 8>), grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((gemv_split_kernel<DT, 16>), grid, dim3(kThreads), 0, s, a); break;
    }
    int st = (int)hipGetLastError();
    if (st != 0 || a.splits <= 1) return st;
    const int64_t mn = (int64_t)a.M * a.N;
    hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((mn + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
    return (int)hipGetLastError();
}

}  // namespace gemv

int launch_gemv(int dtype, const GemvArgs& a, void* stream) {
    if (a.M < 1 || a.M > (a.wide ? kGemvWideRows : kGemvMaxRows) || a.N < 1 || a.splits < 1 ||
        (int64_t)a.splits * a.kw < a.K || (a.splits > 1 && !a.partial) ||
        (int64_t)a.splits * a.M * a.N * 4 >= (int64_t)gemv::kOOB)
        return (int)hipErrorInvalidValue;
    if (a.wide) {  // 16-byte pieces of rows of A and B; every offset below 2 GiB
        if (a.b_col || a.kw < kGemvWKAlign || a.kw % kGemvWKAlign || a.lda % 8 || a.ldb % 8 ||
            a.a_bytes >= (int64_t)gemv::kOOB || (int64_t)a.K * a.ldb * 2 >= (int64_t)gemv::kOOB ||
            (int64_t)a.M * a.lda * 2 >= (int64_t)gemv::kOOB)
            return (int)hipErrorInvalidValue;
    } else if (a.b_col ? (a.kw < kGemvTKAlign || a.kw % kGemvTKAlign || a.K % 8 || a.a_bytes >= (int64_t)gemv::kOOB ||
                          a.b_bytes >= (int64_t)gemv::kOOB)
                       : (a.N % 4 || a.kw < kGemvKAlign || a.kw % kGemvKAlign || a.kw > gemv::Gemv<F16, 1>::KW_MAX)) {
        return (int)hipErrorInvalidValue;
    }
    if (dtype == F16) return gemv::launch_dt<F16>(a, stream);
    if (dtype == BF16) return gemv::launch_dt<BF16>(a, stream);
    return (int)hipErrorInvalidValue;
}

}  // namespace tcm
