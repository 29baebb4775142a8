// Tiled MFMA GEMM kernel for gfx950 (CDNA4), one template for all element
// types.  What each part implements, with the passage that describes it:
//
//  * Tiling + loop order (kimm240.github.io/tvm, GEMM optimisation Step 2):
//    C is cut into BM x BN macro tiles, one per workgroup; each of the
//    WM x WN waves owns a (BM/WM) x (BN/WN) block of 32x32 MFMA tiles whose
//    accumulators stay in registers for the whole k loop.
//  * Cooperative staging through LDS (same page, Step 3): the lanes of the
//    workgroup's copier waves (all waves, or half of them in the eight-wave
//    kernel) copy the A and B k-slabs of one K-step into LDS with 16-byte
//    direct-to-LDS buffer loads (one lane = one 16-byte chunk; a wave
//    instruction fills 1 KiB of LDS), coalesced along the contiguous
//    dimension of each operand.  A convolution gathers A from its NHWC
//    input instead (implicit GEMM).
//  * Bank-conflict-free LDS layout (leiblog.wang, the padding/bank-conflict
//    post and the storage_align answer): instead of padding rows, the
//    16-byte chunk index of every row is XOR-ed with a function of the row,
//    chosen so that the 64 lanes of each fragment read hit distinct banks
//    on gfx950's LDS; no LDS is spent on padding.
//  * Vectorised fragment loads (Step 4): one ds_read_b128 per lane per
//    fragment for k-contiguous operands; for operands stored n-contiguous
//    (row-major B) the gfx950 transpose reads ds_read_b64_tr_b16/_b8 build
//    the k-contiguous fragment directly from the [k][n] LDS tile.
//  * Software pipelining (Step 5): NST LDS stages (two for data-parallel
//    kernels, up to four for Stream-K); the copies of K-steps k+1 ..
//    k+NST-1 are in flight while the MFMAs of step k run.  The eight-wave
//    kernel with an n-contiguous f16/bf16 B runs its two wave groups one
//    phase apart instead (ping-pong: one wave per SIMD reads fragments while
//    the other issues MFMAs).
//  * Unrolled inner loop of matrix-core ops (Step 6; Tensor Core notes on
//    je-d.tistory.com: mixed-precision multiply-accumulate per warp-level
//    operation): v_mfma_f32_32x32x16_{f16,bf16}, v_mfma_i32_32x32x32_i8,
//    v_mfma_f32_32x32x2_f32, fully unrolled over the K-step.
//  * Bias as the reduction's initial value, ReLU before the store
//    (FuseReductionEpilogue posts; Conv2d + Bias + ReLU fusion post).
//  * Stream-K (leiblog.wang, Stream-K reproduction post): the k-iterations
//    of the split tiles are divided evenly over a persistent grid; a tile
//    cut between workgroups is finished by whichever of them arrives last,
//    summing the partial tiles in workgroup order (deterministic result).
#pragma once
#include <hip/hip_runtime.h>

#include "tcm_internal.h"

namespace tcm {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef int i16v_t __attribute__((ext_vector_type(16)));
typedef int i4_t __attribute__((ext_vector_type(4)));
typedef int i2_t __attribute__((ext_vector_type(2)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;

// Offset that lies beyond every buffer descriptor's range: loads through it
// return zeros (used for rows/columns/k beyond the matrix).
constexpr unsigned kOOB = 0x40000000u;
// gfx9 buffer descriptor word 3 for raw (untyped, unswizzled) dword access.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)kOOB, kRsrcWord3);
}

// XOR swizzles of the 16-byte chunk index (see the header comment).
// k-contiguous rows of 128 bytes (8 chunks), read as 32x32 fragments: rows
// r..r+31 at one chunk column; measured conflict-free on gfx950.
__device__ __forceinline__ int swz_k(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int DT>
struct Elem;
template <>
struct Elem<F16> {
    static constexpr int bytes = 2;
};
template <>
struct Elem<BF16> {
    static constexpr int bytes = 2;
};
template <>
struct Elem<F32> {
    static constexpr int bytes = 4;
};
template <>
struct Elem<I8> {
    static constexpr int bytes = 1;
};

// n-contiguous [k][n] tiles (row-major B): swizzle as a function of the k row,
// so the rows that one transpose read touches land on distinct banks.  The
// choice depends on CPR (chunks per k row): with few chunks per row the rows
// of one read wrap onto the same banks sooner, so narrow tiles use a coarser
// pattern.  Each case was checked lane by lane against the 64-bank model
// (half a wave per pass, 8 bytes per lane) for every read the tile issues.
template <int DT, int CPR>
__device__ __forceinline__ int swz_mn(int k) {
    int s;
    if constexpr (DT == I8) {  // 8 rows x 16 B per 16-lane group
        if constexpr (CPR == 4) s = 2 * ((k >> 2) & 1);
        else if constexpr (CPR == 8) s = 2 * ((k >> 1) & 3);
        else s = 2 * (k & 7);
    } else if constexpr (DT == F32) {  // two k rows per wave read
        s = 8 * ((k >> 2) & 1);
    } else {  // 4 rows x 32 B per 16-lane group
        if constexpr (CPR == 8) s = 4 * ((k >> 1) & 1);
        else s = 4 * (k & 3);
    }
    return s & (CPR - 1);
}

// A_MMAJ: A stored column-major (m contiguous), staged as [k][m] tiles and
// read with the transposing fragment reads of an n-contiguous B.
template <int DT, int CFG, bool B_KMAJ, bool CONV = false, int NST = 2, bool A_MMAJ = false>
struct TileKernel {
    static constexpr TileConfig cfg = kConfigs[CFG];
    static constexpr int BM = cfg.bm, BN = cfg.bn, WM = cfg.wm, WN = cfg.wn;
    static constexpr int NW = WM * WN, NT = NW * 64;
    static constexpr int ES = Elem<DT>::bytes;
    static constexpr int CE = kChunkBytes / ES;      // elements per 16-byte chunk
    static constexpr int BKE = kStepBytes / ES;      // elements per K-step
    static constexpr int TM = BM / WM, TN = BN / WN; // wave tile
    static constexpr int FM = TM / 32, FN = TN / 32; // 32x32 MFMA tiles per wave
    static constexpr int A_BYTES = BM * kStepBytes, B_BYTES = BN * kStepBytes;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = NST * STAGE;  // NST stages, copies NST - 1 K-steps ahead of the MFMAs
    // Copier waves.  In the eight-wave GEMM kernel waves 0-3 issue every
    // copy and waves 4-7 none: waves go to the four SIMDs round-robin, so
    // each SIMD pairs one copier with a wave that only feeds the matrix
    // core while the copier's copies queue (8192^3 f16: 2% faster than all
    // eight waves interleaving copies with their MFMAs).  The ping-pong loop
    // splits the copies by operand between the two groups instead.
    static constexpr int NWC = (NW == 8 && !CONV) ? NW / 2 : NW;
    static constexpr int IA = BM / (8 * NWC);        // DMA instructions per copier wave per stage (A)
    static constexpr int IB = BN / (8 * NWC);        // (B)
    static constexpr int B_CPR = BN * ES / kChunkBytes;  // chunks per [k] row of an n-contiguous B tile
    static constexpr int A_CPR = BM * ES / kChunkBytes;  // chunks per [k] row of an m-contiguous A tile
    static_assert((B_CPR & (B_CPR - 1)) == 0, "chunk count per row must be a power of two");
    static_assert(!A_MMAJ || ((A_CPR & (A_CPR - 1)) == 0 && A_CPR >= 4 && A_CPR <= 64 && !CONV),
                  "m-contiguous A: a power-of-two chunk count per row, 4 to 64");
    static_assert(BM % (8 * NWC) == 0 && BN % (8 * NWC) == 0, "tile rows must fill whole wave DMA instructions");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32x32");
    static_assert(LDS <= 160 * 1024, "LDS budget of one CU");
    static_assert(NST >= 2 && (NST - 1) * (BM + BN) / (8 * NWC) <= 63, "pipeline depth within the vmcnt range");

    using Acc = typename std::conditional<DT == I8, i16v_t, f16v_t>::type;
    using AccS = typename std::conditional<DT == I8, int, float>::type;

    // ---------------------------------------------------------------- DMA
    // Lane `lane` of copier wave `wave` fills LDS chunk slot p = (j*NWC + wave)*64 + lane
    // with its j-th copy instruction of a stage (one wave instruction fills
    // 1 KiB of consecutive LDS).  The chunk column of a slot depends on j only
    // through j's parity and its row advances by ADV rows every two
    // instructions, so a lane keeps two offsets per operand and adds a
    // uniform stride.  Rows outside the matrix (m >= M, n >= N for
    // k-contiguous operands; k >= K for m/n-contiguous ones) lie past the end
    // of the step's buffer range and read as zeros; rows m >= M of an
    // m-contiguous A and columns n >= N of an n-contiguous B are folded into
    // the offsets; the k tail of k-contiguous operands is one select per
    // parity.
    static constexpr int A_RPI = A_MMAJ ? 64 / A_CPR : 8;  // rows per instruction of the A tile
    static constexpr int B_RPI = B_KMAJ ? 8 : 64 / B_CPR;  // rows per instruction of the B tile
    static constexpr int A_ADV = 2 * NWC * A_RPI;
    static constexpr int B_ADV = 2 * NWC * B_RPI;

    struct Dma {
        unsigned a_off[2];
        int a_k[2];
        unsigned b_off[2];
        int b_k[2];
        // convolution: per A copy instruction, this lane's output pixel as the
        // element offset of its input origin (image n, row h0, column w0) and
        // h0, w0 themselves (h0 far below zero for rows past M)
        int cv_pix[CONV ? IA : 1], cv_h0[CONV ? IA : 1], cv_w0[CONV ? IA : 1];
    };

    __device__ __forceinline__ static void dma_setup(Dma& d, const TileArgs& a, int m0, int n0, int wave, int lane) {
        if constexpr (CONV) {
            const int pq = a.cv_P * a.cv_Q;
#pragma unroll
            for (int j = 0; j < IA; ++j) {
                const int m = m0 + (((j * NWC + wave) * 64 + lane) >> 3);
                const int mm = m < a.M ? m : a.M - 1;  // rows past M: any real pixel, masked below
                const int n = mm / pq, rem = mm - n * pq, p = rem / a.cv_Q, q = rem - p * a.cv_Q;
                const int h0 = p * a.cv_stride_h - a.cv_pad_h, w0 = q * a.cv_stride_w - a.cv_pad_w;
                d.cv_h0[j] = m < a.M ? h0 : -(1 << 28);
                d.cv_w0[j] = w0;
                d.cv_pix[j] = ((n * a.cv_H + h0) * a.cv_W + w0) * a.cv_C;
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int p = (q * NWC + wave) * 64 + lane;
            if constexpr (A_MMAJ) {
                const int kr = p / A_CPR, c = (p % A_CPR) ^ swz_mn<DT, A_CPR>(kr);
                d.a_off[q] = m0 + c * CE < a.M ? (unsigned)(kr * a.lda + c * CE) * ES : kOOB;
                d.a_k[q] = 0;
            } else {
                const int r = p >> 3, c = (p & 7) ^ swz_k(r);
                d.a_off[q] = (unsigned)(r * a.lda + c * CE) * ES;
                d.a_k[q] = c * CE;
            }
            if constexpr (B_KMAJ) {
                const int r = p >> 3, c = (p & 7) ^ swz_k(r);
                d.b_off[q] = (unsigned)(r * a.ldb + c * CE) * ES;
                d.b_k[q] = c * CE;
            } else {
                const int kr = p / B_CPR, c = (p % B_CPR) ^ swz_mn<DT, B_CPR>(kr);
                d.b_off[q] = n0 + c * CE < a.N ? (unsigned)(kr * a.ldb + c * CE) * ES : kOOB;
                d.b_k[q] = 0;
            }
        }
    }

    __device__ __forceinline__ static int clamp_range(int64_t bytes) {
        return bytes <= 0 ? 0 : (bytes < (int64_t)kOOB ? (int)bytes : (int)kOOB);
    }

    // Issue the copies of K-step kt of tile (m0, n0) into LDS stage `st`:
    // those of operand A if OPS & 1, of operand B if OPS & 2.  With CHECK,
    // waves past the copier waves return at once; without it the caller
    // passes the copier slot (0 .. NWC-1) whose copies this wave issues.
    template <int OPS = 3, bool CHECK = true>
    __device__ __forceinline__ static void dma_issue(const Dma& d, const TileArgs& a, lds_char* smem, int st, int kt,
                                                     int m0, int n0, int wave) {
        if constexpr (NWC < NW && CHECK) {
            if (wave >= NWC) return;
        }
        const int k0 = kt * BKE;
        const int krem = a.K - k0;
        if constexpr (!(OPS & 1)) {
        } else if constexpr (CONV) {
            // this K-step's filter tap (r, s) and first channel: uniform
            const int rs = k0 / a.cv_C, c0 = k0 - rs * a.cv_C;
            const int rr = rs / a.cv_S, ss = rs - rr * a.cv_S;
            const int dh = rr * a.cv_dil_h, dw = ss * a.cv_dil_w;
            const int step = (dh * a.cv_W + dw) * a.cv_C + c0;
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.A), (short)0, a.cv_x_bytes, kRsrcWord3);
            lds_char* la = smem + st * STAGE;
#pragma unroll
            for (int j = 0; j < IA; ++j) {
                const int h = d.cv_h0[j] + dh, w = d.cv_w0[j] + dw;
                const bool in = (unsigned)h < (unsigned)a.cv_H && (unsigned)w < (unsigned)a.cv_W &&  // zero padding
                                d.a_k[j & 1] < krem;
                const unsigned off = in ? (unsigned)((d.cv_pix[j] + step + d.a_k[j & 1]) * ES) : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(la + (j * NWC + wave) * 1024),
                                                         16, off, 0, 0, 0);
            }
        } else {
            const char* base;
            int nrec;
            unsigned o0, o1;
            if constexpr (A_MMAJ) {
                base = (const char*)a.A + ((int64_t)k0 * a.lda + m0) * ES;
                nrec = clamp_range(((int64_t)krem * a.lda - m0) * ES);
                o0 = d.a_off[0];
                o1 = d.a_off[1];
            } else {
                base = (const char*)a.A + ((int64_t)m0 * a.lda + k0) * ES;
                nrec = clamp_range(((int64_t)(a.M - m0) * a.lda - k0) * ES);
                o0 = d.a_k[0] < krem ? d.a_off[0] : kOOB;
                o1 = d.a_k[1] < krem ? d.a_off[1] : kOOB;
            }
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, nrec, kRsrcWord3);
            const unsigned hop = (unsigned)(A_ADV * a.lda * ES);
            lds_char* la = smem + st * STAGE;
#pragma unroll
            for (int j = 0; j < IA; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(la + (j * NWC + wave) * 1024),
                                                         16, ((j & 1) ? o1 : o0) + (j >> 1) * hop, 0, 0, 0);
        }
        if constexpr ((OPS & 2) != 0) {
            const char* base;
            int nrec;
            unsigned o0, o1;
            if constexpr (B_KMAJ) {
                base = (const char*)a.B + ((int64_t)n0 * a.ldb + k0) * ES;
                nrec = clamp_range(((int64_t)(a.N - n0) * a.ldb - k0) * ES);
                o0 = d.b_k[0] < krem ? d.b_off[0] : kOOB;
                o1 = d.b_k[1] < krem ? d.b_off[1] : kOOB;
            } else {
                base = (const char*)a.B + ((int64_t)k0 * a.ldb + n0) * ES;
                nrec = clamp_range(((int64_t)krem * a.ldb - n0) * ES);
                o0 = d.b_off[0];
                o1 = d.b_off[1];
            }
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, nrec, kRsrcWord3);
            const unsigned hop = (unsigned)(B_ADV * a.ldb * ES);
            lds_char* lb = smem + st * STAGE + A_BYTES;
#pragma unroll
            for (int j = 0; j < IB; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lb + (j * NWC + wave) * 1024),
                                                         16, ((j & 1) ? o1 : o0) + (j >> 1) * hop, 0, 0, 0);
        }
    }

    // ------------------------------------------------------ fragment loads
    template <typename V>
    __device__ __forceinline__ static V lds_read16(const lds_char* p) {
        return *(const __attribute__((address_space(3))) V*)p;
    }

    // A fragment (k-contiguous): rows r..r+31 of the wave's block, chunk c.
    __device__ __forceinline__ static i4_t load_a(const lds_char* la, int row, int sub, int h) {
        int c = 2 * sub + h;
        return lds_read16<i4_t>(la + row * kStepBytes + ((c ^ swz_k(row)) << 4));
    }
    __device__ __forceinline__ static i4_t load_b_kmaj(const lds_char* lb, int row, int sub, int h) {
        int c = 2 * sub + h;
        return lds_read16<i4_t>(lb + row * kStepBytes + ((c ^ swz_k(row)) << 4));
    }
    // Fragment from an m- or n-contiguous [k][x] tile of RB bytes per k row
    // and CPR chunks (A column-major, B row-major): the lane's row or
    // column x (the MFMA's A and B operands share one lane layout) and the 8
    // (f16/bf16) or 16 (int8) k-values of chunk c = 2*sub + h.
    template <int RB, int CPR>
    __device__ __forceinline__ static i4_t load_mn(const lds_char* lb, int ncol0, int sub, int lane) {
        const int g = lane >> 4, t = lane & 15, h = g >> 1;
        const int c = 2 * sub + h;
        i4_t out;
        if constexpr (DT == I8) {
            const int n = ncol0 + 16 * (g & 1) + 8 * (t & 1);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int k = 16 * c + 8 * q + (t >> 1);
                const lds_char* p = lb + k * RB + (((n >> 4) ^ swz_mn<DT, CPR>(k)) << 4) + (n & 15);
                i2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i2_t*)p);
                out[2 * q] = v[0];
                out[2 * q + 1] = v[1];
            }
        } else {
            const int n = ncol0 + 16 * (g & 1) + 4 * (t & 3);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int k = 8 * c + 4 * q + (t >> 2);
                const lds_char* p = lb + k * RB + (((n >> 3) ^ swz_mn<DT, CPR>(k)) << 4) + ((n & 7) << 1);
                s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t*)p);
                i2_t w = __builtin_bit_cast(i2_t, v);
                out[2 * q] = w[0];
                out[2 * q + 1] = w[1];
            }
        }
        return out;
    }
    __device__ __forceinline__ static i4_t load_b_mn(const lds_char* lb, int ncol0, int sub, int lane) {
        return load_mn<BN * ES, B_CPR>(lb, ncol0, sub, lane);
    }
    // f32, m- or n-contiguous tile: single k-value e of chunk-substep sub.
    template <int RB, int CPR>
    __device__ __forceinline__ static float load_mn_f32(const lds_char* lb, int n, int sub, int h, int e) {
        const int k = 8 * sub + 4 * h + e;
        return *(const __attribute__((address_space(3))) float*)(lb + k * RB + (((n >> 2) ^ swz_mn<DT, CPR>(k)) << 4) + ((n & 3) << 2));
    }
    __device__ __forceinline__ static float load_b_mn_f32(const lds_char* lb, int n, int sub, int h, int e) {
        return load_mn_f32<BN * ES, B_CPR>(lb, n, sub, h, e);
    }
    // A fragment of 32 rows from row mrow0 of the wave's block, either layout
    __device__ __forceinline__ static i4_t load_a_any(const lds_char* la, int mrow0, int sub, int lane) {
        if constexpr (!A_MMAJ) {
            return load_a(la, mrow0 + (lane & 31), sub, lane >> 5);
        } else if constexpr (DT == F32) {
            f4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = load_mn_f32<BM * ES, A_CPR>(la, mrow0 + (lane & 31), sub, lane >> 5, e);
            return __builtin_bit_cast(i4_t, v);
        } else {
            return load_mn<BM * ES, A_CPR>(la, mrow0, sub, lane);
        }
    }

    // ------------------------------------------------------------- MFMA
    __device__ __forceinline__ static void mma(Acc& acc, i4_t a, i4_t b) {
        if constexpr (DT == F16)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), acc, 0, 0, 0);
        else if constexpr (DT == BF16)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), acc, 0, 0, 0);
        else if constexpr (DT == I8)
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc, 0, 0, 0);
    }
    __device__ __forceinline__ static void mma_f32(Acc& acc, float a, float b) {
        if constexpr (DT == F32) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }

    // Operand fragments of one sub-step (a quarter K-step): for every 32-row
    // block of the wave's A rows and 32-column block of its B columns, the
    // 16 bytes this lane feeds to the MFMA.
    struct Frag {
        i4_t a[FM];
        i4_t b[FN];
    };

    __device__ __forceinline__ static void load_frag(Frag& f, const lds_char* smem, int st, int sub, int wm, int wn, int lane) {
        const lds_char* la = smem + st * STAGE;
        const lds_char* lb = la + A_BYTES;
        const int h = lane >> 5, l32 = lane & 31;
        // issue order = first use by the MFMA sequence: a0, b0..b(FN-1), a1..a(FM-1)
        f.a[0] = load_a_any(la, wm * TM, sub, lane);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            if constexpr (B_KMAJ) {
                f.b[fn] = load_b_kmaj(lb, wn * TN + fn * 32 + l32, sub, h);
            } else if constexpr (DT == F32) {
                f4_t v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = load_b_mn_f32(lb, wn * TN + fn * 32 + l32, sub, h, e);
                f.b[fn] = __builtin_bit_cast(i4_t, v);
            } else {
                f.b[fn] = load_b_mn(lb, wn * TN + fn * 32, sub, lane);
            }
        }
#pragma unroll
        for (int fm = 1; fm < FM; ++fm) f.a[fm] = load_a_any(la, wm * TM + fm * 32, sub, lane);
    }

    __device__ __forceinline__ static void mma_frag(Acc (&acc)[FM][FN], const Frag& f) {
        if constexpr (DT == F32) {
            // Reinterpret whole vectors, then index: this compiler mis-folds
            // __builtin_bit_cast applied to a single vector element (it always
            // yields element 0).
            f4_t fa[FM], fb[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) fa[fm] = __builtin_bit_cast(f4_t, f.a[fm]);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) fb[fn] = __builtin_bit_cast(f4_t, f.b[fn]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) mma_f32(acc[fm][fn], fa[fm][e], fb[fn][e]);
        } else {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) mma(acc[fm][fn], f.a[fm], f.b[fn]);
        }
    }

    // ------------------------------------------------------- tile order
    // Tile t of the (batched) tile space: its coordinates within its entry and
    // the arguments with that entry's operand pointers (uniform per workgroup).
    // The tile at position n of the locality walk: its coordinates, and a copy
    // of the arguments whose operand pointers are its batch entry's.
    __device__ __forceinline__ static TileArgs tile_of(const TileArgs& a, int n, int& tm, int& tn) {
        TileArgs e = a;
        int b;
        tcm::walk_coords(n, a.tiles_m, a.tiles_n, a.group_m, a.super_m, a.super_n, &b, &tm, &tn);
        if (a.batch > 1) {
            e.A = (const char*)a.A + b * a.stride_a * ES;
            e.B = (const char*)a.B + b * a.stride_b * ES;
            e.C = (char*)a.C + b * a.stride_c * c_elem_bytes(a.c_type);
            if (a.bias) e.bias = (const char*)a.bias + b * a.stride_bias * (int64_t)sizeof(AccS);
        }
        return e;
    }

    // The tile at position n of a group's work list: the entry whose first
    // tile is the last at or before n (entries without tiles are left out
    // of the table), then that entry's own tile walk.  The table lives in
    // the kernel arguments: a scalar scan, unrolled so every index is static.
    __device__ __forceinline__ static TileArgs tile_of(const GroupArgs& g, int n, int& tm, int& tn) {
        TileArgs e = g.t;
        int tile0 = 0, sm = 1, sn = 1;
#pragma unroll
        for (int i = 0; i < kMaxGroup; ++i) {
            if (i < g.count && n >= g.e[i].tile0) {
                const GroupEntry& x = g.e[i];
                e.A = x.A;
                e.B = x.B;
                e.C = x.C;
                e.bias = x.bias;
                e.M = x.M;
                e.N = x.N;
                e.lda = x.lda;
                e.ldb = x.ldb;
                e.ldc = x.ldc;
                e.tiles_m = x.tiles_m;
                e.tiles_n = x.tiles_n;
                tile0 = x.tile0;
                sm = x.super_m;
                sn = x.super_n;
            }
        }
        tcm::super_order(n - tile0, e.tiles_m, e.tiles_n, g.t.group_m, sm, sn, &tm, &tn);
        return e;
    }
    __device__ __forceinline__ static const TileArgs& base_args(const TileArgs& a) { return a; }
    __device__ __forceinline__ static const TileArgs& base_args(const GroupArgs& g) { return g.t; }
    // tiles in the work list
    __device__ __forceinline__ static int work_tiles(const TileArgs& a) { return a.tiles_m * a.tiles_n * a.batch; }
    __device__ __forceinline__ static int work_tiles(const GroupArgs& g) { return g.t.dp_tiles + g.t.sk_tiles; }

    // ------------------------------------------------------- epilogue
    // 32x32 accumulator layout: lane l, register r holds row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32 of its MFMA tile.  C is read
    // (initial values) and written through a buffer descriptor whose range
    // ends at row M, with columns >= N given the out-of-range offset: such
    // loads return 0 and such stores are dropped, so there are no per-element
    // branches.  C holds the accumulator type, or f16 / bf16 (c_type).
    struct CView {
        __amdgpu_buffer_rsrc_t rc;
        unsigned coff[FN];  // per fn: byte offset of this lane's column in row 0 of the wave block (or kOOB)
        int row0;           // first row of the lane within the tile
        int cs;             // bytes per C element
    };
    __device__ __forceinline__ static CView c_view(const TileArgs& a, int m0, int n0, int wm, int wn, int lane) {
        CView v;
        v.cs = c_elem_bytes(a.c_type);
        v.row0 = wm * TM + 4 * (lane >> 5);
        const int mrem = a.M - m0;
        const int64_t bytes = ((int64_t)mrem * a.ldc - n0) * v.cs;  // from (m0, n0) to the end of row M-1's stride
        const int nrec = bytes < (int64_t)kOOB ? (int)bytes : (int)kOOB;
        v.rc = __builtin_amdgcn_make_buffer_rsrc((char*)a.C + ((int64_t)m0 * a.ldc + n0) * v.cs, (short)0, nrec, kRsrcWord3);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = wn * TN + fn * 32 + (lane & 31);
            v.coff[fn] = n0 + col < a.N ? (unsigned)((v.row0 * a.ldc + col) * v.cs) : kOOB;
        }
        return v;
    }
    __device__ __forceinline__ static unsigned c_roff(const TileArgs& a, const CView& v, int fm, int r) {
        return (unsigned)((fm * 32 + 8 * (r >> 2) + (r & 3)) * a.ldc * v.cs);
    }
    __device__ __forceinline__ static AccS load_c(const TileArgs& a, const CView& v, unsigned off) {
        if constexpr (DT == I8) {
            return __builtin_amdgcn_raw_buffer_load_b32(v.rc, off, 0, 0);
        } else {
            if (a.c_type == C_F16) {
                const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(v.rc, off, 0, 0);
                return (float)__builtin_bit_cast(_Float16, h);
            }
            if (a.c_type == C_BF16) {
                const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(v.rc, off, 0, 0);
                return __builtin_bit_cast(float, (unsigned)h << 16);
            }
            return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(v.rc, off, 0, 0));
        }
    }
    template <int CT>
    __device__ __forceinline__ static void store_c(const CView& v, unsigned off, AccS x) {
        if constexpr (DT == I8)
            __builtin_amdgcn_raw_buffer_store_b32(x, v.rc, off, 0, 0);
        else if constexpr (CT == C_F16)  // round to nearest even (the conversion's default mode)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (_Float16)x), v.rc, off, 0, 0);
        else if constexpr (CT == C_BF16)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)x), v.rc, off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), v.rc, off, 0, 0);
    }

    // Initial accumulator of a tile segment: with `seed` (the segment that
    // starts at k = 0), bias[col] plus, with accum, C's current value; else 0.
    // STAGED: a 16-bit C_in goes through LDS (data-parallel kernels; the
    // Stream-K kernels keep the direct loads, which cost them no registers)
    template <bool STAGED>
    __device__ __forceinline__ static void init_acc(Acc (&acc)[FM][FN], const TileArgs& a, lds_char* smem, bool seed, int m0,
                                                    int n0, int wm, int wn, int lane) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            AccS v = 0;
            if (seed && a.has_bias) {
                const int col = n0 + wn * TN + fn * 32 + (lane & 31);
                if (col < a.N) v = ((const AccS*)a.bias)[col];
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[fm][fn][r] = v;
        }
        if (seed && a.accum) {
            if constexpr (DT != I8 && STAGED) {
                if (a.c_type != C_ACC && (a.ldc & 7) == 0) {
                    add_c16_staged(acc, a, smem, m0, n0, wm, wn, lane);
                    return;
                }
            }
            const CView cv = c_view(a, m0, n0, wm, wn, lane);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const unsigned roff = c_roff(a, cv, fm, r);
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) acc[fm][fn][r] += load_c(a, cv, cv.coff[fn] + roff);
                }
        }
    }

    // C_in stored in 16 bits: 2-byte loads straight into the accumulator
    // layout cost 30 us of 133 on a 4096^3 bf16 product (32 MB of C), so the
    // tile is staged through LDS, which the main loop has not started to
    // use: 16-byte coalesced direct-to-LDS loads of C's rows (a row-major
    // BM x BN tile), then each lane reads its elements.  Rows past M read as
    // zeros (descriptor range); chunks past N are never used.  The main
    // loop's first barrier orders these reads before its copies.  With
    // Stream-K a segment that starts at k = 0 would need the same (C_in is
    // added once per tile), but there the extra code costs the 128x128
    // kernel register spills, so those kernels load C_in directly.
    __device__ __forceinline__ static void add_c16_staged(Acc (&acc)[FM][FN], const TileArgs& a, lds_char* smem, int m0,
                                                          int n0, int wm, int wn, int lane) {
        constexpr int ROWB = BN * 2;    // bytes of one staged row
        constexpr int CPRC = ROWB / 16; // 16-byte chunks per row
        constexpr int NI = BM * CPRC / NT;  // copy instructions per wave
        static_assert(BM * ROWB <= LDS && (BM * CPRC) % NT == 0, "a 16-bit C tile fills the LDS stages in whole wave copies");
        const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int64_t bytes = ((int64_t)(a.M - m0) * a.ldc - n0) * 2;
        const int nrec = bytes < (int64_t)kOOB ? (int)bytes : (int)kOOB;
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((char*)a.C + ((int64_t)m0 * a.ldc + n0) * 2, (short)0, nrec, kRsrcWord3);
        __syncthreads();  // a previous segment's readers are done with LDS
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int pslot = i * NT + tid, row = pslot / CPRC, c = pslot % CPRC;
            const unsigned off = n0 + c * 8 < a.N ? (unsigned)(row * a.ldc * 2 + c * 16) : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(smem + (i * NT + wave * 64) * 16), 16,
                                                     off, 0, 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const bool bf = a.c_type == C_BF16;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int row = wm * TM + fm * 32 + 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int col = wn * TN + fn * 32 + (lane & 31);
                    const unsigned short h = *(const __attribute__((address_space(3))) unsigned short*)(smem + row * ROWB + col * 2);
                    acc[fm][fn][rr] += bf ? __builtin_bit_cast(float, (unsigned)h << 16) : (float)__builtin_bit_cast(_Float16, h);
                }
            }
    }

    template <int CT>
    __device__ __forceinline__ static void store_tile_as(const Acc (&acc)[FM][FN], const TileArgs& a, int m0, int n0, int wm,
                                                         int wn, int lane) {
        const CView cv = c_view(a, m0, n0, wm, wn, lane);
        const bool relu = a.relu;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const unsigned roff = c_roff(a, cv, fm, r);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    AccS v = acc[fm][fn][r];
                    if (relu) v = v > (AccS)0 ? v : (AccS)0;
                    store_c<CT>(cv, cv.coff[fn] + roff, v);
                }
            }
    }
    // one branch per tile picks the store of C's type
    __device__ __forceinline__ static void store_tile(const Acc (&acc)[FM][FN], const TileArgs& a, int m0, int n0, int wm, int wn, int lane) {
        if constexpr (DT != I8) {
            if (a.c_type == C_F16) {
                store_tile_as<C_F16>(acc, a, m0, n0, wm, wn, lane);
                return;
            }
            if (a.c_type == C_BF16) {
                store_tile_as<C_BF16>(acc, a, m0, n0, wm, wn, lane);
                return;
            }
        }
        store_tile_as<C_ACC>(acc, a, m0, n0, wm, wn, lane);
    }

    // Partial tiles live in the workspace in register order, four
    // accumulator registers (rows 8q..8q+3 of a 32x32 MFMA tile, one column)
    // per 16-byte lane vector: element (wave, fm, fn, q, lane) -> 16 bytes.
    // They cross XCDs (each has its own L2), so they are written and read
    // with the device-coherent cache policy (sc1) instead of whole-cache
    // write-back / invalidate fences.  Quads whose rows all lie at or past M
    // are neither written nor read (out-of-range offset).
    static constexpr int kCoherent = 16;  // buffer-op cache policy: sc1
    __device__ __forceinline__ static __amdgpu_buffer_rsrc_t partial_rsrc(const TileArgs& a, int slot) {
        char* base = (char*)a.ws_partial + (int64_t)slot * BM * BN * 4;
        return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, BM * BN * 4, kRsrcWord3);
    }
    __device__ __forceinline__ static unsigned partial_off(int wave, int fm, int fn, int q, int lane, int wm, int mrem) {
        const int row = wm * TM + fm * 32 + 8 * q + 4 * (lane >> 5);
        return row < mrem ? (unsigned)(((((wave * FM + fm) * FN + fn) * 4 + q) * 64 + lane) * 16) : kOOB;
    }
    __device__ __forceinline__ static void store_partial(const Acc (&acc)[FM][FN], __amdgpu_buffer_rsrc_t r, int wave, int wm,
                                                         int lane, int mrem) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    i4_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = __builtin_bit_cast(int, (AccS)acc[fm][fn][4 * q + e]);
                    __builtin_amdgcn_raw_buffer_store_b128(v, r, partial_off(wave, fm, fn, q, lane, wm, mrem), 0, kCoherent);
                }
    }
    struct Partial {
        i4_t v[FM][FN][4];
    };
    __device__ __forceinline__ static void load_partial(Partial& pt, __amdgpu_buffer_rsrc_t r, int wave, int wm, int lane, int mrem) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    pt.v[fm][fn][q] = __builtin_amdgcn_raw_buffer_load_b128(r, partial_off(wave, fm, fn, q, lane, wm, mrem), 0, kCoherent);
    }
    __device__ __forceinline__ static void add_partial(Acc (&acc)[FM][FN], const Partial& pt, bool first) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (DT == I8) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[fm][fn][4 * q + e] = first ? pt.v[fm][fn][q][e] : acc[fm][fn][4 * q + e] + pt.v[fm][fn][q][e];
                    } else {
                        const f4_t fv = __builtin_bit_cast(f4_t, pt.v[fm][fn][q]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[fm][fn][4 * q + e] = first ? fv[e] : acc[fm][fn][4 * q + e] + fv[e];
                    }
                }
    }

    // ------------------------------------------------------- main loop
    // Interleave the next sub-step's 8 fragment reads with this sub-step's
    // 16 MFMAs (one read between each pair).
    static constexpr int NMF = FM * FN * (DT == F32 ? 4 : 1);              // MFMAs per sub-step
    static constexpr int NRD = FM * ((DT == F32 && A_MMAJ) ? 4 : (A_MMAJ ? 2 : 1)) +
                               FN * ((DT == F32 && !B_KMAJ) ? 4 : (B_KMAJ ? 1 : 2));  // LDS reads per sub-step
    __device__ __forceinline__ static void sched_reads() {
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
    // Last sub-step of a K-step: its MFMAs, the copies of step kt+NST and the
    // reads of the next step's first sub-step.  (Where only some waves copy,
    // the copies sit in a branch of their own and this interleaves nothing.)
    __device__ __forceinline__ static void sched_reads_dma() {
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < IA + IB) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            if (i < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }

    // Wait until at most `steps` K-steps of copies are still in flight (the
    // copies complete in issue order) and every LDS read has returned.
    template <int STEPS>
    __device__ __forceinline__ static void wait_copies() {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(STEPS * (IA + IB)) : "memory");
    }
    // The same for a count known at run time, 0 <= steps <= NST - 1 (the
    // tail of the loop and the prologue).
    __device__ __forceinline__ static void wait_copies(int steps) {
        if constexpr (NST - 1 >= 5) {
            if (steps >= 5) return wait_copies<5>();
        }
        if constexpr (NST - 1 >= 4) {
            if (steps >= 4) return wait_copies<4>();
        }
        if constexpr (NST - 1 >= 3) {
            if (steps >= 3) return wait_copies<3>();
        }
        if constexpr (NST - 1 >= 2) {
            if (steps >= 2) return wait_copies<2>();
        }
        if (steps >= 1) return wait_copies<1>();
        wait_copies<0>();
    }
    static_assert(NST <= 6, "wait_copies covers up to six stages");

    // One K-step kt from stage st, the copies of steps kt+1 .. kt+NST-1
    // issued earlier.  DMA: issue the copies of step kt+NST into stage st
    // once it is drained; NEXT: load sub-step 0 of step kt+1 (next stage).
    template <bool DMA, bool NEXT>
    __device__ __forceinline__ static void kstep(Acc (&acc)[FM][FN], Frag (&f)[2], const Dma& d, const TileArgs& a,
                                                 lds_char* smem, int st, int kt, int k_hi, int m0, int n0, int wave,
                                                 int wm, int wn, int lane) {
#pragma unroll
        for (int sub = 0; sub < 3; ++sub) {
            load_frag(f[(sub + 1) & 1], smem, st, sub + 1, wm, wn, lane);
            mma_frag(acc, f[sub & 1]);
            sched_reads();
        }
        // step kt+1 must have landed; the copies of later steps may still fly
        if constexpr (DMA) wait_copies<NST - 2>();
        else wait_copies(min(k_hi - kt - 2, NST - 2));
        __syncthreads();  // step kt+1 is in LDS everywhere; stage st is drained
        if constexpr (DMA) dma_issue(d, a, smem, st, kt + NST, m0, n0, wave);
        if constexpr (NEXT) load_frag(f[0], smem, st + 1 == NST ? 0 : st + 1, 0, wm, wn, lane);
        mma_frag(acc, f[1]);
        if constexpr (DMA) sched_reads_dma();
        else if constexpr (NEXT) sched_reads();
    }

    // ------------------------------------------------- ping-pong main loop
    // Eight-wave data-parallel kernel, n-contiguous B or m-contiguous A
    // (f16 / bf16): waves
    // 0-3 (group A) and 4-7 (group B) sit one of each per SIMD and run the
    // same loop one phase apart, phases separated by workgroup barriers.  In
    // a memory phase a wave reads all fragments of one K-step from LDS; in a
    // compute phase it issues that step's MFMAs.  While one wave of a SIMD
    // waits on LDS, its partner keeps the matrix core fed.  This pays where
    // fragment reads are many: the transpose reads of an n-contiguous B tile
    // return 8 bytes per lane, twice the LDS instructions of a k-contiguous
    // one (8192^3 f16: 915 against 1023 us), and so do those of an
    // m-contiguous A tile (A column-major, B column-major, 8192^3 f16: 938
    // against 1019 us).  With both operands k-contiguous the interleaved
    // loop below is faster (880 against 925 us), and on int8 the two are
    // even.
    //
    // Copies, two LDS stages.  Group A issues the A-operand copies of step
    // kt+1 in its memory phase of step kt.  Group B (copier slot wave-4)
    // issues the B-operand copies of step kt+2 at the start of its compute
    // phase of step kt, which runs beside group A's memory phase of step
    // kt+1; the stage they fill held step kt, which group B finished reading
    // in the phase before.  Each group waits for its own copies before the
    // barrier that precedes the first read of that step: A at the end of
    // its compute phase, B at the end of its memory phase.  One loop serves
    // both groups: two loops in the branches of a group test spill
    // registers.
    static constexpr bool PINGPONG = NW == 8 && !CONV && NST == 2 && (!B_KMAJ || A_MMAJ) && (DT == F16 || DT == BF16);

    // a workgroup barrier that nothing is scheduled across
    __device__ __forceinline__ static void phase_barrier() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }

    __device__ __forceinline__ static void mainloop_pp(Acc (&acc)[FM][FN], const TileArgs& a, lds_char* smem, int m0, int n0,
                                                       int k_lo, int k_hi, int wave, int lane) {
        static_assert(NWC * 2 == NW, "two groups of copier slots");
        const int wm = wave / WN, wn = wave % WN;
        const bool grp_a = wave < NWC;
        const int slot = grp_a ? wave : wave - NWC;
        Dma d;
        dma_setup(d, a, m0, n0, slot, lane);
        __syncthreads();  // the previous tile's readers are done with every stage
        if (k_lo >= k_hi) return;
        if (grp_a) {
            dma_issue<3, false>(d, a, smem, 0, k_lo, m0, n0, slot);
            wait_copies<0>();
        } else if (k_lo + 1 < k_hi) {
            dma_issue<2, false>(d, a, smem, 1, k_lo + 1, m0, n0, slot);
        }
        __syncthreads();  // step k_lo is in LDS
        if (!grp_a) phase_barrier();  // group B runs one phase behind
        int st = 0;
        for (int kt = k_lo; kt < k_hi; ++kt) {
            // memory phase
            Frag f[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) load_frag(f[s], smem, st, s, wm, wn, lane);
            if (grp_a && kt + 1 < k_hi) dma_issue<1, false>(d, a, smem, st ^ 1, kt + 1, m0, n0, slot);
            if (grp_a) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");  // B's copies of step kt+1
            phase_barrier();
            // compute phase
            if (!grp_a && kt + 2 < k_hi) dma_issue<2, false>(d, a, smem, st, kt + 2, m0, n0, slot);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) mma_frag(acc, f[s]);
            __builtin_amdgcn_sched_barrier(0);
            if (grp_a) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // A's copies of step kt+1
            phase_barrier();
            st ^= 1;
        }
        if (grp_a) phase_barrier();  // pairs with group B's extra barrier: equal counts
    }

    // Accumulate K-steps [k_lo, k_hi) of tile (m0, n0) into acc: NST LDS
    // stages, the copies running NST - 1 K-steps ahead of the MFMAs.
    __device__ __forceinline__ static void mainloop(Acc (&acc)[FM][FN], const TileArgs& a, lds_char* smem, int m0, int n0,
                                                    int k_lo, int k_hi, int wave, int lane) {
        if constexpr (PINGPONG) return mainloop_pp(acc, a, smem, m0, n0, k_lo, k_hi, wave, lane);
        const int wm = wave / WN, wn = wave % WN;
        Dma d;
        dma_setup(d, a, m0, n0, wave, lane);
        __syncthreads();  // the previous tile's readers are done with every stage
        if (k_lo >= k_hi) return;
        const int first = min(NST, k_hi - k_lo);  // steps copied before the loop
#pragma unroll
        for (int i = 0; i < NST; ++i)
            if (i < first) dma_issue(d, a, smem, i, k_lo + i, m0, n0, wave);
        wait_copies(first - 1);  // step k_lo has landed
        __syncthreads();
        Frag f[2];
        load_frag(f[0], smem, 0, 0, wm, wn, lane);
        int kt = k_lo, st = 0;
        for (; kt + NST < k_hi; ++kt) {
            kstep<true, true>(acc, f, d, a, smem, st, kt, k_hi, m0, n0, wave, wm, wn, lane);
            st = st + 1 == NST ? 0 : st + 1;
        }
        for (; kt + 1 < k_hi; ++kt) {
            kstep<false, true>(acc, f, d, a, smem, st, kt, k_hi, m0, n0, wave, wm, wn, lane);
            st = st + 1 == NST ? 0 : st + 1;
        }
        kstep<false, false>(acc, f, d, a, smem, st, kt, k_hi, m0, n0, wave, wm, wn, lane);
    }


    // Data-parallel kernel: workgroup b computes tile b (in L2-aware order).
    template <class Args>
    __device__ __forceinline__ static void run_dp(const Args& g) {
        __shared__ __attribute__((aligned(1024))) char smem_raw[LDS];
        lds_char* smem = (lds_char*)smem_raw;
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: DMA bases go to M0
        const int wm = wave / WN, wn = wave % WN;
        Acc acc[FM][FN];
        int tm, tn;
        const TileArgs e = tile_of(g, xcd_order(blockIdx.x, work_tiles(g)), tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        init_acc<true>(acc, e, smem, true, m0, n0, wm, wn, lane);
        mainloop(acc, e, smem, m0, n0, 0, e.iters, wave, lane);
        store_tile(acc, e, m0, n0, wm, wn, lane);
    }

    // Stream-K kernel: the k-iterations of tiles [dp_tiles, dp_tiles + sk_tiles)
    // are split evenly over the persistent grid; workgroup wg walks its share
    // [it0, it1) tile segment by tile segment.  The grid is never larger than
    // the number of iterations, so every workgroup owns at least one and the
    // workgroups holding a split tile are exactly its first owner .. last owner.
    template <class Args>
    __device__ __forceinline__ static void run_sk(const Args& g) {
        const TileArgs& a = base_args(g);
        __shared__ __attribute__((aligned(1024))) char smem_raw[LDS];
        __shared__ int s_flag;
        lds_char* smem = (lds_char*)smem_raw;
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / WN, wn = wave % WN;
        const int wg = blockIdx.x;
        Acc acc[FM][FN];
        const int64_t I = a.iters;
        const int64_t W = (int64_t)a.sk_tiles * I;
        const int64_t it0 = (int64_t)wg * W / a.grid, it1 = (int64_t)(wg + 1) * W / a.grid;
        const int64_t first_tile = it0 / I;
        for (int64_t it = it0; it < it1;) {
            const int64_t tsk = it / I;
            const int k_lo = (int)(it - tsk * I);
            const int k_hi = (int)min<int64_t>(I, k_lo + (it1 - it));
            int tm, tn;
            const TileArgs e = tile_of(g, xcd_order(a.dp_tiles + (int)tsk, work_tiles(g)), tm, tn);
            const int m0 = tm * BM, n0 = tn * BN;
            init_acc<false>(acc, e, smem, k_lo == 0, m0, n0, wm, wn, lane);
            mainloop(acc, e, smem, m0, n0, k_lo, k_hi, wave, lane);
            it += k_hi - k_lo;
            if (k_lo == 0 && k_hi == I) {
                store_tile(acc, e, m0, n0, wm, wn, lane);
                continue;
            }
            // Split tile: publish this segment (every wave waits until its
            // partial stores are acknowledged), then count the arrival.
            const int slot = 2 * wg + (tsk == first_tile ? 0 : 1);
            store_partial(acc, partial_rsrc(a, slot), wave, wm, lane, e.M - m0);
            if (a.sk_fixup_kernel) continue;  // the fix-up kernel sums this tile after the grid ends
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            // workgroups holding a segment of tile tsk: owners of its first and last iteration
            const int64_t x0 = tsk * I, x1 = tsk * I + I - 1;
            const int w_first = (int)(((x0 + 1) * a.grid + W - 1) / W - 1);
            const int w_last = (int)(((x1 + 1) * a.grid + W - 1) / W - 1);
            if (tid == 0) s_flag = __hip_atomic_fetch_add(a.ws_counter + tsk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const int arrived = s_flag;
            __syncthreads();  // s_flag is rewritten by the next split tile
            if (arrived != w_last - w_first) continue;  // not the last arrival
            // Last arrival: sum every segment's partial in workgroup order,
            // the loads of partial w+1 in flight while partial w is added.
            // every owner after the first starts inside tile tsk (its first
            // tile, slot 0); the first owner used slot 1 if it started in an
            // earlier tile
            const int first_slot1 = ((int64_t)w_first * W / a.grid) < tsk * I ? 1 : 0;
            auto slot_of = [&](int w) { return 2 * w + (w == w_first ? first_slot1 : 0); };
            if constexpr (NW > 4 || FM * FN >= 4) {
                // one partial buffer: eight waves have no room for a second,
                // and for 64x64 wave tiles a second one would halve the
                // workgroups a CU holds
                for (int w = w_first; w <= w_last; ++w) {
                    Partial pw;
                    load_partial(pw, partial_rsrc(a, slot_of(w)), wave, wm, lane, e.M - m0);
                    add_partial(acc, pw, w == w_first);
                }
                store_tile(acc, e, m0, n0, wm, wn, lane);
                if (tid == 0) __hip_atomic_store(a.ws_counter + tsk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                continue;
            }
            if constexpr (NST > 2) {
                // deep-pipeline configs hold two workgroups per CU (LDS),
                // so their registers take four partials at once: a tile
                // split over many short segments waits for one round trip
                // per four partials
                constexpr int NB = 4;
                for (int w0 = w_first; w0 <= w_last; w0 += NB) {
                    Partial pb[NB];
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        if (w0 + j <= w_last) load_partial(pb[j], partial_rsrc(a, slot_of(w0 + j)), wave, wm, lane, e.M - m0);
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        if (w0 + j <= w_last) add_partial(acc, pb[j], w0 + j == w_first);
                }
                store_tile(acc, e, m0, n0, wm, wn, lane);
                if (tid == 0) __hip_atomic_store(a.ws_counter + tsk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                continue;
            }
            // (unrolled by two so both buffers stay in registers)
            Partial p0, p1;
            load_partial(p0, partial_rsrc(a, slot_of(w_first)), wave, wm, lane, e.M - m0);
            for (int w = w_first; w <= w_last; w += 2) {
                if (w + 1 <= w_last) load_partial(p1, partial_rsrc(a, slot_of(w + 1)), wave, wm, lane, e.M - m0);
                add_partial(acc, p0, w == w_first);
                if (w + 1 > w_last) break;
                if (w + 2 <= w_last) load_partial(p0, partial_rsrc(a, slot_of(w + 2)), wave, wm, lane, e.M - m0);
                add_partial(acc, p1, false);
            }
            store_tile(acc, e, m0, n0, wm, wn, lane);
            if (tid == 0) __hip_atomic_store(a.ws_counter + tsk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // Fix-up kernel of a Stream-K launch whose split tiles are summed after
    // the grid ends (sk_fixup_kernel): workgroup b finishes Stream-K tile b
    // if it was split, adding the partials of its segments in workgroup
    // order as the last arrival would, so both ways give the same bits.
    // The kernel boundary makes every partial visible: no segment waits for
    // its stores or counts its arrival.
    template <class Args>
    __device__ __forceinline__ static void run_fixup(const Args& g) {
        const TileArgs& a = base_args(g);
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / WN, wn = wave % WN;
        const int64_t I = a.iters;
        const int64_t W = (int64_t)a.sk_tiles * I;
        const int64_t tsk = blockIdx.x;
        const int64_t x0 = tsk * I, x1 = tsk * I + I - 1;
        const int w_first = (int)(((x0 + 1) * a.grid + W - 1) / W - 1);
        const int w_last = (int)(((x1 + 1) * a.grid + W - 1) / W - 1);
        if (w_first == w_last) return;  // one workgroup held the whole tile and stored it
        int tm, tn;
        const TileArgs e = tile_of(g, xcd_order(a.dp_tiles + (int)tsk, work_tiles(g)), tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int first_slot1 = ((int64_t)w_first * W / a.grid) < x0 ? 1 : 0;
        // partials in flight at once: about 128 registers' worth
        constexpr int NB = FM * FN >= 8 ? 1 : 8 / (FM * FN);
        Acc acc[FM][FN];
        for (int w0 = w_first; w0 <= w_last; w0 += NB) {
            Partial pb[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j)
                if (w0 + j <= w_last)
                    load_partial(pb[j], partial_rsrc(a, 2 * (w0 + j) + (w0 + j == w_first ? first_slot1 : 0)), wave, wm, lane,
                                 e.M - m0);
#pragma unroll
            for (int j = 0; j < NB; ++j)
                if (w0 + j <= w_last) add_partial(acc, pb[j], w0 + j == w_first);
        }
        store_tile(acc, e, m0, n0, wm, wn, lane);
    }

    // Equal shares (a.split = S > 1): the k-iterations of each of the T
    // tiles are cut into S ranges [s*I/S, (s+1)*I/S), one per workgroup, and
    // each range runs on the data-parallel loop (the Stream-K split of the
    // whole work evenly over the grid, aligned to whole shares of tiles).
    // Workgroup ids are renumbered by XCD over the T*S (share, tile) pairs,
    // shares outermost: an XCD runs neighbouring tiles' same share, whose
    // operand panels sit at the same k and stream through its L2 together.
    // Share 0 carries the initial value (bias, C_in); every share stores its
    // partial tile at slot s*T + t.
    template <class Args>
    __device__ __forceinline__ static void run_split(const Args& g) {
        const TileArgs& a = base_args(g);
        __shared__ __attribute__((aligned(1024))) char smem_raw[LDS];
        lds_char* smem = (lds_char*)smem_raw;
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / WN, wn = wave % WN;
        const int T = a.sk_tiles, S = a.split;
        const int n = xcd_order(blockIdx.x, T * S);
        const int s = n / T, t = n - s * T;
        Acc acc[FM][FN];
        int tm, tn;
        const TileArgs e = tile_of(g, t, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int k_lo = (int)((int64_t)s * e.iters / S), k_hi = (int)((int64_t)(s + 1) * e.iters / S);
        init_acc<true>(acc, e, smem, s == 0, m0, n0, wm, wn, lane);
        mainloop(acc, e, smem, m0, n0, k_lo, k_hi, wave, lane);
        store_partial(acc, partial_rsrc(a, s * T + t), wave, wm, lane, e.M - m0);
    }

    // Sum of an equal-shares launch: one wave per 32x32 accumulator block of
    // a tile (workgroup b: tile b / (NW*FM*FN), then wave slot, fm, fn).  It
    // issues the loads of all S partials of its block at once (one memory
    // round trip), adds them in share order and stores the block with the
    // epilogue.  (One workgroup per tile, as the Stream-K fix-up has, waits
    // on a round trip per share with a few hundred kilobytes in flight.)
    __device__ __forceinline__ static void run_split_fixup(const TileArgs& a) {
        const int lane = threadIdx.x;
        const int T = a.sk_tiles, S = a.split;
        int b = blockIdx.x;
        const int fn = b % FN;
        b /= FN;
        const int fm = b % FM;
        b /= FM;
        const int wave = b % NW, t = b / NW;
        const int wm = wave / WN, wn = wave % WN;
        int tm, tn;
        const TileArgs e = tile_of(a, t, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN, mrem = e.M - m0;
        i4_t p[kMaxSplit][4];
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s)
            if (s < S) {
                const __amdgpu_buffer_rsrc_t r = partial_rsrc(a, s * T + t);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    p[s][q] = __builtin_amdgcn_raw_buffer_load_b128(r, partial_off(wave, fm, fn, q, lane, wm, mrem), 0, kCoherent);
            }
        Acc acc = {};
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s)
            if (s < S) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (DT == I8) {
#pragma unroll
                        for (int x = 0; x < 4; ++x) acc[4 * q + x] = s == 0 ? p[s][q][x] : acc[4 * q + x] + p[s][q][x];
                    } else {
                        const f4_t fv = __builtin_bit_cast(f4_t, p[s][q]);
#pragma unroll
                        for (int x = 0; x < 4; ++x) acc[4 * q + x] = s == 0 ? fv[x] : acc[4 * q + x] + fv[x];
                    }
                }
            }
        const CView cv = c_view(e, m0, n0, wm, wn, lane);
        unsigned coff = kOOB;  // this lane's column offset in block column fn (a select, not an indexed register array)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            if (j == fn) coff = cv.coff[j];
        if constexpr (DT != I8) {
            if (e.c_type == C_F16) return store_block<C_F16>(acc, e, cv, coff, fm);
            if (e.c_type == C_BF16) return store_block<C_BF16>(acc, e, cv, coff, fm);
        }
        store_block<C_ACC>(acc, e, cv, coff, fm);
    }
    // one 32x32 accumulator block (rows of fragment fm, the lane's column at coff), with ReLU
    template <int CT>
    __device__ __forceinline__ static void store_block(const Acc& acc, const TileArgs& a, const CView& cv, unsigned coff, int fm) {
        const bool relu = a.relu;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            AccS v = acc[r];
            if (relu) v = v > (AccS)0 ? v : (AccS)0;
            store_c<CT>(cv, coff + c_roff(a, cv, fm, r), v);
        }
    }
};

template <int CFG>
struct TileThreads {
    static constexpr int value = kConfigs[CFG].wm * kConfigs[CFG].wn * 64;
};

// Waves per SIMD the compiler must leave room for: the Stream-K kernel of
// the four-wave 128x128 config is held to two, so a CU runs two of its
// workgroups as it does the data-parallel one (left alone, the fix-up path
// takes it past 256 registers).  The other kernels fit their occupancy by
// themselves.
template <int CFG, bool SK>
struct TileWaves {
    static constexpr int value =
        (SK && kConfigs[CFG].wm * kConfigs[CFG].wn == 4 && kConfigs[CFG].bm == 128 && kConfigs[CFG].bn == 128) ? 2 : 1;
};

template <int DT, int CFG, bool B_KMAJ, bool SK>
__global__ __launch_bounds__(TileThreads<CFG>::value) __attribute__((amdgpu_waves_per_eu(TileWaves<CFG, SK>::value)))
void tile_gemm_kernel(TileArgs a) {
    if constexpr (SK) TileKernel<DT, CFG, B_KMAJ, false, kConfigs[CFG].sk_stages>::run_sk(a);
    else TileKernel<DT, CFG, B_KMAJ>::run_dp(a);
}

// One call = up to two launches on the stream: the data-parallel tiles
// [0, dp_tiles) with one workgroup each, then the Stream-K tiles on the
// persistent grid.
template <int DT, int CFG, bool B_KMAJ>
int sk_occupancy() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, tile_gemm_kernel<DT, CFG, B_KMAJ, true>, TileThreads<CFG>::value, 0) !=
        hipSuccess)
        return 0;
    return n;
}

// Sums the split tiles of a Stream-K launch (one workgroup per Stream-K tile).
template <int DT, int CFG, bool B_KMAJ>
__global__ __launch_bounds__(TileThreads<CFG>::value) void tile_fixup_kernel(TileArgs a) {
    TileKernel<DT, CFG, B_KMAJ, false, kConfigs[CFG].sk_stages>::run_fixup(a);
}

// Equal shares (TileArgs::split > 1, the eight-wave config): the shares on
// the data-parallel loop, then the wave-per-block sum.
template <int DT, int CFG, bool B_KMAJ, bool A_MMAJ>
__global__ __launch_bounds__(TileThreads<CFG>::value) __attribute__((amdgpu_waves_per_eu(TileWaves<CFG, false>::value)))
void tile_split_kernel(TileArgs a) {
    TileKernel<DT, CFG, B_KMAJ, false, 2, A_MMAJ>::run_split(a);
}

// (the sum reads partial tiles and writes C: B's layout plays no part)
template <int DT, int CFG>
__global__ __launch_bounds__(64) void tile_split_fixup_kernel(TileArgs a) {
    TileKernel<DT, CFG, true>::run_split_fixup(a);
}

// Launches an equal-shares plan; returns -1 if this config has no such
// kernels (the planner gives equal shares to the eight-wave config only).
template <int DT, int CFG, bool B_KMAJ, bool A_MMAJ>
int launch_split(const TileArgs& a, hipStream_t s) {
    if constexpr (split_config(CFG)) {
        using K = TileKernel<DT, CFG, true>;
        hipLaunchKernelGGL((tile_split_kernel<DT, CFG, B_KMAJ, A_MMAJ>), dim3(a.sk_tiles * a.split), dim3(TileThreads<CFG>::value),
                           0, s, a);
        hipLaunchKernelGGL((tile_split_fixup_kernel<DT, CFG>), dim3(a.sk_tiles * K::NW * K::FM * K::FN), dim3(64), 0, s, a);
        return (int)hipGetLastError();
    } else {
        return -1;
    }
}

template <int DT, int CFG, bool B_KMAJ>
int launch_tile(const TileArgs& a, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (a.split > 1) return launch_split<DT, CFG, B_KMAJ, false>(a, s);
    if (a.dp_tiles > 0)
        hipLaunchKernelGGL((tile_gemm_kernel<DT, CFG, B_KMAJ, false>), dim3(a.dp_tiles), dim3(TileThreads<CFG>::value), 0, s, a);
    if (a.sk_tiles > 0)
        hipLaunchKernelGGL((tile_gemm_kernel<DT, CFG, B_KMAJ, true>), dim3(a.grid), dim3(TileThreads<CFG>::value), 0, s, a);
    if (a.sk_tiles > 0 && a.sk_fixup_kernel)
        hipLaunchKernelGGL((tile_fixup_kernel<DT, CFG, B_KMAJ>), dim3(a.sk_tiles), dim3(TileThreads<CFG>::value), 0, s, a);
    return (int)hipGetLastError();
}

// Column-major A (m contiguous): the same kernels with A staged as [k][m]
// tiles.  Split tiles are summed by tile_fixup_kernel, which reads only the
// partials.
template <int DT, int CFG, bool B_KMAJ, bool SK>
__global__ __launch_bounds__(TileThreads<CFG>::value) __attribute__((amdgpu_waves_per_eu(TileWaves<CFG, SK>::value)))
void tile_gemm_acol_kernel(TileArgs a) {
    if constexpr (SK) TileKernel<DT, CFG, B_KMAJ, false, kConfigs[CFG].sk_stages, true>::run_sk(a);
    else TileKernel<DT, CFG, B_KMAJ, false, 2, true>::run_dp(a);
}

template <int DT, int CFG, bool B_KMAJ>
int launch_tile_acol(const TileArgs& a, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (a.split > 1) return launch_split<DT, CFG, B_KMAJ, true>(a, s);
    if (a.dp_tiles > 0)
        hipLaunchKernelGGL((tile_gemm_acol_kernel<DT, CFG, B_KMAJ, false>), dim3(a.dp_tiles), dim3(TileThreads<CFG>::value), 0, s,
                           a);
    if (a.sk_tiles > 0)
        hipLaunchKernelGGL((tile_gemm_acol_kernel<DT, CFG, B_KMAJ, true>), dim3(a.grid), dim3(TileThreads<CFG>::value), 0, s, a);
    if (a.sk_tiles > 0 && a.sk_fixup_kernel)
        hipLaunchKernelGGL((tile_fixup_kernel<DT, CFG, B_KMAJ>), dim3(a.sk_tiles), dim3(TileThreads<CFG>::value), 0, s, a);
    return (int)hipGetLastError();
}

// A group of products on one work list (the tiles of each entry in turn).
template <int DT, int CFG, bool B_KMAJ, bool SK>
__global__ __launch_bounds__(TileThreads<CFG>::value) __attribute__((amdgpu_waves_per_eu(TileWaves<CFG, SK>::value)))
void tile_group_kernel(GroupArgs g) {
    if constexpr (SK) TileKernel<DT, CFG, B_KMAJ, false, kConfigs[CFG].sk_stages>::run_sk(g);
    else TileKernel<DT, CFG, B_KMAJ>::run_dp(g);
}

template <int DT, int CFG, bool B_KMAJ>
__global__ __launch_bounds__(TileThreads<CFG>::value) void group_fixup_kernel(GroupArgs g) {
    TileKernel<DT, CFG, B_KMAJ, false, kConfigs[CFG].sk_stages>::run_fixup(g);
}

template <int DT, int CFG, bool B_KMAJ>
int launch_group(const GroupArgs& g, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (g.t.dp_tiles > 0)
        hipLaunchKernelGGL((tile_group_kernel<DT, CFG, B_KMAJ, false>), dim3(g.t.dp_tiles), dim3(TileThreads<CFG>::value), 0, s, g);
    if (g.t.sk_tiles > 0)
        hipLaunchKernelGGL((tile_group_kernel<DT, CFG, B_KMAJ, true>), dim3(g.t.grid), dim3(TileThreads<CFG>::value), 0, s, g);
    if (g.t.sk_tiles > 0 && g.t.sk_fixup_kernel)
        hipLaunchKernelGGL((group_fixup_kernel<DT, CFG, B_KMAJ>), dim3(g.t.sk_tiles), dim3(TileThreads<CFG>::value), 0, s, g);
    return (int)hipGetLastError();
}

// Implicit-GEMM convolution: the same kernel with the A copies gathering
// from the NHWC input; B is the KRSC filter (k-contiguous).
template <int DT, int CFG, bool SK>
__global__ __launch_bounds__(TileThreads<CFG>::value) __attribute__((amdgpu_waves_per_eu(TileWaves<CFG, SK>::value)))
void tile_conv_kernel(TileArgs a) {
    if constexpr (SK) TileKernel<DT, CFG, true, true, kConfigs[CFG].sk_stages>::run_sk(a);
    else TileKernel<DT, CFG, true, true>::run_dp(a);
}

template <int DT, int CFG>
__global__ __launch_bounds__(TileThreads<CFG>::value) void conv_fixup_kernel(TileArgs a) {
    TileKernel<DT, CFG, true, true, kConfigs[CFG].sk_stages>::run_fixup(a);
}

template <int DT, int CFG>
int launch_conv(const TileArgs& a, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (a.dp_tiles > 0)
        hipLaunchKernelGGL((tile_conv_kernel<DT, CFG, false>), dim3(a.dp_tiles), dim3(TileThreads<CFG>::value), 0, s, a);
    if (a.sk_tiles > 0)
        hipLaunchKernelGGL((tile_conv_kernel<DT, CFG, true>), dim3(a.grid), dim3(TileThreads<CFG>::value), 0, s, a);
    if (a.sk_tiles > 0 && a.sk_fixup_kernel)
        hipLaunchKernelGGL((conv_fixup_kernel<DT, CFG>), dim3(a.sk_tiles), dim3(TileThreads<CFG>::value), 0, s, a);
    return (int)hipGetLastError();
}

template <int DT, int CFG>
int conv_occupancy() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, tile_conv_kernel<DT, CFG, true>, TileThreads<CFG>::value, 0) !=
        hipSuccess)
        return 0;
    return n;
}

}  // namespace tcm
