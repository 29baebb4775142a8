// Generic GEMM kernel: any element alignment, any leading dimension, either
// layout of A and B; also the implicit-GEMM convolution for shapes the tiled
// gather does not take (channels not a multiple of the K-step, huge inputs).  It keeps the promise that a problem the fast path
// cannot take still gets the same result, only slower (je-d.tistory.com,
// the auto-tensorcore note: without the matrix-core rewrite the code is
// slower but functionally equal).  Pointers need no alignment at all: a
// call whose operand, C or bias pointer is not a multiple of its element
// size runs the byte-access instance, which reads and writes every element
// as single bytes.  Structure: 64x64 output tile per
// workgroup, four waves of 2x2 16x16 MFMA tiles, a 64-byte k-slab per step
// staged through LDS element by element with bounds checks, bias (plus C's
// current value with accum) as the accumulator's initial value, ReLU before
// the bounds-checked store in C's type (f32 / int32, or f16 / bf16 rounded
// to nearest even).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tcm_internal.h"

namespace tcm {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr int kSlab = 64;             // bytes of k per step
constexpr int kRow = kSlab + 16;      // LDS row pitch (bytes), keeps 16-byte alignment

template <int DT> struct G;
template <> struct G<F16> { using T = uint16_t; using Acc = f4_t; using AccS = float; };
template <> struct G<BF16> { using T = uint16_t; using Acc = f4_t; using AccS = float; };
template <> struct G<F32> { using T = float; using Acc = f4_t; using AccS = float; };
template <> struct G<I8> { using T = int8_t; using Acc = i4_t; using AccS = int; };

template <int DT>
__device__ __forceinline__ void mma16(typename G<DT>::Acc& acc, i4_t a, i4_t b) {
    if constexpr (DT == F16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a), __builtin_bit_cast(h8_t, b), acc, 0, 0, 0);
    else if constexpr (DT == BF16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), acc, 0, 0, 0);
    else if constexpr (DT == I8)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
    else {
        // reinterpret the whole vectors, then index (see the tiled kernel:
        // bit-casting one vector element is mis-folded to element 0)
        const f4_t af = __builtin_bit_cast(f4_t, a), bf = __builtin_bit_cast(f4_t, b);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[e], bf[e], acc, 0, 0, 0);
    }
}

// Element idx of an array of T at p.  BYTES: p may have any alignment, so
// the element is assembled from single-byte loads (stores likewise).
template <typename T, bool BYTES>
__device__ __forceinline__ T ld_elem(const void* p, int64_t idx) {
    if constexpr (BYTES && sizeof(T) > 1) {
        const unsigned char* b = (const unsigned char*)p + idx * (int64_t)sizeof(T);
        unsigned char v[sizeof(T)];
#pragma unroll
        for (int i = 0; i < (int)sizeof(T); ++i) v[i] = b[i];
        return __builtin_bit_cast(T, v);
    } else {
        return ((const T*)p)[idx];
    }
}
template <typename T, bool BYTES>
__device__ __forceinline__ void st_elem(void* p, int64_t idx, T x) {
    if constexpr (BYTES && sizeof(T) > 1) {
        unsigned char* b = (unsigned char*)p + idx * (int64_t)sizeof(T);
        const auto v = __builtin_bit_cast(unsigned char __attribute__((ext_vector_type(sizeof(T)))), x);
#pragma unroll
        for (int i = 0; i < (int)sizeof(T); ++i) b[i] = v[i];
    } else {
        ((T*)p)[idx] = x;
    }
}

// Copy the 64 x slab piece of one operand into LDS as [row][k] (k contiguous).
// rows index M (for A) or N (for B); `kmajor` says whether the operand is
// stored with k contiguous (then consecutive threads walk k).
template <int DT, bool BYTES>
__device__ __forceinline__ void stage(char* lds, const void* X, int64_t ld, bool kmajor, int64_t r0,
                                      int64_t rows, int64_t k0, int64_t K) {
    using T = typename G<DT>::T;
    constexpr int ES = sizeof(T);
    constexpr int BKE = kSlab / ES;
    for (int idx = threadIdx.x; idx < kTile * BKE; idx += 256) {
        int r, kk;
        if (kmajor) { r = idx / BKE; kk = idx % BKE; }
        else { kk = idx / kTile; r = idx % kTile; }
        const int64_t gr = r0 + r, gk = k0 + kk;
        T v = T(0);
        if (gr < rows && gk < K) v = ld_elem<T, BYTES>(X, kmajor ? gr * ld + gk : gk * ld + gr);
        *(T*)(lds + r * kRow + kk * ES) = v;
    }
}

// The same piece of A for a convolution: A is the im2col view of the NHWC
// input, row = output pixel (n, p, q), column = (r*S + s)*C + c; taps that
// fall in the zero padding read as zero.
template <int DT, bool BYTES>
__device__ __forceinline__ void stage_conv(char* lds, const void* X, const GenericArgs& a, int64_t r0,
                                           int64_t k0) {
    using T = typename G<DT>::T;
    constexpr int ES = sizeof(T);
    constexpr int BKE = kSlab / ES;
    for (int idx = threadIdx.x; idx < kTile * BKE; idx += 256) {
        const int r = idx / BKE, kk = idx % BKE;
        const int64_t gr = r0 + r, gk = k0 + kk;
        T v = T(0);
        if (gr < a.M && gk < a.K) {
            const int64_t pq = a.cv_P * a.cv_Q;
            const int64_t n = gr / pq, p = (gr % pq) / a.cv_Q, q = gr % a.cv_Q;
            const int64_t c = gk % a.cv_C, rs = gk / a.cv_C, fr = rs / a.cv_S, fs = rs % a.cv_S;
            const int64_t h = p * a.cv_stride_h - a.cv_pad_h + fr * a.cv_dil_h;
            const int64_t w = q * a.cv_stride_w - a.cv_pad_w + fs * a.cv_dil_w;
            if (h >= 0 && h < a.cv_H && w >= 0 && w < a.cv_W)
                v = ld_elem<T, BYTES>(X, ((n * a.cv_H + h) * a.cv_W + w) * a.cv_C + c);
        }
        *(T*)(lds + r * kRow + kk * ES) = v;
    }
}

// C element (row, col) as the accumulator type, and its store.
template <int DT, bool BYTES>
__device__ __forceinline__ typename G<DT>::AccS load_c(const GenericArgs& a, int64_t idx) {
    if constexpr (DT == I8) {
        return ld_elem<int, BYTES>(a.C, idx);
    } else {
        if (a.c_type == C_F16) return (float)ld_elem<_Float16, BYTES>(a.C, idx);
        if (a.c_type == C_BF16) return __builtin_bit_cast(float, (unsigned)ld_elem<uint16_t, BYTES>(a.C, idx) << 16);
        return ld_elem<float, BYTES>(a.C, idx);
    }
}
template <int DT, bool BYTES>
__device__ __forceinline__ void store_c(const GenericArgs& a, int64_t idx, typename G<DT>::AccS v) {
    if constexpr (DT == I8) {
        st_elem<int, BYTES>(a.C, idx, v);
    } else {
        if (a.c_type == C_F16) st_elem<_Float16, BYTES>(a.C, idx, (_Float16)v);
        else if (a.c_type == C_BF16) st_elem<__bf16, BYTES>(a.C, idx, (__bf16)v);
        else st_elem<float, BYTES>(a.C, idx, v);
    }
}

template <int DT, bool BYTES>
__global__ __launch_bounds__(256) void generic_gemm_kernel(GenericArgs a) {
    using T = typename G<DT>::T;
    using Acc = typename G<DT>::Acc;
    using AccS = typename G<DT>::AccS;
    constexpr int ES = sizeof(T);
    constexpr int BKE = kSlab / ES;
    __shared__ __attribute__((aligned(16))) char As[kTile * kRow];
    __shared__ __attribute__((aligned(16))) char Bs[kTile * kRow];

    // workgroup -> (entry of the batch, tile of that entry)
    const int per = a.tiles_m * a.tiles_n;
    const int bi = blockIdx.x / per, t = blockIdx.x - bi * per;
    a.A = (const T*)a.A + bi * a.stride_a;
    a.B = (const T*)a.B + bi * a.stride_b;
    a.C = (char*)a.C + bi * a.stride_c * c_elem_bytes(a.c_type);
    if (a.bias) a.bias = (const AccS*)a.bias + bi * a.stride_bias;
    const int tm = t / a.tiles_n, tn = t % a.tiles_n;
    const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r16 = lane & 15, grp = lane >> 4;

    Acc acc[2][2];
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
        AccS v = 0;
        const int64_t col = n0 + wn * 32 + fn * 16 + r16;
        if (a.has_bias && col < a.N) v = ld_elem<AccS, BYTES>(a.bias, col);
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[fm][fn][r] = v;
                const int64_t row = m0 + wm * 32 + fm * 16 + 4 * grp + r;
                if (a.accum && row < a.M && col < a.N) acc[fm][fn][r] += load_c<DT, BYTES>(a, row * a.ldc + col);
            }
    }

    for (int64_t k0 = 0; k0 < a.K; k0 += BKE) {
        if (a.conv) stage_conv<DT, BYTES>(As, a.A, a, m0, k0);
        else stage<DT, BYTES>(As, a.A, a.lda, !a.a_col, m0, a.M, k0, a.K);
        stage<DT, BYTES>(Bs, a.B, a.ldb, (bool)a.b_col, n0, a.N, k0, a.K);
        __syncthreads();
        i4_t af[2], bf[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            af[f] = *(const i4_t*)(As + (wm * 32 + f * 16 + r16) * kRow + grp * 16);
            bf[f] = *(const i4_t*)(Bs + (wn * 32 + f * 16 + r16) * kRow + grp * 16);
        }
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
            for (int fn = 0; fn < 2; ++fn) mma16<DT>(acc[fm][fn], af[fm], bf[fn]);
        __syncthreads();
    }

#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
            const int64_t col = n0 + wn * 32 + fn * 16 + r16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 32 + fm * 16 + 4 * grp + r;
                AccS v = acc[fm][fn][r];
                if (a.relu) v = v > (AccS)0 ? v : (AccS)0;
                if (row < a.M && col < a.N) store_c<DT, BYTES>(a, row * a.ldc + col, v);
            }
        }
}

__global__ void fill_zero_kernel(int* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

int launch_generic(int dtype, const GenericArgs& a, void* stream) {
    const int64_t blocks = (int64_t)a.tiles_m * a.tiles_n * a.batch;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)blocks), block(256);
    const bool bytes = a.bytewise != 0;
    switch (dtype) {
    case F16:
        if (bytes) hipLaunchKernelGGL((generic_gemm_kernel<F16, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((generic_gemm_kernel<F16, false>), grid, block, 0, s, a);
        break;
    case BF16:
        if (bytes) hipLaunchKernelGGL((generic_gemm_kernel<BF16, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((generic_gemm_kernel<BF16, false>), grid, block, 0, s, a);
        break;
    case F32:
        if (bytes) hipLaunchKernelGGL((generic_gemm_kernel<F32, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((generic_gemm_kernel<F32, false>), grid, block, 0, s, a);
        break;
    case I8:
        if (bytes) hipLaunchKernelGGL((generic_gemm_kernel<I8, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((generic_gemm_kernel<I8, false>), grid, block, 0, s, a);
        break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

int launch_fill_zero(int* p, int64_t n, void* stream) {
    if (n <= 0) return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, p, n);
    return (int)hipGetLastError();
}

}  // namespace tcm
