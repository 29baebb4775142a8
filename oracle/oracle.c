/*
 * oracle.c -- plain, slow CPU definition of the dense GEMM with a fused
 * bias/ReLU epilogue.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the CPU-baseline leg of the benchmark may call it; the product path
 * (the HIP library) never does, and this file shares no code, header, table
 * or helper with it.
 *
 * What it computes (one definition, written out):
 *
 *     C[i][j] = epi( c_in[i][j] + bias[j] + sum_{k=0}^{K-1} a(i,k) * b(k,j) )
 *
 *   - The problem statement is the matrix product with an added bias,
 *     Output = Input * Weight + Bias, from the FuseReductionEpilogue series
 *     (page "kimm240.github.io/tvm", post "1. Problem Analysis and Limitations
 *     of Existing Solutions").
 *   - The bias is the initial value of the reduction rather than a separate
 *     addition afterwards (same page, post "2. TIR Structure Transformation
 *     Design": reduction init = Bias instead of 0).  The oracle therefore
 *     starts every accumulator at bias[j] (or 0 without bias) and adds the
 *     products in ascending k.
 *   - The same post's generalisation, an arbitrary per-element tensor as the
 *     reduction's initial value, is the optional c_in: when given, the
 *     accumulator starts at c_in[i][j] + bias[j].  c_in is stored row-major
 *     with its own leading dimension, as f16, bf16 or f32 for the float
 *     types (cin_type 0, 1, 2) and as int32 for int8.
 *   - ReLU after the bias is the Conv2d + Bias + ReLU pattern (same page, post
 *     "Implement and enable Conv2d-Reshape-Add-ReLU fusion"); epi(x) is x, or
 *     x > 0 ? x : 0 with ReLU.
 *   - Low-precision inputs with a wide accumulator is the mixed-precision
 *     multiply-accumulate of the Tensor Core notes (page
 *     "je-d.tistory.com/entry/tvm", first section).  The oracle goes further
 *     than any GPU: f16, bf16 and f32 inputs are decoded to their exact values
 *     and accumulated in IEEE binary64; int8 inputs are accumulated as exact
 *     integers that must stay inside int32 (the GPU's accumulator), checked
 *     at every step.
 *
 * Operand storage (element offsets):
 *   a(i,k) = A[i*lda + k]     (a_col == 0, row-major)   or  A[k*lda + i]  (a_col == 1)
 *   b(k,j) = B[k*ldb + j]     (b_col == 0, row-major)   or  B[j*ldb + k]  (b_col == 1)
 *   C[i*ldc + j]  -- double for the float types, int32 for int8.
 *   c_in[i*ldcin + j]  -- optional; see above.
 *
 * Decoders are written from the IEEE 754 binary16 field layout (1 sign bit,
 * 5 exponent bits, bias 15, 10 fraction bits) and the bfloat16 layout (1 sign
 * bit, 8 exponent bits, bias 127, 7 fraction bits).  binary32 is read as the
 * host's float.
 *
 * The full entry point nests its loops i, k, j so that a row of C is built
 * while streaming rows of b; every C[i][j] still receives bias[j] first and
 * then the products in ascending k, one binary64 add each -- the same
 * operations in the same order as the per-entry entry point, which the tests
 * check bit-for-bit.
 *
 * Return codes: 0 = ok, 1 = invalid argument, 2 = an int8 sum left the int32
 * range (the result is then not what an int32 accumulator holds).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F16 = 0, OR_BF16 = 1, OR_F32 = 2, OR_I8 = 3 };

/* ---- exact decoders -------------------------------------------------- */

double oracle_decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)          /* zero / subnormal: frac * 2^(1-15-10) */
        v = ldexp((double)frac, -24);
    else if (expo == 0x1f)  /* infinity / NaN */
        v = frac ? NAN : INFINITY;
    else                    /* (1 + frac/2^10) * 2^(expo-15) */
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

double oracle_decode_bf16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 7) & 0xff;
    int frac = h & 0x7f;
    double v;
    if (expo == 0)          /* zero / subnormal: frac * 2^(1-127-7) */
        v = ldexp((double)frac, -133);
    else if (expo == 0xff)
        v = frac ? NAN : INFINITY;
    else                    /* (1 + frac/2^7) * 2^(expo-127) */
        v = ldexp((double)(128 + frac), expo - 134);
    return sign ? -v : v;
}

static double decode_f32(const float* p) { return (double)*p; }

/* value of element `idx` of a float-typed operand, exactly */
static double elem_f(const void* X, int dtype, int64_t idx) {
    switch (dtype) {
    case OR_F16:  return oracle_decode_f16(((const uint16_t*)X)[idx]);
    case OR_BF16: return oracle_decode_bf16(((const uint16_t*)X)[idx]);
    default:      return decode_f32((const float*)X + idx);
    }
}

static int64_t a_off(int64_t i, int64_t k, int64_t lda, int a_col) { return a_col ? k * lda + i : i * lda + k; }
static int64_t b_off(int64_t k, int64_t j, int64_t ldb, int b_col) { return b_col ? j * ldb + k : k * ldb + j; }

static double relu_f(double x) { return x > 0.0 ? x : 0.0; }

static int check_args(int64_t M, int64_t N, int64_t K, int64_t lda, int a_col, int64_t ldb, int b_col, int dtype) {
    if (M < 0 || N < 0 || K < 0) return 1;
    if (dtype < OR_F16 || dtype > OR_I8) return 1;
    if (lda < (a_col ? M : K) || lda < 1) return 1;
    if (ldb < (b_col ? K : N) || ldb < 1) return 1;
    return 0;
}

static int check_cin(const void* cin, int64_t ldcin, int cin_type, int64_t N, int dtype) {
    if (!cin) return 0;
    if (ldcin < N || ldcin < 1) return 1;
    if (dtype == OR_I8) return cin_type != OR_I8;  /* int32 storage */
    return cin_type < OR_F16 || cin_type > OR_F32;
}

/* initial value of C[i][j]: c_in (if any) plus bias (if any) */
static double init_f(const void* cin, int64_t ldcin, int cin_type, const float* bias, int64_t i, int64_t j) {
    double v = cin ? elem_f(cin, cin_type, i * ldcin + j) : 0.0;
    return bias ? v + (double)bias[j] : v;
}
static int64_t init_i(const int32_t* cin, int64_t ldcin, const int32_t* bias, int64_t i, int64_t j) {
    int64_t v = cin ? (int64_t)cin[i * ldcin + j] : 0;
    return bias ? v + bias[j] : v;
}

/* ---- decode a whole operand (used by tests to pin the decoders) -------- */

int oracle_decode(int dtype, const void* X, int64_t n, double* out) {
    if (dtype < OR_F16 || dtype > OR_I8) return 1;
    for (int64_t t = 0; t < n; ++t)
        out[t] = dtype == OR_I8 ? (double)((const int8_t*)X)[t] : elem_f(X, dtype, t);
    return 0;
}

/* ---- full product ------------------------------------------------------- */

int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda, int a_col,
                const void* B, int64_t ldb, int b_col,
                int dtype, const void* bias, int relu,
                const void* cin, int64_t ldcin, int cin_type,
                void* C, int64_t ldc) {
    if (check_args(M, N, K, lda, a_col, ldb, b_col, dtype) || ldc < N) return 1;
    if (check_cin(cin, ldcin, cin_type, N, dtype)) return 1;
    if (M == 0 || N == 0) return 0;
    int overflow = 0;

    if (dtype == OR_I8) {
        const int8_t* a8 = (const int8_t*)A;
        const int8_t* b8 = (const int8_t*)B;
        const int32_t* bi = (const int32_t*)bias;
        int32_t* c = (int32_t*)C;
        /* b(k,j) as a dense K x N int32 array */
        int32_t* bd = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1) * (size_t)N);
        if (!bd) return 1;
        for (int64_t k = 0; k < K; ++k)
            for (int64_t j = 0; j < N; ++j) bd[k * N + j] = b8[b_off(k, j, ldb, b_col)];
#pragma omp parallel for schedule(dynamic, 1) reduction(| : overflow)
        for (int64_t i = 0; i < M; ++i) {
            int64_t* acc = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
            for (int64_t j = 0; j < N; ++j) {
                acc[j] = init_i((const int32_t*)cin, ldcin, bi, i, j);
                if (acc[j] > INT32_MAX || acc[j] < INT32_MIN) overflow = 1;
            }
            for (int64_t k = 0; k < K; ++k) {
                int64_t aik = a8[a_off(i, k, lda, a_col)];
                const int32_t* brow = bd + k * N;
                for (int64_t j = 0; j < N; ++j) {
                    acc[j] += aik * brow[j];
                    if (acc[j] > INT32_MAX || acc[j] < INT32_MIN) overflow = 1;
                }
            }
            for (int64_t j = 0; j < N; ++j) {
                int64_t v = acc[j];
                if (relu && !(v > 0)) v = 0;
                c[i * ldc + j] = (int32_t)v;
            }
            free(acc);
        }
        free(bd);
        return overflow ? 2 : 0;
    }

    const float* bf = (const float*)bias;
    double* c = (double*)C;
    double* bd = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)N);
    if (!bd) return 1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) bd[k * N + j] = elem_f(B, dtype, b_off(k, j, ldb, b_col));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        double* acc = c + i * ldc;
        for (int64_t j = 0; j < N; ++j) acc[j] = init_f(cin, ldcin, cin_type, bf, i, j);
        for (int64_t k = 0; k < K; ++k) {
            double aik = elem_f(A, dtype, a_off(i, k, lda, a_col));
            const double* brow = bd + k * N;
            for (int64_t j = 0; j < N; ++j) acc[j] += aik * brow[j];
        }
        if (relu)
            for (int64_t j = 0; j < N; ++j) acc[j] = relu_f(acc[j]);
    }
    free(bd);
    return 0;
}

/* ---- selected entries ---------------------------------------------------- */

int oracle_gemm_entries(int64_t M, int64_t N, int64_t K,
                        const void* A, int64_t lda, int a_col,
                        const void* B, int64_t ldb, int b_col,
                        int dtype, const void* bias, int relu,
                        const void* cin, int64_t ldcin, int cin_type,
                        const int64_t* ii, const int64_t* jj, int64_t n, void* out) {
    if (check_args(M, N, K, lda, a_col, ldb, b_col, dtype) || n < 0) return 1;
    if (check_cin(cin, ldcin, cin_type, N, dtype)) return 1;
    for (int64_t t = 0; t < n; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N) return 1;
    int overflow = 0;
    if (dtype == OR_I8) {
        const int8_t* a8 = (const int8_t*)A;
        const int8_t* b8 = (const int8_t*)B;
        const int32_t* bi = (const int32_t*)bias;
        int32_t* o = (int32_t*)out;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : overflow)
        for (int64_t t = 0; t < n; ++t) {
            int64_t i = ii[t], j = jj[t];
            int64_t acc = init_i((const int32_t*)cin, ldcin, bi, i, j);
            if (acc > INT32_MAX || acc < INT32_MIN) overflow = 1;
            for (int64_t k = 0; k < K; ++k) {
                acc += (int64_t)a8[a_off(i, k, lda, a_col)] * (int64_t)b8[b_off(k, j, ldb, b_col)];
                if (acc > INT32_MAX || acc < INT32_MIN) overflow = 1;
            }
            if (relu && !(acc > 0)) acc = 0;
            o[t] = (int32_t)acc;
        }
        return overflow ? 2 : 0;
    }
    const float* bf = (const float*)bias;
    double* o = (double*)out;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = ii[t], j = jj[t];
        double acc = init_f(cin, ldcin, cin_type, bf, i, j);
        for (int64_t k = 0; k < K; ++k)
            acc += elem_f(A, dtype, a_off(i, k, lda, a_col)) * elem_f(B, dtype, b_off(k, j, ldb, b_col));
        o[t] = relu ? relu_f(acc) : acc;
    }
    return 0;
}

/* ---- threads used by the parallel loops ---------------------------------- */

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---- 2-D convolution -------------------------------------------------------
 *
 * The Conv2d + Bias + ReLU pattern (kimm240.github.io/tvm, post "Implement
 * and enable Conv2d-Reshape-Add-ReLU fusion") written out directly, with the
 * same exact decoders and wide accumulation as the product above:
 *
 *   y[n][p][q][k] = epi( bias[k] + sum_{r,s,c} x[n][h][w][c] * f[k][r][s][c] ),
 *   h = p*stride_h - pad_h + r*dil_h,   w = q*stride_w - pad_w + s*dil_w,
 *
 * where taps with h or w outside the input contribute nothing (zero padding),
 * and the sum runs over r (outer), s, c (inner) in ascending order after the
 * bias.  x is NHWC, f is KRSC, y is NPQK (all dense, channels fastest), with
 * P = (H + 2*pad_h - dil_h*(R-1) - 1) / stride_h + 1 and Q likewise.
 * y is double for float types, int32 for int8 (range checked as above).
 */
typedef struct {
    int64_t N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, P, Q;
} conv_geom;

/* The geometry of a call, or 1 for invalid arguments. */
static int conv_setup(conv_geom* g, int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                      int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h, int64_t dil_w,
                      int dtype) {
    if (N < 0 || H < 0 || W < 0 || C < 0 || K < 0 || R < 1 || S < 1) return 1;
    if (pad_h < 0 || pad_w < 0 || stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1) return 1;
    if (dtype < OR_F16 || dtype > OR_I8) return 1;
    const int64_t eh = H + 2 * pad_h - dil_h * (R - 1) - 1, ew = W + 2 * pad_w - dil_w * (S - 1) - 1;
    if (eh < 0 || ew < 0) return 1;
    conv_geom c = {N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, eh / stride_h + 1, ew / stride_w + 1};
    *g = c;
    return 0;
}

/* One output y[n][p][q][k]: int8 into *yi (setting *overflow when a partial
 * sum leaves the int32 range), float types into *yf. */
static void conv_point(const conv_geom* g, const void* x, const void* f, int dtype, const void* bias, int relu,
                       int64_t n, int64_t p, int64_t q, int64_t k, double* yf, int32_t* yi, int* overflow) {
    const int64_t H = g->H, W = g->W, C = g->C, R = g->R, S = g->S;
    if (dtype == OR_I8) {
        const int8_t* x8 = (const int8_t*)x;
        const int8_t* f8 = (const int8_t*)f;
        int64_t acc = bias ? ((const int32_t*)bias)[k] : 0;
        for (int64_t r = 0; r < R; ++r)
            for (int64_t s = 0; s < S; ++s) {
                const int64_t h = p * g->stride_h - g->pad_h + r * g->dil_h, w = q * g->stride_w - g->pad_w + s * g->dil_w;
                if (h < 0 || h >= H || w < 0 || w >= W) continue;
                for (int64_t c = 0; c < C; ++c) {
                    acc += (int64_t)x8[((n * H + h) * W + w) * C + c] * (int64_t)f8[((k * R + r) * S + s) * C + c];
                    if (acc > INT32_MAX || acc < INT32_MIN) *overflow = 1;
                }
            }
        if (relu && !(acc > 0)) acc = 0;
        *yi = (int32_t)acc;
        return;
    }
    double acc = bias ? (double)((const float*)bias)[k] : 0.0;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t s = 0; s < S; ++s) {
            const int64_t h = p * g->stride_h - g->pad_h + r * g->dil_h, w = q * g->stride_w - g->pad_w + s * g->dil_w;
            if (h < 0 || h >= H || w < 0 || w >= W) continue;
            for (int64_t c = 0; c < C; ++c)
                acc += elem_f(x, dtype, ((n * H + h) * W + w) * C + c) * elem_f(f, dtype, ((k * R + r) * S + s) * C + c);
        }
    *yf = relu ? relu_f(acc) : acc;
}

int oracle_conv2d(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                  int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h, int64_t dil_w,
                  const void* x, const void* f, int dtype, const void* bias, int relu, void* y) {
    conv_geom g;
    if (conv_setup(&g, N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, dtype)) return 1;
    int overflow = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : overflow)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t p = 0; p < g.P; ++p)
            for (int64_t q = 0; q < g.Q; ++q)
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t out = ((n * g.P + p) * g.Q + q) * K + k;
                    conv_point(&g, x, f, dtype, bias, relu, n, p, q, k, (double*)y + out, (int32_t*)y + out, &overflow);
                }
    return overflow ? 2 : 0;
}

/* The same outputs at listed positions only: output t is pixel mm[t] (the
 * row (n*P + p)*Q + q of y seen as an N*P*Q x K matrix) and channel kk[t]. */
int oracle_conv2d_entries(int64_t N, int64_t H, int64_t W, int64_t C, int64_t K, int64_t R, int64_t S,
                          int64_t pad_h, int64_t pad_w, int64_t stride_h, int64_t stride_w, int64_t dil_h, int64_t dil_w,
                          const void* x, const void* f, int dtype, const void* bias, int relu,
                          const int64_t* mm, const int64_t* kk, int64_t n_out, void* out) {
    conv_geom g;
    if (conv_setup(&g, N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, dtype) || n_out < 0) return 1;
    for (int64_t t = 0; t < n_out; ++t)
        if (mm[t] < 0 || mm[t] >= N * g.P * g.Q || kk[t] < 0 || kk[t] >= K) return 1;
    int overflow = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : overflow)
    for (int64_t t = 0; t < n_out; ++t) {
        const int64_t n = mm[t] / (g.P * g.Q), p = mm[t] / g.Q % g.P, q = mm[t] % g.Q;
        conv_point(&g, x, f, dtype, bias, relu, n, p, q, kk[t], (double*)out + t, (int32_t*)out + t, &overflow);
    }
    return overflow ? 2 : 0;
}
