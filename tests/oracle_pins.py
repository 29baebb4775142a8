"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each pin takes an ``oracle.Oracle`` (the real build, or a build with a
planted mistake) and raises AssertionError when the oracle disagrees with
  * a value printed on the pages (the 256-element block sum, 32640),
  * a closed form (all-ones products, identity matrices),
  * exact rational arithmetic on tiny inputs (Python's fractions),
  * a library routine on inputs where that routine is exact (numpy's integer
    and float64 matmul, numpy's float16 and torch's bfloat16 decoders),
  * an invariant of the product (transposition, linearity),
  * the oracle's own two entry points against each other.
Inputs are built here from logical matrices with numpy/torch casts; nothing
below calls the HIP library.
"""
import json
import os
from fractions import Fraction

import numpy as np
import torch

F16, BF16, F32, I8 = 0, 1, 2, 3
FLOATS = (F16, BF16, F32)
ALL = (F16, BF16, F32, I8)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = 2.0 ** -53


# ---------------------------------------------------------------- helpers

def to_storage(vals, dtype):
    """Logical values (exactly representable) -> storage array of `dtype`."""
    v = np.asarray(vals, dtype=np.float64)
    if dtype == F32:
        return v.astype(np.float32)
    if dtype == F16:
        return v.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return v.astype(np.int8)


def lib_decode(store, dtype):
    """Exact values of storage elements via numpy / torch casts (not the oracle)."""
    s = np.asarray(store)
    if dtype == F16:
        return s.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return torch.from_numpy(s.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    if dtype == F32:
        return s.astype(np.float64)
    return s.astype(np.float64)


def pad_value(dtype):
    return {F16: np.float16(np.nan).view(np.uint16), BF16: np.uint16(0x7FC0),
            F32: np.float32(np.nan), I8: np.int8(99)}[dtype]


def store_matrix(logical, dtype, col_major, ld):
    """Lay out a logical R x C matrix in storage (row- or column-major, leading
    dimension ld); padding elements hold NaN (floats) or 99 (int8)."""
    logical = np.asarray(logical)
    R, C = logical.shape
    body = logical.T if col_major else logical
    rows, cols = body.shape
    assert ld >= cols
    s = to_storage(body, dtype)
    out = np.full((rows, ld), pad_value(dtype), dtype=s.dtype)
    out[:, :cols] = s
    return out.reshape(-1)


def random_logical(rng, shape, dtype, lo=-1.0, hi=1.0):
    """Random values that are exactly representable in `dtype`."""
    if dtype == I8:
        return rng.integers(-128, 128, size=shape).astype(np.float64)
    x = rng.uniform(lo, hi, size=shape)
    return lib_decode(to_storage(x, dtype), dtype).reshape(shape)


def run(o, A_log, B_log, dtype, a_col=False, b_col=False, bias=None, relu=False, pad=(0, 0)):
    """Store logical A (M x K), B (K x N) and call the oracle's full product."""
    M, K = A_log.shape
    K2, N = B_log.shape
    assert K == K2
    lda = (M if a_col else K) + pad[0]
    ldb = (K if b_col else N) + pad[1]
    A = store_matrix(A_log, dtype, a_col, max(lda, 1))
    B = store_matrix(B_log, dtype, b_col, max(ldb, 1))
    return o.gemm(M, N, K, A, max(lda, 1), a_col, B, max(ldb, 1), b_col, dtype, bias=bias, relu=relu)


def _layouts():
    return [(False, False), (False, True), (True, False), (True, True)]


# ---------------------------------------------------------------- pins

def pin_decoders(o):
    """All 65536 binary16 and bfloat16 bit patterns decode to the values numpy's
    float16 and torch's bfloat16 casts give (NaN patterns to NaN)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dtype in (F16, BF16):
        got = o.decode(dtype, bits)
        want = lib_decode(bits, dtype)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), f"NaN set differs for dtype {dtype}"
        assert np.array_equal(got[~nan], want[~nan]), f"decoded values differ for dtype {dtype}"
    x = np.array([0.0, -0.0, 1.5, -3.25e-3, 6.0e-8, 3.4e38, np.inf], dtype=np.float32)
    assert np.array_equal(o.decode(F32, x), x.astype(np.float64))
    i = np.arange(-128, 128, dtype=np.int64).astype(np.int8)
    assert np.array_equal(o.decode(I8, i), np.arange(-128, 128, dtype=np.float64))


def pin_identity(o):
    """A . I = A and I . B = B exactly, every type and layout, with NaN/99
    padding past the leading dimension that must never reach C."""
    rng = np.random.default_rng(11)
    M, K, N = 5, 7, 6
    for dtype in ALL:
        for a_col, b_col in _layouts():
            A = random_logical(rng, (M, K), dtype)
            C = run(o, A, np.eye(K), dtype, a_col, b_col, pad=(3, 2))
            assert np.array_equal(C.astype(np.float64), A), f"A.I != A (dtype {dtype}, layout {a_col},{b_col})"
            B = random_logical(rng, (K, N), dtype)
            C = run(o, np.eye(K), B, dtype, a_col, b_col, pad=(1, 4))
            assert np.array_equal(C.astype(np.float64), B), f"I.B != B (dtype {dtype}, layout {a_col},{b_col})"


def pin_closed_forms(o):
    """All-ones operands give C = K; with a bias, K + bias[j]; with A = -1,
    B = 1, bias and ReLU, max(0, bias[j] - K)."""
    M, N, K = 3, 5, 37
    for dtype in ALL:
        for a_col, b_col in _layouts():
            C = run(o, np.ones((M, K)), np.ones((K, N)), dtype, a_col, b_col)
            assert np.all(C == K), f"ones: dtype {dtype}"
            bias = (np.arange(N) * 3 - 7).astype(np.int32 if dtype == I8 else np.float32)
            C = run(o, np.ones((M, K)), np.ones((K, N)), dtype, a_col, b_col, bias=bias)
            assert np.array_equal(C, np.broadcast_to(K + bias.astype(np.float64), (M, N))), f"ones+bias: dtype {dtype}"
            bias = (np.arange(N) * 20 - 10).astype(np.int32 if dtype == I8 else np.float32)
            C = run(o, -np.ones((M, K)), np.ones((K, N)), dtype, a_col, b_col, bias=bias, relu=True)
            want = np.maximum(0.0, bias.astype(np.float64) - K)
            assert np.array_equal(C, np.broadcast_to(want, (M, N))), f"relu(bias-K): dtype {dtype}"


def pin_printed_value(o):
    """The pages' worked example: the sum of arange(256) is 32640 (exact for
    f16, bf16 and f32 inputs, since 0..255 are representable in all three).
    The int8 variant a = k - 128 gives 32640 - 128*256 = -128."""
    with open(os.path.join(GOLDEN, "block_sum_arange256.json")) as f:
        g = json.load(f)
    expected = g["expected"]
    k = np.arange(256, dtype=np.float64)
    for dtype in FLOATS:
        C = run(o, k.reshape(1, 256), np.ones((256, 1)), dtype)
        assert C[0, 0] == expected, f"block sum {C[0, 0]} != {expected} (dtype {dtype})"
        C = run(o, np.ones((1, 256)), k.reshape(256, 1), dtype, True, True)
        assert C[0, 0] == expected
    C = run(o, (k - 128).reshape(1, 256), np.ones((256, 1)), I8)
    assert C[0, 0] == expected - 128 * 256 == -128


def _bound(terms_abs_sum, n_adds):
    """Rigorous bound of recursive binary64 summation: gamma_n * sum|terms|."""
    n = n_adds + 1
    return n * U / (1 - n * U) * terms_abs_sum


def pin_bruteforce_exact(o):
    """Tiny random problems vs the exact rational sum (fractions.Fraction of
    the library-decoded inputs): float results lie within the recursive
    summation error bound, int8 results are equal."""
    rng = np.random.default_rng(12)
    for trial in range(60):
        dtype = ALL[trial % 4]
        M, N, K = (int(x) for x in rng.integers(1, 10, size=3))
        a_col, b_col = _layouts()[trial % 4]
        A = random_logical(rng, (M, K), dtype)
        B = random_logical(rng, (K, N), dtype)
        use_bias = trial % 3 == 0
        relu = trial % 2 == 1
        bias = None
        if use_bias:
            bias = (rng.integers(-300, 300, size=N).astype(np.int32) if dtype == I8
                    else rng.uniform(-1, 1, size=N).astype(np.float32))
        C = run(o, A, B, dtype, a_col, b_col, bias=bias, relu=relu)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)]
                b = Fraction(float(bias[j])) if bias is not None else Fraction(0)
                exact = b + sum(terms)
                if relu:
                    exact = max(exact, Fraction(0))
                if dtype == I8:
                    assert Fraction(int(C[i, j])) == exact, f"int8 brute force ({i},{j})"
                else:
                    tol = _bound(float(abs(b) + sum(abs(t) for t in terms)), K)
                    assert abs(Fraction(float(C[i, j])) - exact) <= Fraction(tol), f"float brute force ({i},{j})"


def pin_library_matmul(o):
    """Where numpy's matmul is exact it must agree bit-for-bit: int8 (int64
    matmul) with bias and ReLU, and small-integer floats (every partial sum is
    an integer far below 2^53).  For general floats both results lie within
    the summation bound of the exact value, so within twice it of each other."""
    rng = np.random.default_rng(13)
    M, N, K = 33, 47, 65
    A = random_logical(rng, (M, K), I8)
    B = random_logical(rng, (K, N), I8)
    bias = rng.integers(-2 ** 20, 2 ** 20, size=N).astype(np.int32)
    C = run(o, A, B, I8, bias=bias, relu=True)
    want = np.maximum(0, A.astype(np.int64) @ B.astype(np.int64) + bias)
    assert np.array_equal(C.astype(np.int64), want), "int8 vs numpy int64 matmul"
    for dtype in FLOATS:
        Ai = rng.integers(-8, 9, size=(M, K)).astype(np.float64)
        Bi = rng.integers(-8, 9, size=(K, N)).astype(np.float64)
        C = run(o, Ai, Bi, dtype, False, True)
        assert np.array_equal(C, Ai @ Bi), f"small-integer floats vs numpy (dtype {dtype})"
        A = random_logical(rng, (M, K), dtype)
        B = random_logical(rng, (K, N), dtype)
        C = run(o, A, B, dtype, True, False)
        ref = A @ B
        tol = 2 * _bound(1.0, K) * (np.abs(A) @ np.abs(B))
        assert np.all(np.abs(C - ref) <= tol), f"floats vs numpy matmul (dtype {dtype})"


def pin_transpose(o):
    """(A.B)^T = B^T.A^T: the same storage read through the other layout flag
    gives the transposed product, bit-for-bit (same k order)."""
    rng = np.random.default_rng(14)
    M, N, K = 9, 11, 13
    for dtype in ALL:
        A_log = random_logical(rng, (M, K), dtype)
        B_log = random_logical(rng, (K, N), dtype)
        A = store_matrix(A_log, dtype, False, K)       # row-major A  == column-major A^T
        B = store_matrix(B_log, dtype, False, N)       # row-major B  == column-major B^T
        C = o.gemm(M, N, K, A, K, False, B, N, False, dtype)
        Ct = o.gemm(N, M, K, B, N, True, A, K, True, dtype)
        assert np.array_equal(C.T, Ct), f"transpose invariant (dtype {dtype})"


def pin_linearity_int(o):
    """A.(B1 + B2) = A.B1 + A.B2 exactly for int8 (integers, no rounding)."""
    rng = np.random.default_rng(15)
    M, N, K = 17, 19, 129
    A = random_logical(rng, (M, K), I8)
    B1 = rng.integers(-64, 64, size=(K, N)).astype(np.float64)
    B2 = rng.integers(-64, 64, size=(K, N)).astype(np.float64)
    C = run(o, A, B1 + B2, I8)
    C1 = run(o, A, B1, I8)
    C2 = run(o, A, B2, I8)
    assert np.array_equal(C.astype(np.int64), C1.astype(np.int64) + C2), "linearity"


def pin_entries_match_full(o):
    """The per-entry and the full entry points agree bit-for-bit."""
    rng = np.random.default_rng(16)
    M, N, K = 21, 23, 70
    for dtype in ALL:
        a_col, b_col = _layouts()[dtype]
        A_log = random_logical(rng, (M, K), dtype)
        B_log = random_logical(rng, (K, N), dtype)
        lda, ldb = (M if a_col else K) + 2, (K if b_col else N) + 1
        A = store_matrix(A_log, dtype, a_col, lda)
        B = store_matrix(B_log, dtype, b_col, ldb)
        bias = (rng.integers(-99, 99, size=N).astype(np.int32) if dtype == I8
                else rng.uniform(-1, 1, size=N).astype(np.float32))
        C = o.gemm(M, N, K, A, lda, a_col, B, ldb, b_col, dtype, bias=bias, relu=True)
        ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        E = o.gemm_entries(M, N, K, A, lda, a_col, B, ldb, b_col, dtype, ii.ravel(), jj.ravel(), bias=bias, relu=True)
        assert np.array_equal(E.reshape(M, N), C), f"entries != full (dtype {dtype})"


def pin_int32_range(o):
    """An int8 sum that leaves int32 is reported; one just inside is exact."""
    ok_k = (2 ** 31 - 1) // (128 * 128)            # 131071: 131071 * 16384 < 2^31
    A = np.full(ok_k + 1, -128, dtype=np.int8)
    C = o.gemm(1, 1, ok_k, A, ok_k, False, A, 1, False, I8)
    assert int(C[0, 0]) == ok_k * 16384
    try:
        o.gemm(1, 1, ok_k + 1, A, ok_k + 1, False, A, 1, False, I8)
    except OverflowError:
        pass
    else:
        raise AssertionError("int32 overflow not reported")


def pin_degenerate(o):
    """K = 0 gives epi(bias or 0); M = 0 or N = 0 gives an empty result."""
    for dtype in ALL:
        bias = np.array([3, -2, 0, 5], dtype=np.int32 if dtype == I8 else np.float32)
        A = to_storage(np.zeros(1), dtype)
        C = o.gemm(2, 4, 0, A, 1, False, A, 4, False, dtype, bias=bias, relu=True)
        assert np.array_equal(C, np.broadcast_to(np.maximum(bias, 0).astype(C.dtype), (2, 4)))
        C = o.gemm(2, 4, 0, A, 1, False, A, 4, False, dtype)
        assert np.all(C == 0)
        assert o.gemm(0, 4, 3, A, 3, False, to_storage(np.zeros(12), dtype), 4, False, dtype).shape == (0, 4)


def _cin_store(logical, ctype, ld):
    """Row-major initial-value tensor in storage (padding: NaN / int32 sentinel)."""
    logical = np.asarray(logical, dtype=np.float64)
    R, C = logical.shape
    if ctype == I8:
        out = np.full((R, ld), -77777, dtype=np.int32)
        out[:, :C] = logical.astype(np.int32)
        return out.reshape(-1)
    s = to_storage(logical, ctype)
    out = np.full((R, ld), pad_value(ctype), dtype=s.dtype)
    out[:, :C] = s
    return out.reshape(-1)


def _cin_types(dtype):
    return (I8,) if dtype == I8 else (F16, BF16, F32)


def pin_init_tensor_closed_forms(o):
    """With an initial-value tensor c_in (stored f16 / bf16 / f32, or int32 for
    int8; row-major with padding past its leading dimension):
      K = 0            -> C = epi(c_in + bias), c_in decoded by numpy / torch;
      all-ones, K = 37 -> C = c_in + 37 exactly;
    with an asymmetric c_in, so a transposed or mis-strided read fails."""
    rng = np.random.default_rng(21)
    M, N = 4, 6
    for dtype in ALL:
        for ct in _cin_types(dtype):
            ld = N + 3
            logical = (rng.integers(-40, 40, size=(M, N)) if ct == I8
                       else random_logical(rng, (M, N), ct, -8.0, 8.0))
            cin = _cin_store(logical, ct, ld)
            want_cin = logical if ct == I8 else lib_decode(to_storage(logical, ct), ct).reshape(M, N)
            bias = (rng.integers(-9, 9, size=N).astype(np.int32) if dtype == I8
                    else rng.integers(-9, 9, size=N).astype(np.float32))
            Z = to_storage(np.zeros(1), dtype)
            C = o.gemm(M, N, 0, Z, 1, False, Z, N, False, dtype, bias=bias, relu=True, c_in=cin, c_in_type=ct,
                       ldcin=ld)
            assert np.array_equal(C.astype(np.float64), np.maximum(want_cin + bias, 0)), \
                f"K=0 with c_in != relu(c_in + bias) (dtype {dtype}, c_in type {ct})"
            K = 37
            ones = np.ones((M, K))
            C = run_cin(o, ones, np.ones((K, N)), dtype, cin, ct, ld)
            assert np.array_equal(C.astype(np.float64), want_cin + K), f"ones with c_in (dtype {dtype}, {ct})"


def run_cin(o, A_log, B_log, dtype, cin, ct, ld, bias=None, relu=False):
    M, K = A_log.shape
    N = B_log.shape[1]
    A = store_matrix(A_log, dtype, False, K)
    B = store_matrix(B_log, dtype, False, N)
    return o.gemm(M, N, K, A, K, False, B, N, False, dtype, bias=bias, relu=relu, c_in=cin, c_in_type=ct, ldcin=ld)


def pin_init_tensor_linearity(o):
    """int8: C(A, B, c_in) - C(A, B, no c_in) == c_in exactly, entry by entry
    (a dropped, doubled or shifted c_in changes the difference); the int32
    range check covers the initial value too."""
    rng = np.random.default_rng(22)
    M, N, K = 7, 9, 33
    A = rng.integers(-128, 128, size=(M, K)).astype(np.float64)
    B = rng.integers(-128, 128, size=(K, N)).astype(np.float64)
    X = rng.integers(-10 ** 6, 10 ** 6, size=(M, N))
    cin = _cin_store(X, I8, N + 2)
    C1 = run_cin(o, A, B, I8, cin, I8, N + 2)
    A8, B8 = store_matrix(A, I8, False, K), store_matrix(B, I8, False, N)
    C0 = o.gemm(M, N, K, A8, K, False, B8, N, False, I8)
    assert np.array_equal(C1.astype(np.int64) - C0.astype(np.int64), X)
    # c_in + bias leaves int32 although the final sum (after a product of -1) is back inside
    big = _cin_store(np.full((1, 1), 2 ** 31 - 1), I8, 1)
    one, neg = to_storage(np.ones(1), I8), to_storage(-np.ones(1), I8)
    b1 = np.ones(1, dtype=np.int32)
    for call in (lambda: o.gemm(1, 1, 1, neg, 1, False, one, 1, False, I8, bias=b1, c_in=big, ldcin=1),
                 lambda: o.gemm_entries(1, 1, 1, neg, 1, False, one, 1, False, I8, [0], [0], bias=b1, c_in=big,
                                        ldcin=1)):
        try:
            call()
        except OverflowError:
            pass
        else:
            raise AssertionError("int32 overflow through c_in not reported")


def pin_init_tensor_entries(o):
    """Per-entry and full entry points agree bit-for-bit with a c_in (every type)."""
    rng = np.random.default_rng(23)
    M, N, K = 9, 11, 40
    for dtype in ALL:
        for ct in _cin_types(dtype):
            A_log = random_logical(rng, (M, K), dtype)
            B_log = random_logical(rng, (K, N), dtype)
            X = rng.integers(-500, 500, size=(M, N)) if ct == I8 else random_logical(rng, (M, N), ct)
            cin = _cin_store(X, ct, N + 1)
            A = store_matrix(A_log, dtype, False, K)
            B = store_matrix(B_log, dtype, True, K)
            C = o.gemm(M, N, K, A, K, False, B, K, True, dtype, c_in=cin, c_in_type=ct, ldcin=N + 1)
            ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
            E = o.gemm_entries(M, N, K, A, K, False, B, K, True, dtype, ii.ravel(), jj.ravel(), c_in=cin,
                               c_in_type=ct, ldcin=N + 1)
            assert np.array_equal(E.reshape(M, N), C), f"entries != full with c_in (dtype {dtype}, {ct})"


# ---------------------------------------------------------------- convolution

CONV_CASES = [  # (N, H, W, C, K, R, S, pad, stride, dil)
    (2, 7, 6, 3, 4, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 9, 8, 2, 3, 3, 2, (0, 1), (2, 1), (1, 1)),
    (1, 10, 9, 2, 2, 3, 3, (2, 2), (1, 2), (2, 1)),
    (3, 5, 5, 4, 5, 1, 1, (0, 0), (1, 1), (1, 1)),
    (1, 11, 11, 1, 2, 5, 5, (2, 2), (3, 3), (1, 2)),
]


def _conv_torch(x_log, f_log, pad, stride, dil, bias, relu):
    """torch's CPU conv2d in float64 on logical NHWC / KRSC values (exact for small integers)."""
    import torch.nn.functional as Fn
    xt = torch.from_numpy(np.ascontiguousarray(x_log.transpose(0, 3, 1, 2)))
    ft = torch.from_numpy(np.ascontiguousarray(f_log.transpose(0, 3, 1, 2)))
    bt = None if bias is None else torch.from_numpy(np.asarray(bias, dtype=np.float64))
    y = Fn.conv2d(xt, ft, bias=bt, stride=stride, padding=pad, dilation=dil).numpy().transpose(0, 2, 3, 1)
    return np.maximum(y, 0) if relu else y


def pin_conv_vs_torch(o):
    """The convolution equals torch's CPU conv2d (float64) on small-integer inputs,
    every type, with padding, stride, dilation, bias and ReLU."""
    rng = np.random.default_rng(31)
    for case in CONV_CASES:
        N, H, W, C, K, R, S, pad, stride, dil = case
        for dtype in ALL:
            lo, hi = (-128, 128) if dtype == I8 else (-8, 9)
            x_log = rng.integers(lo, hi, size=(N, H, W, C)).astype(np.float64)
            f_log = rng.integers(lo, hi, size=(K, R, S, C)).astype(np.float64)
            bias = rng.integers(-50, 50, size=K)
            b_st = bias.astype(np.int32 if dtype == I8 else np.float32)
            y = o.conv2d(to_storage(x_log, dtype).reshape(x_log.shape), to_storage(f_log, dtype).reshape(f_log.shape),
                         dtype, pad=pad, stride=stride, dil=dil, bias=b_st, relu=True)
            want = _conv_torch(x_log, f_log, pad, stride, dil, bias, True)
            assert y.shape == want.shape, f"conv output shape {y.shape} vs {want.shape} for {case}"
            assert np.array_equal(y.astype(np.float64), want), f"conv != torch conv2d (dtype {dtype}, {case})"


def pin_conv_closed_form_padding(o):
    """All-ones input and filter: each output is C times the number of taps that
    land inside the input, counted here independently per row and column."""
    N, H, W, C, K, R, S = 1, 6, 5, 3, 2, 3, 3
    pad, stride, dil = (1, 2), (2, 1), (1, 2)
    for dtype in ALL:
        x = to_storage(np.ones(N * H * W * C), dtype).reshape(N, H, W, C)
        f = to_storage(np.ones(K * R * S * C), dtype).reshape(K, R, S, C)
        y = o.conv2d(x, f, dtype, pad=pad, stride=stride, dil=dil)
        P, Q = y.shape[1], y.shape[2]
        for p in range(P):
            rows = sum(0 <= p * stride[0] - pad[0] + r * dil[0] < H for r in range(R))
            for q in range(Q):
                cols = sum(0 <= q * stride[1] - pad[1] + s * dil[1] < W for s in range(S))
                assert np.all(y[0, p, q, :] == rows * cols * C), (dtype, p, q)


def pin_conv_1x1_is_the_product(o):
    """A 1x1, stride-1, unpadded convolution is the (N*H*W x C) . (C x K) product."""
    rng = np.random.default_rng(33)
    for dtype in ALL:
        x_log = random_logical(rng, (2, 3, 4, 5), dtype)
        f_log = random_logical(rng, (6, 1, 1, 5), dtype)
        y = o.conv2d(to_storage(x_log, dtype).reshape(x_log.shape), to_storage(f_log, dtype).reshape(f_log.shape), dtype)
        C = run(o, x_log.reshape(24, 5), f_log.reshape(6, 5).T, dtype)
        assert np.array_equal(y.reshape(24, 6), C)


def pin_conv_entries_vs_torch(o):
    """Sampled convolution outputs equal torch's conv2d at the same (pixel, channel)
    positions, every type, with padding, stride and dilation; positions repeat."""
    rng = np.random.default_rng(35)
    for case in CONV_CASES:
        N, H, W, C, K, R, S, pad, stride, dil = case
        for dtype in ALL:
            lo, hi = (-128, 128) if dtype == I8 else (-8, 9)
            x_log = rng.integers(lo, hi, size=(N, H, W, C)).astype(np.float64)
            f_log = rng.integers(lo, hi, size=(K, R, S, C)).astype(np.float64)
            bias = rng.integers(-50, 50, size=K)
            want = _conv_torch(x_log, f_log, pad, stride, dil, bias, True)
            Mp = want.shape[0] * want.shape[1] * want.shape[2]
            mm = rng.integers(0, Mp, size=40)
            kk = rng.integers(0, K, size=40)
            got = o.conv2d_entries(to_storage(x_log, dtype).reshape(x_log.shape),
                                   to_storage(f_log, dtype).reshape(f_log.shape), dtype, mm, kk, pad=pad,
                                   stride=stride, dil=dil, bias=bias.astype(np.int32 if dtype == I8 else np.float32),
                                   relu=True)
            assert np.array_equal(got.astype(np.float64), want.reshape(Mp, K)[mm, kk]), (dtype, case)


ALL_PINS = [pin_decoders, pin_identity, pin_closed_forms, pin_printed_value, pin_bruteforce_exact,
            pin_library_matmul, pin_transpose, pin_linearity_int, pin_entries_match_full,
            pin_int32_range, pin_degenerate, pin_init_tensor_closed_forms, pin_init_tensor_linearity,
            pin_init_tensor_entries, pin_conv_vs_torch, pin_conv_closed_form_padding, pin_conv_1x1_is_the_product,
            pin_conv_entries_vs_torch]
