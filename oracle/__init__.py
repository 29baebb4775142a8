"""CPU oracle for the GEMM hot path -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  It is a plain C triple loop (see oracle.c for the definition and
the passages it follows) loaded with ctypes; it shares no code with the HIP
library and never imports it.

Operands are passed in their storage form as numpy arrays:
  dtype 0 (f16) and 1 (bf16): uint16 bit patterns;  2 (f32): float32;
  3 (int8): int8.  Bias: float32 (float types) or int32 (int8).
  Optional c_in (the reduction's per-element initial value, row-major with
  leading dimension ldcin): for float problems stored as f16/bf16 (uint16,
  c_in_type 0/1) or float32 (c_in_type 2); for int8 problems int32.
Results: float64 for the float types (the exact-input, binary64-accumulated
value), int32 for int8.
"""
import ctypes
import os

import numpy as np

F16, BF16, F32, I8 = 0, 1, 2, 3
_STORAGE = {F16: np.uint16, BF16: np.uint16, F32: np.float32, I8: np.int8}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")


class OracleError(RuntimeError):
    pass


class Oracle:
    """ctypes view of one build of oracle.c (the default build, or a test variant)."""

    def __init__(self, path=_LIB_PATH):
        if not os.path.exists(path):
            from . import build as _b
            if os.path.abspath(path) != os.path.abspath(_LIB_PATH):
                raise OracleError(f"oracle library not found: {path}")
            _b.build(quiet=True)
        self.path = path
        lib = ctypes.CDLL(path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_gemm.argtypes = [i64, i64, i64, vp, i64, ci, vp, i64, ci, ci, vp, ci, vp, i64, ci, vp, i64]
        lib.oracle_gemm.restype = ci
        lib.oracle_gemm_entries.argtypes = [i64, i64, i64, vp, i64, ci, vp, i64, ci, ci, vp, ci, vp, i64, ci, vp, vp, i64,
                                            vp]
        lib.oracle_gemm_entries.restype = ci
        lib.oracle_conv2d.argtypes = [i64] * 13 + [vp, vp, ci, vp, ci, vp]
        lib.oracle_conv2d_entries.argtypes = [i64] * 13 + [vp, vp, ci, vp, ci, vp, vp, i64, vp]
        lib.oracle_conv2d_entries.restype = ci
        lib.oracle_conv2d.restype = ci
        lib.oracle_decode.argtypes = [ci, vp, i64, vp]
        lib.oracle_decode.restype = ci
        lib.oracle_max_threads.restype = ci
        lib.oracle_set_threads.argtypes = [ci]
        self.lib = lib

    # -- helpers ---------------------------------------------------------
    @staticmethod
    def _buf(x, dtype):
        want = _STORAGE[dtype]
        x = np.ascontiguousarray(x)
        if x.dtype != want:
            if x.dtype.itemsize != np.dtype(want).itemsize:
                raise OracleError(f"operand dtype {x.dtype} does not match storage {np.dtype(want)}")
            x = x.view(want)
        return x

    @staticmethod
    def _bias(bias, dtype):
        if bias is None:
            return None
        return np.ascontiguousarray(bias, dtype=np.int32 if dtype == I8 else np.float32)

    @staticmethod
    def _check_extent(x, rows, cols, ld, name):
        need = 0 if rows == 0 or cols == 0 else (rows - 1) * ld + cols
        if x.size < need:
            raise OracleError(f"{name} holds {x.size} elements, needs {need}")

    def _prep(self, M, N, K, A, lda, a_col, B, ldb, b_col, dtype, bias):
        A = self._buf(A, dtype)
        B = self._buf(B, dtype)
        self._check_extent(A, K if a_col else M, M if a_col else K, lda, "A")
        self._check_extent(B, N if b_col else K, K if b_col else N, ldb, "B")
        bias = self._bias(bias, dtype)
        if bias is not None and bias.size < N:
            raise OracleError("bias shorter than N")
        return A, B, bias

    def _cin(self, c_in, c_in_type, ldcin, M, N, dtype):
        """(pointer, ld, type code, array) of the optional initial-value tensor."""
        if c_in is None:
            return None, max(N, 1), 0, None
        if dtype == I8:
            c_in_type = I8
            c_in = np.ascontiguousarray(c_in, dtype=np.int32)
        else:
            if c_in_type not in (F16, BF16, F32):
                raise OracleError("c_in_type must be 0 (f16), 1 (bf16) or 2 (f32)")
            c_in = self._buf(c_in, c_in_type)
        ldcin = ldcin if ldcin is not None else max(N, 1)
        self._check_extent(c_in, M, N, ldcin, "c_in")
        return c_in.ctypes.data, ldcin, c_in_type, c_in

    # -- entry points ----------------------------------------------------
    def gemm(self, M, N, K, A, lda, a_col, B, ldb, b_col, dtype, bias=None, relu=False, c_in=None, c_in_type=None,
             ldcin=None):
        """Full C (M x N): float64 for float types, int32 for int8."""
        A, B, bias = self._prep(M, N, K, A, lda, a_col, B, ldb, b_col, dtype, bias)
        cp, cld, ct, _keep = self._cin(c_in, c_in_type, ldcin, M, N, dtype)
        C = np.zeros((M, N), dtype=np.int32 if dtype == I8 else np.float64)
        rc = self.lib.oracle_gemm(M, N, K, A.ctypes.data, lda, int(a_col), B.ctypes.data, ldb, int(b_col),
                                  dtype, None if bias is None else bias.ctypes.data, int(relu),
                                  cp, cld, ct, C.ctypes.data, max(N, 1))
        self._rc(rc)
        return C

    def gemm_entries(self, M, N, K, A, lda, a_col, B, ldb, b_col, dtype, ii, jj, bias=None, relu=False, c_in=None,
                     c_in_type=None, ldcin=None):
        """C at the listed (ii[t], jj[t]) entries, same arithmetic as gemm()."""
        A, B, bias = self._prep(M, N, K, A, lda, a_col, B, ldb, b_col, dtype, bias)
        cp, cld, ct, _keep = self._cin(c_in, c_in_type, ldcin, M, N, dtype)
        ii = np.ascontiguousarray(ii, dtype=np.int64)
        jj = np.ascontiguousarray(jj, dtype=np.int64)
        if ii.shape != jj.shape:
            raise OracleError("index arrays differ in length")
        out = np.zeros(ii.size, dtype=np.int32 if dtype == I8 else np.float64)
        rc = self.lib.oracle_gemm_entries(M, N, K, A.ctypes.data, lda, int(a_col), B.ctypes.data, ldb, int(b_col),
                                          dtype, None if bias is None else bias.ctypes.data, int(relu),
                                          cp, cld, ct, ii.ctypes.data, jj.ctypes.data, ii.size, out.ctypes.data)
        self._rc(rc)
        return out

    def conv2d(self, x, f, dtype, pad=(0, 0), stride=(1, 1), dil=(1, 1), bias=None, relu=False):
        """y (N, P, Q, K) of the NHWC input x (N, H, W, C) and KRSC filter f
        (K, R, S, C), both storage arrays; float64 for float types, int32 for int8."""
        x = self._buf(x, dtype)
        f = self._buf(f, dtype)
        if x.ndim != 4 or f.ndim != 4 or x.shape[3] != f.shape[3]:
            raise OracleError("x must be (N, H, W, C) and f (K, R, S, C) with the same C")
        N, H, W, C = x.shape
        K, R, S, _ = f.shape
        P = (H + 2 * pad[0] - dil[0] * (R - 1) - 1) // stride[0] + 1
        Q = (W + 2 * pad[1] - dil[1] * (S - 1) - 1) // stride[1] + 1
        bias = self._bias(bias, dtype)
        if bias is not None and bias.size < K:
            raise OracleError("bias shorter than K")
        y = np.zeros((N, max(P, 0), max(Q, 0), K), dtype=np.int32 if dtype == I8 else np.float64)
        rc = self.lib.oracle_conv2d(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
                                    x.ctypes.data, f.ctypes.data, dtype, None if bias is None else bias.ctypes.data,
                                    int(relu), y.ctypes.data)
        self._rc(rc)
        return y

    def conv2d_entries(self, x, f, dtype, mm, kk, pad=(0, 0), stride=(1, 1), dil=(1, 1), bias=None, relu=False):
        """Outputs of conv2d() at output pixel mm[t] (row of y seen as an
        (N*P*Q, K) matrix) and channel kk[t], same arithmetic as conv2d()."""
        x = self._buf(x, dtype)
        f = self._buf(f, dtype)
        if x.ndim != 4 or f.ndim != 4 or x.shape[3] != f.shape[3]:
            raise OracleError("x must be (N, H, W, C) and f (K, R, S, C) with the same C")
        N, H, W, C = x.shape
        K, R, S, _ = f.shape
        bias = self._bias(bias, dtype)
        if bias is not None and bias.size < K:
            raise OracleError("bias shorter than K")
        mm = np.ascontiguousarray(mm, dtype=np.int64)
        kk = np.ascontiguousarray(kk, dtype=np.int64)
        if mm.shape != kk.shape:
            raise OracleError("index arrays differ in length")
        out = np.zeros(mm.size, dtype=np.int32 if dtype == I8 else np.float64)
        rc = self.lib.oracle_conv2d_entries(N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
                                            x.ctypes.data, f.ctypes.data, dtype,
                                            None if bias is None else bias.ctypes.data, int(relu), mm.ctypes.data,
                                            kk.ctypes.data, mm.size, out.ctypes.data)
        self._rc(rc)
        return out

    def decode(self, dtype, X):
        X = self._buf(X, dtype)
        out = np.empty(X.size, dtype=np.float64)
        self._rc(self.lib.oracle_decode(dtype, X.ctypes.data, X.size, out.ctypes.data))
        return out

    def max_threads(self):
        return int(self.lib.oracle_max_threads())

    def set_threads(self, n):
        self.lib.oracle_set_threads(int(n))

    @staticmethod
    def _rc(rc):
        if rc == 1:
            raise OracleError("invalid argument")
        if rc == 2:
            raise OverflowError("int8 product sum left the int32 range")
        if rc != 0:
            raise OracleError(f"oracle returned {rc}")


_default = None


def get():
    """The oracle built from oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def gemm(*a, **kw):
    return get().gemm(*a, **kw)


def gemm_entries(*a, **kw):
    return get().gemm_entries(*a, **kw)


def decode(*a, **kw):
    return get().decode(*a, **kw)
