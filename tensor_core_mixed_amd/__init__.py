"""tensor_core_mixed_amd -- MI355X (gfx950) dense GEMM engine, Python binding.

The engine is the C-ABI library ``_build/libtcm.so`` (declared in
``include/tcm.h``); every step of the product runs in its HIP kernels.  This
module only marshals arguments: the ``tcm_*`` functions take and return
exactly what the C functions do (device pointers as Python ints), and
``gemm`` turns torch tensors into those arguments.  There is no fallback:
if the library is missing, importing the binding's functions raises.

Build the library with ``python -m tensor_core_mixed_amd.build``.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libtcm.so")

# element types and flags (include/tcm.h)
TCM_F16_F32, TCM_BF16_F32, TCM_F32_F32, TCM_I8_I32 = 0, 1, 2, 3
TCM_A_COLMAJOR, TCM_B_COLMAJOR = 1 << 8, 1 << 9
TCM_C_F16, TCM_C_BF16 = 1 << 10, 1 << 11
TCM_EPI_NONE, TCM_EPI_BIAS, TCM_EPI_RELU, TCM_EPI_BIAS_RELU, TCM_EPI_ACCUM = 0, 1, 2, 3, 4
TCM_OK, TCM_ERR_INVALID_VALUE, TCM_ERR_NOT_SUPPORTED, TCM_ERR_HIP, TCM_ERR_ALLOC = 0, 1, 2, 3, 4
TCM_MAX_GROUP = 32


class TcmError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {tcm_status_string(status)}" if what else tcm_status_string(status))


class _PlanInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("config", ctypes.c_int32), ("bm", ctypes.c_int32),
                ("bn", ctypes.c_int32), ("bk", ctypes.c_int32), ("mode", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("iters_per_tile", ctypes.c_int64), ("dp_tiles", ctypes.c_int64),
                ("sk_tiles", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("fixup_kernel", ctypes.c_int32), ("split", ctypes.c_int32)]


class GroupEntry(ctypes.Structure):
    """tcm_group_entry: one product of a group (device addresses as ints)."""
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("A", ctypes.c_void_p), ("lda", ctypes.c_int64),
                ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64),
                ("bias", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded libtcm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libtcm.so not found at {LIB_PATH}; build it with "
                               "`python -m tensor_core_mixed_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.tcm_gemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, vp, ci, vp]
        L.tcm_gemm.restype = ci
        L.tcm_gemm_noalloc.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, vp, ci, vp]
        L.tcm_gemm_noalloc.restype = ci
        L.tcm_noalloc_scratch_bytes.argtypes = []
        L.tcm_noalloc_scratch_bytes.restype = i64
        L.tcm_gemm_batched.argtypes = [i64, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, ci, vp, i64, ci, vp]
        L.tcm_gemm_batched.restype = ci
        L.tcm_gemm_grouped.argtypes = [i64, ctypes.POINTER(GroupEntry), i64, ci, ci, vp]
        L.tcm_gemm_grouped.restype = ci
        L.tcm_conv2d.argtypes = [i64] * 13 + [vp, vp, vp, ci, vp, ci, vp]
        L.tcm_conv2d.restype = ci
        L.tcm_status_string.argtypes = [ci]
        L.tcm_status_string.restype = ctypes.c_char_p
        L.tcm_set_option.argtypes = [ctypes.c_char_p, i64]
        L.tcm_set_option.restype = ci
        L.tcm_get_option.argtypes = [ctypes.c_char_p]
        L.tcm_get_option.restype = i64
        L.tcm_plan.argtypes = [i64, i64, i64, i64, i64, i64, ci, ci, ci, ctypes.POINTER(_PlanInfo)]
        L.tcm_plan.restype = ci
        L.tcm_plan_batched.argtypes = [i64, i64, i64, i64, i64, i64, i64, ci, ci, ci, ctypes.POINTER(_PlanInfo)]
        L.tcm_plan_batched.restype = ci
        L.tcm_config_count.restype = ci
        L.tcm_config_info.argtypes = [ci, ci] + [ctypes.POINTER(ctypes.c_int32)] * 4
        L.tcm_config_info.restype = ci
        L.tcm_streamk_range.argtypes = [i64, i64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.tcm_streamk_range.restype = ci
        L.tcm_tile_order.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
        L.tcm_tile_order.restype = ci
        L.tcm_tune.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, vp, ci, ci, vp, ctypes.POINTER(_PlanInfo)]
        L.tcm_tune.restype = ci
        L.tcm_tune_table.argtypes = [ctypes.c_char_p, i64]
        L.tcm_tune_table.restype = ci
        L.tcm_tune_load.argtypes = [ctypes.c_char_p]
        L.tcm_tune_load.restype = ci
        L.tcm_tune_clear.restype = None
        L.tcm_last_plan.argtypes = [ctypes.c_char_p, i64]
        L.tcm_last_plan.restype = ci
        L.tcm_release_workspace.restype = None
        L.tcm_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ---------------------------------------------------------------- C ABI mirror

def tcm_gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, bias, epilogue, stream):
    """C = epi(bias + A.B); pointers are device addresses (ints), stream a
    hipStream_t handle (int) or None.  Returns the tcm status code."""
    return lib().tcm_gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, bias, epilogue, stream)


def tcm_gemm_noalloc(M, N, K, A, lda, B, ldb, C, ldc, dtype, bias, epilogue, stream):
    """tcm_gemm without any allocation (split-k scratch in a fixed device
    array).  Returns the tcm status code."""
    return lib().tcm_gemm_noalloc(M, N, K, A, lda, B, ldb, C, ldc, dtype, bias, epilogue, stream)


def tcm_noalloc_scratch_bytes():
    return lib().tcm_noalloc_scratch_bytes()


def tcm_gemm_batched(batch, M, N, K, A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c, dtype, bias, stride_bias,
                     epilogue, stream):
    """`batch` products C_e = epi(bias_e + A_e.B_e), entry e of each operand
    `stride_*` elements after entry e-1.  Returns the tcm status code."""
    return lib().tcm_gemm_batched(batch, M, N, K, A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c, dtype, bias,
                                  stride_bias, epilogue, stream)


def tcm_status_string(status):
    return lib().tcm_status_string(status).decode()


def tcm_set_option(key, value):
    return lib().tcm_set_option(key.encode(), int(value))


def tcm_get_option(key):
    return lib().tcm_get_option(key.encode())


def tcm_plan(M, N, K, lda, ldb, ldc, dtype, epilogue=0, aligned=True):
    """The plan tcm_gemm would use (host-only query) as a dict."""
    info = _PlanInfo()
    st = lib().tcm_plan(M, N, K, lda, ldb, ldc, dtype, epilogue, int(aligned), ctypes.byref(info))
    if st != TCM_OK:
        raise TcmError(st, "tcm_plan")
    return {f: getattr(info, f) for f, _ in _PlanInfo._fields_}


def tcm_plan_batched(batch, M, N, K, lda, ldb, ldc, dtype, epilogue=0, aligned=True):
    """The plan tcm_gemm_batched would use for `batch` entries (host-only query) as a dict."""
    info = _PlanInfo()
    st = lib().tcm_plan_batched(batch, M, N, K, lda, ldb, ldc, dtype, epilogue, int(aligned), ctypes.byref(info))
    if st != TCM_OK:
        raise TcmError(st, "tcm_plan_batched")
    return {f: getattr(info, f) for f, _ in _PlanInfo._fields_}


def tcm_config_count():
    return lib().tcm_config_count()


def tcm_config_info(index, dtype):
    v = [ctypes.c_int32() for _ in range(4)]
    st = lib().tcm_config_info(index, dtype, *[ctypes.byref(x) for x in v])
    if st != TCM_OK:
        raise TcmError(st, "tcm_config_info")
    return tuple(x.value for x in v)


def tcm_streamk_range(sk_tiles, iters_per_tile, grid, wg):
    b, e = ctypes.c_int64(), ctypes.c_int64()
    st = lib().tcm_streamk_range(sk_tiles, iters_per_tile, grid, wg, ctypes.byref(b), ctypes.byref(e))
    if st != TCM_OK:
        raise TcmError(st, "tcm_streamk_range")
    return b.value, e.value


def tcm_tile_order(t, tiles_m, tiles_n):
    tm, tn = ctypes.c_int32(), ctypes.c_int32()
    st = lib().tcm_tile_order(t, tiles_m, tiles_n, ctypes.byref(tm), ctypes.byref(tn))
    if st != TCM_OK:
        raise TcmError(st, "tcm_tile_order")
    return tm.value, tn.value


def tcm_tune(M, N, K, A, lda, B, ldb, C, ldc, dtype, bias, epilogue, iters, stream):
    """Time every (tile config, mode) on this problem, remember the fastest;
    returns (status, chosen plan as a dict or None)."""
    info = _PlanInfo()
    st = lib().tcm_tune(M, N, K, A, lda, B, ldb, C, ldc, dtype, bias, epilogue, iters, stream, ctypes.byref(info))
    return st, ({f: getattr(info, f) for f, _ in _PlanInfo._fields_} if st == TCM_OK else None)


def tcm_tune_table():
    n = lib().tcm_tune_table(None, 0)
    buf = ctypes.create_string_buffer(n + 1)
    lib().tcm_tune_table(buf, n + 1)
    return buf.value.decode()


def tcm_tune_load(text):
    return lib().tcm_tune_load(text.encode())


def tcm_tune_clear():
    lib().tcm_tune_clear()


def tcm_last_plan():
    n = lib().tcm_last_plan(None, 0)
    buf = ctypes.create_string_buffer(n + 1)
    lib().tcm_last_plan(buf, n + 1)
    return buf.value.decode()


def tcm_release_workspace():
    lib().tcm_release_workspace()


def tcm_gemm_grouped(entries, K, dtype, epilogue, stream):
    """`entries`: a sequence of GroupEntry (or of 9-tuples M, N, A, lda, B,
    ldb, C, ldc, bias).  Returns the tcm status code."""
    arr = (GroupEntry * max(len(entries), 1))()
    for i, e in enumerate(entries):
        arr[i] = e if isinstance(e, GroupEntry) else GroupEntry(*e)
    return lib().tcm_gemm_grouped(len(entries), arr, K, dtype, epilogue, stream)


def tcm_conv2d(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, x, f, y, dtype, bias, epilogue,
               stream):
    """y = epi(bias + conv2d(x, f)) for NHWC x, KRSC f, NPQK y (device
    addresses as ints).  Returns the tcm status code."""
    return lib().tcm_conv2d(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, x, f, y, dtype, bias,
                            epilogue, stream)


def tcm_version():
    return lib().tcm_version().decode()


# ---------------------------------------------------------------- torch convenience

def _torch_dtype_code(t):
    import torch
    codes = {torch.float16: TCM_F16_F32, torch.bfloat16: TCM_BF16_F32, torch.float32: TCM_F32_F32,
             torch.int8: TCM_I8_I32}
    if t.dtype not in codes:
        raise TypeError(f"unsupported operand dtype {t.dtype}")
    return codes[t.dtype]


def _layout(t, name):
    """(leading dimension, column-major?) of a 2-D view with one unit stride."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    r, c = t.shape
    s0, s1 = t.stride()
    if s1 == 1 and (r <= 1 or s0 >= max(c, 1)):
        return max(s0, c, 1), False
    if s0 == 1 and (c <= 1 or s1 >= max(r, 1)):
        return max(s1, r, 1), True
    raise ValueError(f"{name} needs one unit stride (row- or column-major view)")


def gemm(A, B, C=None, bias=None, relu=False, accumulate=False, out_dtype=None, stream=None):
    """C = relu?(A @ B + bias [+ C]) on the GPU via tcm_gemm.

    A: (M, K) and B: (K, N) CUDA tensors of one type (float16, bfloat16,
    float32 or int8), each a row- or column-major view (transposed views
    select the layout flags).  C: optional (M, N) row-major output; its type
    is the accumulator's (float32, int32 for int8) or, for float inputs,
    float16 / bfloat16 (rounded to nearest even); `out_dtype` picks the type
    of a new C.  With `accumulate`, C's current contents are the initial
    value of the sum (C must be given).  bias: optional length-N float32
    (int32) vector.  Runs on `stream` (default: torch's current stream) and
    returns C."""
    import torch
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    code = _torch_dtype_code(A)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: {K} vs {K2}")
    lda, a_col = _layout(A, "A")
    ldb, b_col = _layout(B, "B")
    acc_dtype = torch.int32 if code == TCM_I8_I32 else torch.float32
    if accumulate and C is None:
        raise ValueError("accumulate needs C")
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype or acc_dtype, device=A.device)
    c_flags = {torch.float16: TCM_C_F16, torch.bfloat16: TCM_C_BF16}.get(C.dtype, 0)
    if c_flags and code == TCM_I8_I32:
        raise TypeError("int8 products have an int32 C")
    if (C.dtype != acc_dtype and not c_flags) or C.dim() != 2 or tuple(C.shape) != (M, N) or (N > 1 and C.stride(1) != 1):
        raise ValueError("C must be a row-major (M, N) tensor of the accumulator type, float16 or bfloat16")
    ldc = max(C.stride(0), N, 1)
    epi = (TCM_EPI_BIAS if bias is not None else 0) | (TCM_EPI_RELU if relu else 0) | (TCM_EPI_ACCUM if accumulate else 0)
    if bias is not None:
        if bias.dtype != acc_dtype or bias.numel() < N or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous length-N vector of the accumulator type")
    dtype = code | (TCM_A_COLMAJOR if a_col else 0) | (TCM_B_COLMAJOR if b_col else 0) | c_flags
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    st = tcm_gemm(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, dtype,
                  bias.data_ptr() if bias is not None else None, epi, stream)
    if st != TCM_OK:
        raise TcmError(st, "tcm_gemm")
    return C


def gemm_batched(A, B, C=None, bias=None, relu=False, accumulate=False, out_dtype=None, stream=None):
    """C[e] = relu?(A[e] @ B[e] + bias [+ C[e]]) for every e, via tcm_gemm_batched.

    A: (batch, M, K), B: (batch, K, N) CUDA tensors whose last two dimensions
    are row- or column-major views; a batch stride of 0 (an expanded tensor)
    shares that operand across the batch.  C: optional (batch, M, N) with
    row-major entries.  bias: optional (N,) shared or (batch, N) per entry.
    Other arguments as gemm()."""
    import torch
    if A.dim() != 3 or B.dim() != 3 or A.shape[0] != B.shape[0]:
        raise ValueError("A and B must be (batch, M, K) and (batch, K, N)")
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    code = _torch_dtype_code(A)
    batch, M, K = A.shape
    _, K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: {K} vs {K2}")
    lda, a_col = _layout(A[0], "A")
    ldb, b_col = _layout(B[0], "B")
    acc_dtype = torch.int32 if code == TCM_I8_I32 else torch.float32
    if accumulate and C is None:
        raise ValueError("accumulate needs C")
    if C is None:
        C = torch.empty((batch, M, N), dtype=out_dtype or acc_dtype, device=A.device)
    c_flags = {torch.float16: TCM_C_F16, torch.bfloat16: TCM_C_BF16}.get(C.dtype, 0)
    if c_flags and code == TCM_I8_I32:
        raise TypeError("int8 products have an int32 C")
    if (C.dtype != acc_dtype and not c_flags) or C.dim() != 3 or tuple(C.shape) != (batch, M, N) or \
            (N > 1 and C.stride(2) != 1):
        raise ValueError("C must be (batch, M, N) with row-major entries of the accumulator type, float16 or bfloat16")
    ldc = max(C.stride(1), N, 1)
    sb_bias = 0
    if bias is not None:
        if bias.dtype != acc_dtype or bias.shape[-1] < N or bias.stride(-1) != 1:
            raise ValueError("bias must be (N,) or (batch, N) of the accumulator type with contiguous rows")
        sb_bias = bias.stride(0) if bias.dim() == 2 else 0
    epi = (TCM_EPI_BIAS if bias is not None else 0) | (TCM_EPI_RELU if relu else 0) | (TCM_EPI_ACCUM if accumulate else 0)
    dtype = code | (TCM_A_COLMAJOR if a_col else 0) | (TCM_B_COLMAJOR if b_col else 0) | c_flags
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    st = tcm_gemm_batched(batch, M, N, K, A.data_ptr(), lda, A.stride(0), B.data_ptr(), ldb, B.stride(0), C.data_ptr(),
                          ldc, C.stride(0), dtype, bias.data_ptr() if bias is not None else None, sb_bias, epi, stream)
    if st != TCM_OK:
        raise TcmError(st, "tcm_gemm_batched")
    return C


def conv2d(x, f, bias=None, relu=False, padding=0, stride=1, dilation=1, out_dtype=None, stream=None):
    """y = relu?(conv2d(x, f) + bias) on the GPU via tcm_conv2d.

    x: (N, H, W, C) and f: (K, R, S, C) contiguous CUDA tensors of one type
    (float16, bfloat16, float32 or int8), channels last.  padding, stride,
    dilation: an int or an (h, w) pair.  bias: optional length-K vector of
    the accumulator type.  Returns y (N, P, Q, K) of the accumulator type
    (float32, int32 for int8) or `out_dtype` float16 / bfloat16."""
    import torch
    if x.dim() != 4 or f.dim() != 4 or x.shape[3] != f.shape[3]:
        raise ValueError("x must be (N, H, W, C) and f (K, R, S, C) with the same C")
    if x.dtype != f.dtype:
        raise TypeError("x and f must have the same dtype")
    if not (x.is_contiguous() and f.is_contiguous()):
        raise ValueError("x and f must be contiguous (channels last)")
    pair = lambda v: (v, v) if isinstance(v, int) else tuple(v)
    (ph, pw), (sh, sw), (dh, dw) = pair(padding), pair(stride), pair(dilation)
    code = _torch_dtype_code(x)
    N, H, W, C = x.shape
    K, R, S, _ = f.shape
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    acc_dtype = torch.int32 if code == TCM_I8_I32 else torch.float32
    y = torch.empty((N, max(P, 0), max(Q, 0), K), dtype=out_dtype or acc_dtype, device=x.device)
    c_flags = {torch.float16: TCM_C_F16, torch.bfloat16: TCM_C_BF16}.get(y.dtype, 0)
    if c_flags and code == TCM_I8_I32:
        raise TypeError("int8 convolutions have an int32 output")
    if bias is not None and (bias.dtype != acc_dtype or bias.numel() < K or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous length-K vector of the accumulator type")
    epi = (TCM_EPI_BIAS if bias is not None else 0) | (TCM_EPI_RELU if relu else 0)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = tcm_conv2d(N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw, x.data_ptr(), f.data_ptr(), y.data_ptr(),
                    code | c_flags, bias.data_ptr() if bias is not None else None, epi, stream)
    if st != TCM_OK:
        raise TcmError(st, "tcm_conv2d")
    return y


def gemm_grouped(As, Bs, Cs=None, biases=None, relu=False, accumulate=False, out_dtype=None, stream=None):
    """Cs[e] = relu?(As[e] @ Bs[e] + biases[e] [+ Cs[e]]) for every e, via tcm_gemm_grouped.

    As[e]: (M_e, K) and Bs[e]: (K, N_e) CUDA tensors of one type, row- or
    column-major views (one layout for all entries of a kind); Cs: optional
    row-major outputs; biases: optional list of length-N_e vectors.  Other
    arguments as gemm().  Returns the list of C tensors."""
    import torch
    if not As or len(As) != len(Bs) or len(As) > TCM_MAX_GROUP:
        raise ValueError(f"As and Bs: 1..{TCM_MAX_GROUP} matching entries")
    code = _torch_dtype_code(As[0])
    K = As[0].shape[1]
    acc_dtype = torch.int32 if code == TCM_I8_I32 else torch.float32
    if accumulate and Cs is None:
        raise ValueError("accumulate needs Cs")
    outs, ents, flags = [], [], set()
    for i, (A, B) in enumerate(zip(As, Bs)):
        if A.dtype != As[0].dtype or B.dtype != As[0].dtype:
            raise TypeError("every A and B must have the same dtype")
        M, Ka = A.shape
        Kb, N = B.shape
        if Ka != K or Kb != K:
            raise ValueError("every entry must share K")
        lda, a_col = _layout(A, "A")
        ldb, b_col = _layout(B, "B")
        C = Cs[i] if Cs is not None else torch.empty((M, N), dtype=out_dtype or acc_dtype, device=A.device)
        c_flags = {torch.float16: TCM_C_F16, torch.bfloat16: TCM_C_BF16}.get(C.dtype, 0)
        if (C.dtype != acc_dtype and not c_flags) or tuple(C.shape) != (M, N) or (N > 1 and C.stride(1) != 1):
            raise ValueError("each C must be a row-major (M, N) tensor of the accumulator type, float16 or bfloat16")
        bias = biases[i] if biases is not None else None
        if bias is not None and (bias.dtype != acc_dtype or bias.numel() < N or not bias.is_contiguous()):
            raise ValueError("each bias must be a contiguous length-N vector of the accumulator type")
        flags.add((a_col, b_col, c_flags))
        ents.append(GroupEntry(M, N, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), max(C.stride(0), N, 1),
                               bias.data_ptr() if bias is not None else None))
        outs.append(C)
    if len(flags) != 1:
        raise ValueError("every entry must have the same layouts and output type")
    a_col, b_col, c_flags = flags.pop()
    dtype = code | (TCM_A_COLMAJOR if a_col else 0) | (TCM_B_COLMAJOR if b_col else 0) | c_flags
    epi = (TCM_EPI_BIAS if biases is not None else 0) | (TCM_EPI_RELU if relu else 0) | (TCM_EPI_ACCUM if accumulate else 0)
    if stream is None:
        stream = torch.cuda.current_stream(As[0].device).cuda_stream
    st = tcm_gemm_grouped(ents, K, dtype, epi, stream)
    if st != TCM_OK:
        raise TcmError(st, "tcm_gemm_grouped")
    return outs
