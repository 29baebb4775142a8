"""Seeded synthetic inputs for the GEMM workloads.

This module only draws numbers: it holds none of the product's arithmetic,
and both the CPU oracle side (tests) and the HIP side (tests, benchmark) take
their inputs from it.

Recipe (one numpy PCG64 generator per problem, ``np.random.default_rng(seed)``):
  * draw A, then B, then the bias, each in its *storage* order: a row-major
    M x K operand is drawn as an (M, K) array, a column-major one as the
    (K, M) array it is stored as (likewise B: (K, N) row-major, (N, K)
    column-major);
  * "uniform": ``rng.uniform(-1, 1)``; "normal": ``rng.standard_normal()``;
    both are drawn in float64, rounded to float32 (round-to-nearest-even),
    then to the operand type: float16 with numpy's RNE cast, bfloat16 with
    torch's RNE cast on the CPU, float32 as is;
  * int8 operands: ``rng.integers(-128, 127, endpoint=True)``; int32 bias:
    ``rng.integers(-2**20, 2**20, endpoint=True)``;
  * a batch of ``batch`` entries draws each operand for all entries at once,
    entry after entry (A: (batch, storage shape), then B -- one shared entry
    with ``b_shared`` --, then the bias (batch, N), then C_in);
  * with ``accum``, the initial-value tensor C_in (the M x ldc storage of C
    before the call, padding included) is drawn last: float problems
    ``rng.uniform(-1, 1)`` rounded like the operands to C's type (f32, f16
    or bf16), int8 problems int32 ``rng.integers(-2**20, 2**20, endpoint=True)``;
  * f16/bf16 operands are returned as uint16 bit patterns, f32 as float32,
    int8 as int8, bias as float32 or int32.
The sampled-entry list of a large problem comes from a second generator,
``default_rng(1000 + seed)``: 4096 rows then 4096 columns (duplicates kept),
followed by every entry of rows 0 and M - 1.

Convolutions (ConvProblem): one ``default_rng(seed)`` draws x as its
(N, H, W, C) storage array, then f as (K, R, S, C), then the bias (K,), with
the same distributions and roundings as the GEMM operands; their sampled
outputs come from ``default_rng(1000 + seed)`` as above, over the
N*P*Q x K output matrix (4096 pixels then 4096 channels, then every channel
of the first and last pixel).
"""
from dataclasses import dataclass, replace

import numpy as np

# element-type codes (the same numbering as the library's dtype argument)
F16, BF16, F32, I8 = 0, 1, 2, 3
DTYPE_NAMES = {F16: "f16", BF16: "bf16", F32: "f32", I8: "i8"}


@dataclass(frozen=True)
class Problem:
    name: str
    dtype: int
    M: int
    N: int
    K: int
    a_col: bool = False
    b_col: bool = False
    dist: str = "uniform"      # "uniform" | "normal" | "int"; "uniform12" | "ones" | "zeros" for power studies
    seed: int = 0
    bias: bool = False
    relu: bool = False
    lda: int = 0               # 0 = tight
    ldb: int = 0
    ldc: int = 0
    c_type: str = "acc"        # C storage: "acc" (f32 / int32), "f16", "bf16"
    accum: bool = False        # C's contents before the call seed the accumulator
    batch: int = 1             # entries of a strided batch (arrays gain a leading batch axis when > 1)
    b_shared: bool = False     # one B for every entry (batch stride 0)

    @property
    def LDA(self):
        return self.lda or (self.M if self.a_col else self.K)

    @property
    def LDB(self):
        return self.ldb or (self.K if self.b_col else self.N)

    @property
    def LDC(self):
        return self.ldc or self.N

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K * self.batch

    @property
    def in_bytes(self):
        return 1 if self.dtype == I8 else (4 if self.dtype == F32 else 2)

    @property
    def c_bytes(self):
        return 4 if self.c_type == "acc" else 2

    def entry(self, e=0):
        """One entry of a batch as a single problem (same shapes and storage)."""
        return replace(self, batch=1, b_shared=False, name=f"{self.name}[{e}]")

    @property
    def alg_bytes(self):
        """Bytes the product must move at least: A and B read once, C written once (and read
        once with accum), bias read once."""
        nb = 1 if self.b_shared else self.batch
        b = self.batch * self.M * self.K * self.in_bytes + nb * self.K * self.N * self.in_bytes
        b += self.batch * self.M * self.N * self.c_bytes * (2 if self.accum else 1)
        if self.bias:
            b += self.batch * self.N * 4
        return b


def _workloads():
    w = {}
    w["f16_512"] = Problem("f16_512", F16, 512, 512, 512, dist="uniform", seed=0)
    w["f32_2048"] = Problem("f32_2048", F32, 2048, 2048, 2048, dist="uniform", seed=1)
    w["f16_8192"] = Problem("f16_8192", F16, 8192, 8192, 8192, b_col=True, dist="normal", seed=2)
    w["bf16_8192"] = Problem("bf16_8192", BF16, 8192, 8192, 8192, b_col=True, dist="normal", seed=2)
    # the same product with B stored row-major (k rows of n contiguous)
    w["f16_8192_brow"] = Problem("f16_8192_brow", F16, 8192, 8192, 8192, dist="normal", seed=2)
    # A stored column-major (k columns of m contiguous: a transposed operand)
    w["f16_4096_acol"] = Problem("f16_4096_acol", F16, 4096, 4096, 4096, a_col=True, b_col=True, dist="normal", seed=9)
    for m in (1, 16, 64, 256):
        w[f"skinny_m{m}"] = Problem(f"skinny_m{m}", F16, m, 4096, 4096, dist="uniform", seed=3)
    w["sk_1536x1536x16384"] = Problem("sk_1536x1536x16384", F16, 1536, 1536, 16384, dist="uniform", seed=3)
    w["sk_3840x3840x4096"] = Problem("sk_3840x3840x4096", F16, 3840, 3840, 4096, dist="uniform", seed=3)
    w["i8_4096"] = Problem("i8_4096", I8, 4096, 4096, 4096, dist="int", seed=4, bias=True, relu=True)
    # wider epilogues: low-precision C, C's own contents as the initial value
    w["f16_8192_c16"] = Problem("f16_8192_c16", F16, 8192, 8192, 8192, b_col=True, dist="normal", seed=2, c_type="f16")
    w["bf16_4096_accum"] = Problem("bf16_4096_accum", BF16, 4096, 4096, 4096, b_col=True, dist="normal", seed=5,
                                   bias=True, relu=True, c_type="bf16", accum=True)
    w["i8_4096_accum"] = Problem("i8_4096_accum", I8, 4096, 4096, 4096, dist="int", seed=6, bias=True, relu=True,
                                 accum=True)
    w["skinny_m16_accum_c16"] = Problem("skinny_m16_accum_c16", F16, 16, 4096, 4096, dist="uniform", seed=7,
                                        c_type="f16", accum=True)
    # a strided batch of skinny products, each with its own B (experts of a mixture, a few rows each)
    w["batch8_m16_4096"] = Problem("batch8_m16_4096", F16, 16, 4096, 4096, dist="uniform", seed=8, batch=8)
    # a strided batch of two long-K products whose 72 tiles of 256x256 fill under a third of the CUs
    w["sk_batch2_1536x1536x16384"] = Problem("sk_batch2_1536x1536x16384", F16, 1536, 1536, 16384, dist="uniform",
                                             seed=10, batch=2)
    return w


WORKLOADS = _workloads()


def workload(name, **overrides):
    p = WORKLOADS[name]
    return replace(p, **overrides) if overrides else p


def _to_storage(x64, dtype):
    x32 = x64.astype(np.float32)
    if dtype == F32:
        return x32
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        import torch
        t = torch.from_numpy(x32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def _draw(rng, shape, dist, dtype):
    if dtype == I8:
        return rng.integers(-128, 127, size=shape, endpoint=True, dtype=np.int8)
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape)
    elif dist == "uniform12":  # [1, 2): the exponent never changes, only the mantissa toggles
        x = rng.uniform(1.0, 2.0, size=shape)
    elif dist == "ones":
        x = np.ones(shape)
    elif dist == "zeros":
        x = np.zeros(shape)
    else:
        raise ValueError(f"distribution {dist!r} needs an int8 problem")
    return _to_storage(x, dtype)


def _operand_shape(rows, cols, col_major, ld):
    """Storage array shape of a rows x cols logical operand (padded to ld)."""
    return (cols, ld) if col_major else (rows, ld)


C_TYPE_CODE = {"f16": F16, "bf16": BF16}   # storage codes of a low-precision C


def c_storage_dtype(p: Problem):
    """numpy storage type of C (uint16 bit patterns for f16 / bf16)."""
    if p.c_type != "acc":
        return np.uint16
    return np.int32 if p.dtype == I8 else np.float32


def generate(p: Problem):
    """Storage arrays {'A', 'B', 'bias', 'C_in'} of problem p (bias / C_in None when unused).

    With ld larger than the extent, the padding columns are drawn too (from
    the same stream, as part of the storage array)."""
    rng = np.random.default_rng(p.seed)
    lead = (p.batch,) if p.batch > 1 else ()
    A = _draw(rng, lead + _operand_shape(p.M, p.K, p.a_col, p.LDA), p.dist, p.dtype)
    B = _draw(rng, (lead if not p.b_shared else (1,) if lead else ()) + _operand_shape(p.K, p.N, p.b_col, p.LDB),
              p.dist, p.dtype)
    bias = None
    if p.bias:
        if p.dtype == I8:
            bias = rng.integers(-2 ** 20, 2 ** 20, size=lead + (p.N,), endpoint=True, dtype=np.int64).astype(np.int32)
        else:
            bias = rng.uniform(-1.0, 1.0, size=lead + (p.N,)).astype(np.float32)
    c_in = None
    if p.accum:
        shape = lead + (max(p.M, 1), p.LDC)
        if p.dtype == I8:
            c_in = rng.integers(-2 ** 20, 2 ** 20, size=shape, endpoint=True, dtype=np.int64).astype(np.int32)
        else:
            c_in = _to_storage(rng.uniform(-1.0, 1.0, size=shape), C_TYPE_CODE.get(p.c_type, F32))
    return {"A": A, "B": B, "bias": bias, "C_in": c_in}


def sample_entries(p: Problem, n=4096):
    """(ii, jj) int64 arrays: n seeded random entries plus all of rows 0 and M-1."""
    rng = np.random.default_rng(1000 + p.seed)
    ii = rng.integers(0, p.M, size=n, dtype=np.int64)
    jj = rng.integers(0, p.N, size=n, dtype=np.int64)
    cols = np.arange(p.N, dtype=np.int64)
    rows = [0] if p.M == 1 else [0, p.M - 1]
    ii = np.concatenate([ii] + [np.full(p.N, r, dtype=np.int64) for r in rows])
    jj = np.concatenate([jj] + [cols for _ in rows])
    return ii, jj


def small_problem(dtype, M, N, K, seed=0, a_col=False, b_col=False, bias=False, relu=False,
                  lda=0, ldb=0, ldc=0, dist=None, c_type="acc", accum=False, batch=1, b_shared=False):
    """An ad-hoc problem for parity cases (ragged shapes, padding, layouts)."""
    if dist is None:
        dist = "int" if dtype == I8 else "uniform"
    return Problem(f"{DTYPE_NAMES[dtype]}_{M}x{N}x{K}" + (f"_b{batch}" if batch > 1 else ""), dtype, M, N, K,
                   a_col=a_col, b_col=b_col, dist=dist, seed=seed, bias=bias, relu=relu, lda=lda, ldb=ldb, ldc=ldc,
                   c_type=c_type, accum=accum, batch=batch, b_shared=b_shared)


def entry_inputs(p: Problem, g, e):
    """The storage arrays of entry e of a batched problem's inputs g."""
    if p.batch == 1:
        return g
    return {"A": g["A"][e], "B": g["B"][0 if p.b_shared else e],
            "bias": None if g["bias"] is None else g["bias"][e],
            "C_in": None if g["C_in"] is None else g["C_in"][e]}


@dataclass(frozen=True)
class ConvProblem:
    """A 2-D convolution: NHWC input x, KRSC filter f, NPQK output y."""
    name: str
    dtype: int
    N: int
    H: int
    W: int
    C: int
    K: int
    R: int
    S: int
    pad: tuple = (0, 0)
    stride: tuple = (1, 1)
    dil: tuple = (1, 1)
    dist: str = "uniform"
    seed: int = 0
    bias: bool = False
    relu: bool = False
    c_type: str = "acc"

    @property
    def P(self):
        return (self.H + 2 * self.pad[0] - self.dil[0] * (self.R - 1) - 1) // self.stride[0] + 1

    @property
    def Q(self):
        return (self.W + 2 * self.pad[1] - self.dil[1] * (self.S - 1) - 1) // self.stride[1] + 1

    def gemm(self):
        """The implicit GEMM it is: M = N*P*Q pixels, N = K channels, K = R*S*C taps."""
        return Problem(self.name, self.dtype, self.N * self.P * self.Q, self.K, self.R * self.S * self.C, b_col=True,
                       dist=self.dist, seed=self.seed, bias=self.bias, relu=self.relu, c_type=self.c_type)

    @property
    def flops(self):
        return 2 * self.N * self.P * self.Q * self.K * self.R * self.S * self.C

    @property
    def alg_bytes(self):
        """Unique bytes: x and f read once, y written once (+ the bias)."""
        es = {F16: 2, BF16: 2, F32: 4, I8: 1}[self.dtype]
        b = (self.N * self.H * self.W * self.C + self.K * self.R * self.S * self.C) * es
        b += self.N * self.P * self.Q * self.K * self.gemm().c_bytes
        if self.bias:
            b += self.K * 4
        return b


def generate_conv(p: ConvProblem):
    """Storage arrays {'x', 'f', 'bias'} of convolution p (bias None when unused)."""
    rng = np.random.default_rng(p.seed)
    x = _draw(rng, (p.N, p.H, p.W, p.C), p.dist, p.dtype)
    f = _draw(rng, (p.K, p.R, p.S, p.C), p.dist, p.dtype)
    bias = None
    if p.bias:
        if p.dtype == I8:
            bias = rng.integers(-2 ** 20, 2 ** 20, size=(p.K,), endpoint=True, dtype=np.int64).astype(np.int32)
        else:
            bias = rng.uniform(-1.0, 1.0, size=(p.K,)).astype(np.float32)
    return {"x": x, "f": f, "bias": bias}


def sample_conv_entries(p: ConvProblem, n=4096):
    """(mm, kk) int64 arrays over the N*P*Q x K output: n seeded random
    positions plus every channel of the first and last pixel."""
    rng = np.random.default_rng(1000 + p.seed)
    M = p.N * p.P * p.Q
    mm = rng.integers(0, M, size=n, dtype=np.int64)
    kk = rng.integers(0, p.K, size=n, dtype=np.int64)
    ch = np.arange(p.K, dtype=np.int64)
    mm = np.concatenate([mm, np.zeros(p.K, dtype=np.int64), np.full(p.K, M - 1, dtype=np.int64)])
    return mm, np.concatenate([kk, ch, ch])


def small_conv(dtype, N, H, W, C, K, R, S, pad=(0, 0), stride=(1, 1), dil=(1, 1), seed=0, bias=False, relu=False,
               c_type="acc", dist=None):
    """An ad-hoc convolution for parity cases."""
    if dist is None:
        dist = "int" if dtype == I8 else "uniform"
    return ConvProblem(f"conv_{DTYPE_NAMES[dtype]}_{N}x{H}x{W}x{C}_k{K}r{R}s{S}", dtype, N, H, W, C, K, R, S,
                       pad=tuple(pad), stride=tuple(stride), dil=tuple(dil), dist=dist, seed=seed, bias=bias,
                       relu=relu, c_type=c_type)


def _conv_workloads():
    """3x3 convolutions with the shapes of a residual network's middle stages
    (channels-last, batch 128), bias + ReLU fused; float layers write their
    activations in f16 for the next layer, int8 layers int32."""
    w = {}
    w["conv_f16_28x28_c128"] = ConvProblem("conv_f16_28x28_c128", F16, 128, 28, 28, 128, 128, 3, 3, pad=(1, 1),
                                           dist="normal", seed=11, bias=True, relu=True, c_type="f16")
    w["conv_f16_14x14_c256"] = ConvProblem("conv_f16_14x14_c256", F16, 128, 14, 14, 256, 256, 3, 3, pad=(1, 1),
                                           dist="normal", seed=12, bias=True, relu=True, c_type="f16")
    w["conv_f16_56x56_s2_c128"] = ConvProblem("conv_f16_56x56_s2_c128", F16, 128, 56, 56, 128, 128, 3, 3, pad=(1, 1),
                                              stride=(2, 2), dist="normal", seed=13, bias=True, relu=True,
                                              c_type="f16")
    w["conv_i8_14x14_c256"] = ConvProblem("conv_i8_14x14_c256", I8, 128, 14, 14, 256, 256, 3, 3, pad=(1, 1),
                                          dist="int", seed=14, bias=True, relu=True)
    return w


CONV_WORKLOADS = _conv_workloads()


def _group_workloads():
    """A mixture-of-experts layer: eight experts of one 4096 x 4096 f16
    weight each (B row-major), a few to a hundred-odd token rows routed to
    each (one expert gets none), uniform values; one seed per expert."""
    rows = (3, 41, 17, 0, 96, 8, 150, 29)
    return {"moe8_4096": [Problem(f"moe8_4096_e{i}", F16, m, 4096, 4096, dist="uniform", seed=300 + i)
                          for i, m in enumerate(rows)]}


GROUP_WORKLOADS = _group_workloads()
