"""Seeded random parity sweep through tcm_gemm and tcm_gemm_batched: element
type, both layouts of A and B, shapes on and off the 16-byte piece grid (so
that the tiled kernel, the split-k GEMV and the generic kernel all take
part), padded leading dimensions, every epilogue flag, 16-bit outputs, and
now and then a forced tile config, mode or Stream-K grid (forced Stream-K
without a grid plans the eight-wave tile's equal shares in 40 of the 320
single cases); batches of 2 to 5 entries (B shared or not) at padded
strides.  Each case is drawn from its
own seed, printed before it touches the GPU, and compared with the oracle
on every entry (C's padding columns, and the gaps between batch entries,
must keep their fill).  A third set draws larger products (up to 2048 x
2048, K up to 8192), half of them on the eight-wave tile's equal shares."""
import numpy as np
import pytest

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import check, check_padding_untouched, run_tcm, say

pytestmark = pytest.mark.gpu

CE = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}  # elements per 16-byte piece
N_CASES = 320


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    for k, v in (("force_mode", 0), ("force_config", -1), ("sk_grid", 0), ("sk_fixup", 0), ("gemv", 0),
                 ("gemv_wide", 0), ("grid_shares", 0)):
        T.tcm_set_option(k, v)


def _dim(rng, lo, hi, ce, on_grid):
    x = int(rng.integers(lo, hi + 1))
    return max(ce, x // ce * ce) if on_grid else x


def draw(seed):
    """Case `seed`: the problem and the options it runs under."""
    rng = np.random.default_rng(9000 + seed)
    dtype = [S.F16, S.BF16, S.F32, S.I8][int(rng.integers(4))]
    ce = CE[dtype]
    on_grid = rng.random() < 0.75  # most cases can take the tiles
    a_col, b_col = bool(rng.integers(2)), bool(rng.integers(2))
    small_m = rng.random() < 0.3
    M = _dim(rng, 1, 40, ce, on_grid and a_col) if small_m else _dim(rng, 1, 600, ce, on_grid and a_col)
    N = _dim(rng, 1, 600, ce, on_grid and not b_col)
    K = _dim(rng, 1, 1100, ce, on_grid)
    pad = lambda: int(rng.integers(0, 3)) * ce if rng.random() < 0.5 else 0
    lda = (M if a_col else K) + pad()
    ldb = (K if b_col else N) + pad()
    ldc = N + pad()
    bias, relu = bool(rng.integers(2)), bool(rng.integers(2))
    c_type = "acc" if dtype in (S.I8, S.F32) else ["acc", "f16", "bf16"][int(rng.integers(3))]
    if c_type == "bf16" and dtype == S.F16:
        c_type = "f16"
    if c_type == "f16" and dtype == S.BF16:
        c_type = "bf16"
    accum = rng.random() < 0.25
    p = S.small_problem(dtype, M, N, K, seed=300 + seed, a_col=a_col, b_col=b_col, bias=bias, relu=relu, lda=lda,
                        ldb=ldb, ldc=ldc, c_type=c_type, accum=accum)
    opts = {}
    r = rng.random()
    if r < 0.2:
        opts["force_mode"] = int(rng.integers(1, 3))
    elif r < 0.35:
        opts["force_mode"] = 2
        opts["sk_grid"] = int(rng.integers(1, 400))
        opts["sk_fixup"] = int(rng.integers(0, 3))
    elif r < 0.45:
        opts["force_config"] = int(rng.integers(0, T.tcm_config_count()))
    return p, opts


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    p, opts = draw(seed)
    for k, v in opts.items():
        assert T.tcm_set_option(k, v) == T.TCM_OK
    say(f"[case] random {seed}: {p.name} dtype={p.dtype} M={p.M} N={p.N} K={p.K} a_col={p.a_col} b_col={p.b_col} "
        f"lda={p.LDA} ldb={p.LDB} ldc={p.LDC} bias={p.bias} relu={p.relu} c={p.c_type} accum={p.accum} opts={opts}")
    g = S.generate(p)
    C, plan = run_tcm(p, g)
    say(f"       plan: {plan}")
    check(p, g, C)
    if p.c_type == "acc" and not p.accum:
        check_padding_untouched(p, C, -7 if p.dtype == S.I8 else float("nan"))


def test_random_cases_reach_every_kernel():
    """The drawn set plans the tiled kernel (both A layouts), the split-k
    GEMV and the generic kernel (checked on the CPU with tcm_plan), and among
    the tiled plans at least ten equal-shares ones (forced Stream-K without a
    grid on the eight-wave tile)."""
    kinds = set()
    shares = 0
    for seed in range(N_CASES):
        p, opts = draw(seed)
        code = p.dtype | (T.TCM_A_COLMAJOR if p.a_col else 0) | (T.TCM_B_COLMAJOR if p.b_col else 0)
        code |= {"acc": 0, "f16": T.TCM_C_F16, "bf16": T.TCM_C_BF16}[p.c_type]
        for k, v in opts.items():
            T.tcm_set_option(k, v)
        try:
            q = T.tcm_plan(p.M, p.N, p.K, p.LDA, p.LDB, p.LDC, code)
        finally:
            for k, v in (("force_mode", 0), ("force_config", -1), ("sk_grid", 0), ("sk_fixup", 0)):
                T.tcm_set_option(k, v)
        kinds.add((q["kernel"], p.a_col if q["kernel"] == 1 else None))
        shares += q["split"] > 1
    assert {(0, None), (1, False), (1, True), (2, None)} <= kinds, kinds
    assert shares >= 10, shares


N_BATCHED = 64


def draw_batched(seed):
    """Batched case `seed`: a drawn problem of a few entries (own or shared B)
    and the entries' padding (16-byte multiples keep the tiles eligible)."""
    p, opts = draw(5000 + seed)
    rng = np.random.default_rng(19000 + seed)
    batch = int(rng.integers(2, 6))
    b_shared = rng.random() < 0.25
    from dataclasses import replace
    p = replace(p, batch=batch, b_shared=b_shared, M=min(p.M, 300), K=min(p.K, 600))
    if p.a_col:
        p = replace(p, lda=max(p.LDA, p.M) if p.lda else 0)
    else:
        p = replace(p, lda=max(p.LDA, p.K) if p.lda else 0)
    if p.b_col:
        p = replace(p, ldb=max(p.LDB, p.K) if p.ldb else 0)
    pads = tuple(int(x) for x in rng.integers(0, 4, 3) * 64)
    return p, opts, pads


@pytest.mark.parametrize("seed", range(N_BATCHED))
def test_random_batched_case(seed):
    from test_gpu_batched import check_batch, run_batched
    p, opts, pads = draw_batched(seed)
    for k, v in opts.items():
        assert T.tcm_set_option(k, v) == T.TCM_OK
    say(f"[case] random batched {seed}: {p.name} dtype={p.dtype} batch={p.batch} b_shared={p.b_shared} M={p.M} N={p.N} "
        f"K={p.K} a_col={p.a_col} b_col={p.b_col} lda={p.LDA} ldb={p.LDB} ldc={p.LDC} bias={p.bias} relu={p.relu} "
        f"c={p.c_type} accum={p.accum} pads={pads} opts={opts}")
    g = S.generate(p)
    C, plan = run_batched(p, g, pads=pads)
    say(f"       plan: {plan}")
    check_batch(p, g, C)


N_LARGE = 40


def draw_large(seed):
    """Larger case `seed`: 64 to 2048 rows and columns (whole 16-byte pieces),
    K from 256 to 8192, either layout of A and B, padded leading dimensions,
    a batch of 2-3 now and then (smaller entries), any epilogue; half of the
    cases forced onto the eight-wave tile's Stream-K (its equal shares,
    sometimes with a given share count)."""
    rng = np.random.default_rng(77000 + seed)
    dtype = [S.F16, S.BF16, S.F32, S.I8][int(rng.integers(4))]
    ce = CE[dtype]
    a_col, b_col = bool(rng.integers(2)), bool(rng.integers(2))
    M = int(rng.integers(64, 2049)) // ce * ce
    N = int(rng.integers(64, 2049)) // ce * ce
    K = int(rng.integers(256, 8193)) // ce * ce
    batch = 1 if rng.random() < 0.7 else int(rng.integers(2, 4))
    if batch > 1:
        M, N, K = min(M, 768), min(N, 768), min(K, 4096)
    bias, relu = bool(rng.integers(2)), bool(rng.integers(2))
    c_type = "acc" if dtype in (S.I8, S.F32) else ["acc", "f16", "bf16"][int(rng.integers(3))]
    if c_type == "bf16" and dtype == S.F16:
        c_type = "f16"
    if c_type == "f16" and dtype == S.BF16:
        c_type = "bf16"
    accum = rng.random() < 0.25
    pad = lambda: int(rng.integers(0, 3)) * ce
    p = S.small_problem(dtype, M, N, K, seed=900 + seed, a_col=a_col, b_col=b_col, bias=bias, relu=relu,
                        lda=(M if a_col else K) + pad(), ldb=(K if b_col else N) + pad(), ldc=N + pad(), c_type=c_type,
                        accum=accum)
    if batch > 1:
        from dataclasses import replace
        p = replace(p, batch=batch)
    opts = {}
    if rng.random() < 0.5:
        opts = {"force_config": 0, "force_mode": 2}
        if rng.random() < 0.5:
            opts["grid_shares"] = int(rng.integers(2, 9))
    return p, opts


@pytest.mark.parametrize("seed", range(N_LARGE))
def test_random_large_case(seed):
    from test_gpu_batched import check_batch, run_batched
    p, opts = draw_large(seed)
    for k, v in opts.items():
        assert T.tcm_set_option(k, v) == T.TCM_OK
    say(f"[case] random large {seed}: {p.name} dtype={p.dtype} batch={p.batch} M={p.M} N={p.N} K={p.K} a_col={p.a_col} "
        f"b_col={p.b_col} lda={p.LDA} ldb={p.LDB} ldc={p.LDC} bias={p.bias} relu={p.relu} c={p.c_type} accum={p.accum} "
        f"opts={opts}")
    g = S.generate(p)
    if p.batch > 1:
        C, plan = run_batched(p, g)
        say(f"       plan: {plan}")
        check_batch(p, g, C)
    else:
        C, plan = run_tcm(p, g)
        say(f"       plan: {plan}")
        if p.M * p.N * p.K > 2e9:  # sampled entries, computed one by one by the oracle
            ii, jj = S.sample_entries(p)
            check(p, g, C, ii, jj)
        else:
            check(p, g, C)
