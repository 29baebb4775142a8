"""GPU parity of the split-k GEMV kernels (products of at most 16 rows, f16
and bf16, row-major A; B row-major or column-major) against the oracle, on
every entry.

Shapes cover every rows bucket (1, 2, 4, 8, 16 and sizes between), column
counts that end inside a workgroup's block of columns, K that ends inside a
chunk and inside a workgroup's k range, padded leading dimensions, one k
range (the epilogue in the first kernel) and several (partials summed by
the second kernel), and the whole epilogue: bias, ReLU, C_in, 16-bit C.
Column-major B needs K a multiple of 8 (16-byte pieces of k)."""
import numpy as np
import pytest

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import check, run_tcm, say

pytestmark = pytest.mark.gpu
DT = [S.F16, S.BF16]


@pytest.fixture(params=[False, True], ids=["b_row", "b_col"])
def b_col(request):
    return request.param


def _ranges(p, splits):
    """k ranges the planner makes for an asked-for count: multiples of 64
    rows, at most 1024 (row-major B), or of 256 rows (column-major B)."""
    q = -(-p.K // splits)
    kw = max(256, -(-q // 256) * 256) if p.b_col else min(1024, -(-q // 64) * 64)
    return -(-p.K // kw)


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    T.tcm_set_option("gemv", 0)
    T.tcm_set_option("gemv_splits", 0)


def _run(p, splits=0):
    T.tcm_set_option("gemv", 2)
    T.tcm_set_option("gemv_splits", splits)
    say(f"[case] gemv {p.name} dtype={p.dtype} M={p.M} N={p.N} K={p.K} lda={p.LDA} ldb={p.LDB} ldc={p.LDC} "
        f"splits={splits} bias={p.bias} relu={p.relu} accum={p.accum} c={p.c_type} seed={p.seed}")
    g = S.generate(p)
    C, plan = run_tcm(p, g)
    say(f"       plan: {plan}")
    assert "kernel=gemv" in plan
    return g, C, plan


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 13, 16])
def test_gemv_rows_buckets(dtype, M, b_col):
    p = S.small_problem(dtype, M, 1028, 1000, seed=200 + M, bias=True, relu=(M % 2 == 1), b_col=b_col)
    g, C, _ = _run(p)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("splits", [1, 3, 7, 16])
def test_gemv_split_counts(dtype, splits, b_col):
    """One k range (the first kernel runs the epilogue) and several."""
    p = S.small_problem(dtype, 6, 772, 1480, seed=210 + splits, bias=True, b_col=b_col)
    g, C, plan = _run(p, splits)
    assert f"splits={_ranges(p, splits)}" in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("K", [1, 15, 64, 65, 200, 4097])
def test_gemv_k_tails(dtype, K):
    p = S.small_problem(dtype, 4, 516, K, seed=220 + K % 97, bias=True, lda=-(-K // 8) * 8)
    g, C, _ = _run(p)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("K", [8, 56, 248, 264, 4104])
def test_gemv_k_tails_b_col(dtype, K):
    """Column-major B: K ending inside a 32-k step and inside a 256-row range."""
    p = S.small_problem(dtype, 5, 300, K, seed=225 + K % 97, bias=True, b_col=True)
    g, C, _ = _run(p)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
def test_gemv_padded_leading_dimensions(dtype, b_col):
    """lda, ldb and ldc past the row lengths: the padding (NaN fill in C)
    is neither read into a sum nor written."""
    if b_col:  # columns of B 344 elements apart, 336 of them used
        p = S.small_problem(dtype, 11, 261, 336, seed=231, lda=344, ldb=344, ldc=270, bias=True, relu=True, b_col=True)
    else:
        p = S.small_problem(dtype, 11, 260, 333, seed=230, lda=344, ldb=268, ldc=270, bias=True, relu=True)
    g, C, _ = _run(p)
    check(p, g, C)
    assert np.all(np.isnan(C[:, p.N:])), "padding columns of C were written"


@pytest.mark.parametrize("variant", [("acc", True), ("f16", False), ("f16", True), ("bf16", True)])
@pytest.mark.parametrize("splits", [1, 5])
def test_gemv_wider_epilogue(variant, splits, b_col):
    c_type, accum = variant
    dtype = S.BF16 if c_type == "bf16" else S.F16
    p = S.small_problem(dtype, 7, 516, 904, seed=240, bias=True, relu=True, c_type=c_type, accum=accum, b_col=b_col)
    g, C, _ = _run(p, splits)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
def test_gemv_deterministic(dtype, b_col):
    """The k ranges are added in a fixed order: repeated calls give the same bits."""
    p = S.small_problem(dtype, 16, 1024, 4096, seed=250, b_col=b_col)
    g, C1, _ = _run(p)
    _, C2, _ = _run(p)
    check(p, g, C1)
    assert np.array_equal(C1, C2)


def test_gemv_is_a_tuning_candidate(b_col):
    """tcm_tune times the GEMV beside the tile plans; the class entry it
    records (config 100: the GEMV, or a tile plan) is what the next call runs,
    and the result stays correct."""
    from gpu_util import to_device
    import torch
    saved = T.tcm_tune_table()
    T.tcm_tune_clear()
    try:
        p = S.small_problem(S.F16, 2, 4096, 4096, seed=260, bias=True, b_col=b_col)
        g = S.generate(p)
        ka, pa = to_device(g["A"], p.dtype)
        kb, pb = to_device(g["B"], p.dtype)
        kbias = torch.from_numpy(g["bias"].copy()).cuda()
        C = torch.empty((p.M, p.LDC), dtype=torch.float32, device="cuda")
        say(f"[case] tune {p.name}")
        code = p.dtype | (T.TCM_B_COLMAJOR if b_col else 0)
        st, best = T.tcm_tune(p.M, p.N, p.K, pa, p.LDA, pb, p.LDB, C.data_ptr(), p.LDC, code, kbias.data_ptr(),
                              T.TCM_EPI_BIAS, 5, torch.cuda.current_stream().cuda_stream)
        assert st == T.TCM_OK
        line = T.tcm_tune_table().split()
        say(f"       tuned: {' '.join(line)}")
        C2, plan = run_tcm(p, g)
        say(f"       plan: {plan}")
        assert " tuned=" in plan
        assert ("kernel=gemv" in plan) == (line[11] == "100") == (best["kernel"] == 2)
        check(p, g, C2)
    finally:
        T.tcm_tune_clear()
        assert T.tcm_tune_load(saved) == T.TCM_OK
