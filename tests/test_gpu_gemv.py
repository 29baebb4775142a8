"""GPU parity of the split-k GEMV kernel (products of at most 16 rows, f16
and bf16, row-major A and B) against the oracle, on every entry.

Shapes cover every rows bucket (1, 2, 4, 8, 16 and sizes between), column
counts that end inside a 256-column block, K that ends inside a 16-row
chunk and inside a workgroup's k range, padded leading dimensions, one k
range (the epilogue in the first kernel) and several (partials summed by
the second kernel), and the whole epilogue: bias, ReLU, C_in, 16-bit C."""
import numpy as np
import pytest

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import check, run_tcm, say

pytestmark = pytest.mark.gpu
DT = [S.F16, S.BF16]


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
def test_gemv_rows_buckets(dtype, M):
    p = S.small_problem(dtype, M, 1028, 1000, seed=200 + M, bias=True, relu=(M % 2 == 1))
    g, C, _ = _run(p)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("splits", [1, 3, 7, 16])
def test_gemv_split_counts(dtype, splits):
    """One k range (the first kernel runs the epilogue) and several."""
    p = S.small_problem(dtype, 6, 772, 1480, seed=210 + splits, bias=True)
    g, C, plan = _run(p, splits)
    # the k range per workgroup is a multiple of 64 rows and at most 1024
    kw = min(1024, -(-(-(-p.K // splits)) // 64) * 64)
    assert f"splits={-(-p.K // kw)}" in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("K", [1, 15, 64, 65, 200, 4097])
def test_gemv_k_tails(dtype, K):
    p = S.small_problem(dtype, 4, 516, K, seed=220 + K % 97, bias=True, lda=-(-K // 8) * 8)
    g, C, _ = _run(p)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
def test_gemv_padded_leading_dimensions(dtype):
    """lda, ldb and ldc past the row lengths: the padding (NaN fill in C)
    is neither read into a sum nor written."""
    p = S.small_problem(dtype, 11, 260, 333, seed=230, lda=344, ldb=268, ldc=270, bias=True, relu=True)
    g, C, _ = _run(p)
    check(p, g, C)
    assert np.all(np.isnan(C[:, p.N:])), "padding columns of C were written"


@pytest.mark.parametrize("variant", [("acc", True), ("f16", False), ("f16", True), ("bf16", True)])
@pytest.mark.parametrize("splits", [1, 5])
def test_gemv_wider_epilogue(variant, splits):
    c_type, accum = variant
    dtype = S.BF16 if c_type == "bf16" else S.F16
    p = S.small_problem(dtype, 7, 516, 900, seed=240, bias=True, relu=True, c_type=c_type, accum=accum, lda=904)
    g, C, _ = _run(p, splits)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
def test_gemv_deterministic(dtype):
    """The k ranges are added in a fixed order: repeated calls give the same bits."""
    p = S.small_problem(dtype, 16, 1024, 4096, seed=250)
    g, C1, _ = _run(p)
    _, C2, _ = _run(p)
    check(p, g, C1)
    assert np.array_equal(C1, C2)


def test_gemv_is_a_tuning_candidate():
    """tcm_tune times the GEMV beside the tile plans; the class entry it
    records (config 100: the GEMV, or a tile plan) is what the next call runs,
    and the result stays correct."""
    from gpu_util import to_device
    import torch
    saved = T.tcm_tune_table()
    T.tcm_tune_clear()
    try:
        p = S.small_problem(S.F16, 2, 4096, 4096, seed=260, bias=True)
        g = S.generate(p)
        ka, pa = to_device(g["A"], p.dtype)
        kb, pb = to_device(g["B"], p.dtype)
        kbias = torch.from_numpy(g["bias"].copy()).cuda()
        C = torch.empty((p.M, p.LDC), dtype=torch.float32, device="cuda")
        say(f"[case] tune {p.name}")
        st, best = T.tcm_tune(p.M, p.N, p.K, pa, p.LDA, pb, p.LDB, C.data_ptr(), p.LDC, p.dtype, kbias.data_ptr(),
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
