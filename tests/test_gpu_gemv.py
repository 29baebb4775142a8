"""GPU parity of the split-k GEMV kernels (f16 and bf16, row-major A; B
row-major on the 4x4x4 kernel (at most 16 rows) or the 16x16x32 one (at
most 64 rows), or B column-major) against the oracle, on every entry.

Shapes cover every rows bucket (1, 2, 4, 8, 16, 32, 64 and sizes between),
column counts that end inside a workgroup's block of columns, K that ends
inside a chunk and inside a workgroup's k range, padded leading dimensions
(with non-finite values in A's padding past K), one k range (the epilogue in
the first kernel) and several (partials summed by the second kernel), and
the whole epilogue: bias, ReLU, C_in, 16-bit C.  Column-major B needs K a
multiple of 8 (16-byte pieces of k); the 16x16x32 row-major kernel needs
lda and ldb multiples of 8."""
import numpy as np
import pytest

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import check, run_tcm, say

pytestmark = pytest.mark.gpu
DT = [S.F16, S.BF16]
FORMS = ["b_row", "b_wide", "b_col"]


@pytest.fixture(params=FORMS)
def form(request):
    return request.param


def _ranges(p, splits, form):
    """k ranges the planner makes for an asked-for count: multiples of 64
    rows, at most 1024 (4x4x4 kernel), of 128 (16x16x32 row-major kernel)
    or of 256 rows (column-major B)."""
    q = -(-p.K // splits)
    if form == "b_col":
        kw = max(256, -(-q // 256) * 256)
    elif form == "b_wide":
        kw = max(128, -(-q // 128) * 128)
    else:
        kw = min(1024, -(-q // 64) * 64)
    return -(-p.K // kw)


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    T.tcm_set_option("gemv", 0)
    T.tcm_set_option("gemv_splits", 0)
    T.tcm_set_option("gemv_wide", 0)


def _run(p, splits=0, form=None, g=None):
    T.tcm_set_option("gemv", 2)
    T.tcm_set_option("gemv_splits", splits)
    T.tcm_set_option("gemv_wide", 2 if form == "b_wide" else 1)
    say(f"[case] gemv {form} {p.name} dtype={p.dtype} M={p.M} N={p.N} K={p.K} lda={p.LDA} ldb={p.LDB} ldc={p.LDC} "
        f"splits={splits} bias={p.bias} relu={p.relu} accum={p.accum} c={p.c_type} seed={p.seed}")
    if g is None:
        g = S.generate(p)
    C, plan = run_tcm(p, g)
    say(f"       plan: {plan}")
    assert "kernel=gemv" in plan
    assert ("mfma=16x16x32" in plan) == (form != "b_row")
    return g, C, plan


def _problem(form, dtype, M, N, K, **kw):
    if form == "b_wide":  # rows of A and B 16-byte aligned
        kw.setdefault("ldb", -(-N // 8) * 8)
        kw.setdefault("lda", -(-K // 8) * 8)
    return S.small_problem(dtype, M, N, K, b_col=(form == "b_col"), **kw)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 13, 16])
def test_gemv_rows_buckets(dtype, M, form):
    p = _problem(form, dtype, M, 1028, 1000, seed=200 + M, bias=True, relu=(M % 2 == 1))
    g, C, _ = _run(p, form=form)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("M", [17, 24, 32, 33, 47, 63, 64])
def test_gemv_wide_rows_buckets(dtype, M):
    """17 to 64 rows: the 16x16x32 kernel's 32- and 64-row buckets."""
    p = _problem("b_wide", dtype, M, 1000, 1064, seed=300 + M, bias=True, relu=(M % 2 == 0))
    g, C, _ = _run(p, form="b_wide")
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("splits", [1, 3, 7, 16])
def test_gemv_split_counts(dtype, splits, form):
    """One k range (the first kernel runs the epilogue) and several."""
    p = _problem(form, dtype, 6 if form != "b_wide" else 40, 772, 1480, seed=210 + splits, bias=True)
    g, C, plan = _run(p, splits, form)
    assert f"splits={_ranges(p, splits, form)}" in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("K", [1, 15, 64, 65, 200, 4097])
@pytest.mark.parametrize("form", ["b_row", "b_wide"])
def test_gemv_k_tails(dtype, K, form):
    M = 4 if form == "b_row" else 21
    p = _problem(form, dtype, M, 516, K, seed=220 + K % 97, bias=True, lda=-(-K // 8) * 8)
    g, C, _ = _run(p, form=form)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("form", ["b_row", "b_wide"])
def test_gemv_nonfinite_padding_past_k(dtype, form):
    """A's padding columns past K hold NaN and infinities: they meet zero rows
    of B (or nothing), and must not reach a sum."""
    K = 203
    p = _problem(form, dtype, 12 if form == "b_row" else 40, 264, K, seed=228, bias=True, lda=216, ldb=272)
    g = S.generate(p)
    A = g["A"].reshape(p.M, p.LDA).view(np.uint16)
    nan, inf = (0x7E00, 0x7C00) if dtype == S.F16 else (0x7FC0, 0x7F80)
    A[:, K::2] = nan
    A[:, K + 1::2] = inf
    g, C, _ = _run(p, form=form, g=g)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("K", [8, 56, 248, 264, 4104])
def test_gemv_k_tails_b_col(dtype, K):
    """Column-major B: K ending inside a 32-k step and inside a 256-row range."""
    p = S.small_problem(dtype, 5, 300, K, seed=225 + K % 97, bias=True, b_col=True)
    g, C, _ = _run(p, form="b_col")
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
def test_gemv_padded_leading_dimensions(dtype, form):
    """lda, ldb and ldc past the row lengths: the padding (NaN fill in C)
    is neither read into a sum nor written."""
    if form == "b_col":  # columns of B 344 elements apart, 336 of them used
        p = S.small_problem(dtype, 11, 261, 336, seed=231, lda=344, ldb=344, ldc=270, bias=True, relu=True, b_col=True)
    elif form == "b_wide":  # N = 261 ends inside a 16-byte piece of a row of B
        p = S.small_problem(dtype, 37, 261, 333, seed=232, lda=344, ldb=272, ldc=270, bias=True, relu=True)
    else:
        p = S.small_problem(dtype, 11, 260, 333, seed=230, lda=344, ldb=268, ldc=270, bias=True, relu=True)
    g, C, _ = _run(p, form=form)
    check(p, g, C)
    assert np.all(np.isnan(C[:, p.N:])), "padding columns of C were written"


@pytest.mark.parametrize("variant", [("acc", True), ("f16", False), ("f16", True), ("bf16", True)])
@pytest.mark.parametrize("splits", [1, 5])
def test_gemv_wider_epilogue(variant, splits, form):
    c_type, accum = variant
    dtype = S.BF16 if c_type == "bf16" else S.F16
    p = _problem(form, dtype, 7 if form != "b_wide" else 50, 516, 904, seed=240, bias=True, relu=True, c_type=c_type,
                 accum=accum)
    g, C, _ = _run(p, splits, form)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DT)
def test_gemv_deterministic(dtype, form):
    """The k ranges are added in a fixed order: repeated calls give the same bits."""
    p = _problem(form, dtype, 16 if form != "b_wide" else 64, 1024, 4096, seed=250)
    g, C1, _ = _run(p, form=form)
    _, C2, _ = _run(p, form=form, g=g)
    check(p, g, C1)
    assert np.array_equal(C1, C2)


@pytest.mark.parametrize("b_col", [False, True], ids=["b_row", "b_col"])
def test_gemv_is_a_tuning_candidate(b_col):
    """tcm_tune times the GEMV kernels beside the tile plans; the class entry
    it records (config 100: the 4x4x4 or column-major-B GEMV, 101: the
    16x16x32 row-major-B one, or a tile plan) is what the next call runs, and
    the result stays correct."""
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
        assert ("kernel=gemv" in plan) == (line[11] in ("100", "101")) == (best["kernel"] == 2)
        assert ("mfma=16x16x32" in plan and not b_col) == (line[11] == "101")
        check(p, g, C2)
    finally:
        T.tcm_tune_clear()
        assert T.tcm_tune_load(saved) == T.TCM_OK
