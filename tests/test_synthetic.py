"""The seeded input generator: determinism, shapes, ranges and sampled entries."""
import numpy as np
import pytest

import synthetic as S


def test_workloads_listed():
    names = set(S.WORKLOADS)
    assert {"f16_512", "f32_2048", "f16_8192", "bf16_8192", "i8_4096", "skinny_m1", "skinny_m16",
            "skinny_m64", "skinny_m256", "sk_1536x1536x16384", "sk_3840x3840x4096"} <= names
    p = S.workload("f16_8192")
    assert (p.M, p.N, p.K, p.a_col, p.b_col, p.dist, p.seed) == (8192, 8192, 8192, False, True, "normal", 2)
    p = S.workload("i8_4096")
    assert p.bias and p.relu and p.dtype == S.I8 and p.seed == 4


@pytest.mark.parametrize("dtype", [S.F16, S.BF16, S.F32, S.I8])
def test_deterministic_and_typed(dtype):
    p = S.small_problem(dtype, 37, 29, 53, seed=5, bias=True, b_col=True)
    g1, g2 = S.generate(p), S.generate(p)
    for k in ("A", "B", "bias"):
        assert np.array_equal(g1[k], g2[k])
    want = {S.F16: np.uint16, S.BF16: np.uint16, S.F32: np.float32, S.I8: np.int8}[dtype]
    assert g1["A"].dtype == want and g1["A"].shape == (37, 53)
    assert g1["B"].shape == (29, 53)          # column-major B is stored as N x K
    assert g1["bias"].dtype == (np.int32 if dtype == S.I8 else np.float32)
    g3 = S.generate(S.small_problem(dtype, 37, 29, 53, seed=6, bias=True, b_col=True))
    assert not np.array_equal(g1["A"], g3["A"])


def test_ranges():
    g = S.generate(S.small_problem(S.I8, 300, 300, 300, seed=4, bias=True))
    assert g["A"].min() == -128 and g["A"].max() == 127
    assert g["bias"].min() >= -2 ** 20 and g["bias"].max() <= 2 ** 20
    g = S.generate(S.small_problem(S.F16, 200, 100, 100, seed=0))
    a = g["A"].view(np.float16).astype(np.float64)
    assert a.min() >= -1 and a.max() <= 1 and abs(a.mean()) < 0.02


def test_padding_is_drawn():
    p = S.small_problem(S.F32, 10, 12, 14, lda=20, ldb=16)
    g = S.generate(p)
    assert g["A"].shape == (10, 20) and g["B"].shape == (14, 16)


def test_sample_entries():
    p = S.workload("f16_8192")
    ii, jj = S.sample_entries(p)
    assert ii.shape == jj.shape == (4096 + 2 * 8192,)
    assert ii.min() >= 0 and ii.max() < p.M and jj.min() >= 0 and jj.max() < p.N
    assert np.all(ii[4096:4096 + 8192] == 0) and np.all(ii[4096 + 8192:] == p.M - 1)
    ii2, jj2 = S.sample_entries(p)
    assert np.array_equal(ii, ii2) and np.array_equal(jj, jj2)


@pytest.mark.parametrize("dist,lo,hi", [("uniform12", 1.0, 2.0), ("ones", 1.0, 1.0), ("zeros", 0.0, 0.0)])
def test_power_study_distributions(dist, lo, hi):
    """The extra value distributions (used to show the clock's dependence on the data) stay in range."""
    for dt in (S.F16, S.BF16, S.F32):
        p = S.small_problem(dt, 8, 16, 32, dist=dist)
        g = S.generate(p)
        for x in (g["A"], g["B"]):
            if dt == S.F16:
                v = x.view(np.float16).astype(np.float64)
            elif dt == S.BF16:
                v = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            else:
                v = x.astype(np.float64)
            assert v.min() >= lo and v.max() <= hi
