"""Parity at the full workload sizes, in the launch configuration the benchmark
uses (the planner's choice), plus forced data-parallel / Stream-K for the
split-k sweep.  Small products are compared on every entry; the large ones
on 4096 seeded entries plus all of rows 0 and M-1, computed one by one by
the oracle."""
import numpy as np
import pytest

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import FULL_SIZE_GUARD, check, run_tcm, say

pytestmark = pytest.mark.gpu

FULL = {"f16_512", "f32_2048", "skinny_m1", "skinny_m16", "skinny_m64", "skinny_m256"}
SPLITK = ["skinny_m1", "skinny_m16", "skinny_m64", "skinny_m256", "sk_1536x1536x16384", "sk_3840x3840x4096",
          "batch8_m16_4096", "sk_batch2_1536x1536x16384"]


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    T.tcm_set_option("force_mode", 0)


def _check_workload(name, mode):
    p = S.workload(name)
    T.tcm_set_option("force_mode", mode)
    say(f"[case] workload {name} M={p.M} N={p.N} K={p.K} dtype={p.dtype} b_col={p.b_col} batch={p.batch} "
        f"seed={p.seed} force_mode={mode}")
    g = S.generate(p)
    if p.batch > 1:
        from test_gpu_batched import check_batch, run_batched
        C, plan = run_batched(p, g)
        say(f"       plan: {plan}")
        err = check_batch(p, g, C)  # every entry of every product
    else:
        C, plan = run_tcm(p, g)
        say(f"       plan: {plan}")
        if name in FULL:
            err = check(p, g, C)
        else:
            ii, jj = S.sample_entries(p)
            err = check(p, g, C, ii, jj)
    say(f"       normalised error {err:.3e}")
    if p.dtype in (S.F16, S.BF16):
        assert err <= FULL_SIZE_GUARD, f"{name}: normalised error {err:.3e} above the regression guard {FULL_SIZE_GUARD:.0e}"
    return C, plan


@pytest.mark.parametrize("name", list(S.WORKLOADS))
def test_workload_as_benchmarked(name):
    _check_workload(name, 0)


@pytest.mark.parametrize("name", SPLITK)
@pytest.mark.parametrize("mode", [1, 2])
def test_splitk_sweep_both_modes(name, mode):
    C, plan = _check_workload(name, mode)
    assert ("mode=dp" if mode == 1 else "mode=streamk") in plan


def test_equal_shares_full_size():
    """1536^2 x 16384 as equal shares of the eight-wave 256x256 tile: 36 tiles
    in 7 shares of 36-37 K-steps on 252 workgroups, sampled entries."""
    T.tcm_set_option("force_config", 0)
    try:
        C, plan = _check_workload("sk_1536x1536x16384", 2)
    finally:
        T.tcm_set_option("force_config", -1)
    assert "config=0" in plan and "split=7" in plan and "grid=252" in plan


def test_int8_full_rows_bit_exact():
    """int8 4096^3 with bias + ReLU: 64 complete rows bit-exact (plus the sampled entries above)."""
    p = S.workload("i8_4096")
    say(f"[case] i8_4096 64 full rows")
    g = S.generate(p)
    C, plan = run_tcm(p, g)
    rows = np.arange(0, p.M, p.M // 64)
    ii = np.repeat(rows, p.N)
    jj = np.tile(np.arange(p.N), rows.size)
    check(p, g, C, ii, jj)


@pytest.mark.parametrize("name", list(S.WORKLOADS))
def test_host_plan_query_matches_launch(name):
    """tcm_plan / tcm_plan_batched (no launch) report the kernel, config, mode and grid the call then launches."""
    p = S.workload(name)
    code = p.dtype | (T.TCM_A_COLMAJOR if p.a_col else 0) | (T.TCM_B_COLMAJOR if p.b_col else 0)
    code |= {"acc": 0, "f16": T.TCM_C_F16, "bf16": T.TCM_C_BF16}[p.c_type]
    epi = (T.TCM_EPI_BIAS if p.bias else 0) | (T.TCM_EPI_RELU if p.relu else 0) | (T.TCM_EPI_ACCUM if p.accum else 0)
    q = T.tcm_plan_batched(p.batch, p.M, p.N, p.K, p.LDA, p.LDB, p.LDC, code, epi, True)
    say(f"[case] plan query {name}: {q}")
    g = S.generate(p)
    if p.batch > 1:
        from test_gpu_batched import run_batched
        _, plan = run_batched(p, g)
    else:
        _, plan = run_tcm(p, g)
    f = dict(kv.split("=", 1) for kv in plan.split() if "=" in kv)
    if q["kernel"] == 2:  # the split-k GEMV
        assert f["kernel"] == "gemv" and int(f["grid"]) == q["grid"]
        assert int(f["splits"]) == q["iters_per_tile"] and int(f["k_per_wg"]) == q["bk"] and int(f["rows"]) == q["bm"]
        return
    assert f["kernel"] == ("tile" if q["kernel"] == 1 else "generic")
    assert int(f["config"]) == q["config"]
    assert f["mode"] == ("dp" if q["mode"] == 1 else "streamk")
    assert int(f["grid"]) == q["grid"]
    assert int(f["dp_tiles"]) == q["dp_tiles"] and int(f["sk_tiles"]) == q["sk_tiles"]
