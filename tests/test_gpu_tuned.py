"""GPU: calls whose class the shipped tuning table holds run the table's
plan (the plan text names the class it came from) and match the oracle.

Cases: the headline class (f16 8192^3, B column-major: data-parallel
256x256 tiles with the table's group rows; sampled entries), a small
product the cost model used to send to Stream-K (1024^3: data-parallel
64x64 tiles in the table; every entry), the long-K product (1536^2 x 16384:
Stream-K on 128x128 units in equal shares; sampled entries), and a shape
the table does not hold but whose nearest class (within one half octave)
it does (every entry)."""
import pytest

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import FULL_SIZE_GUARD, check, run_tcm, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _table_on():
    T.tcm_set_option("tuned", 1)
    yield


def _entry(M, N, K, code, epi=0):
    q = T.tcm_plan(M, N, K, K, (K if code & T.TCM_B_COLMAJOR else N), N, code, epi, True)
    return q


@pytest.mark.parametrize("name,full", [("f16_8192", False), ("sk_1536x1536x16384", False)])
def test_shipped_entry_used_for_workload(name, full):
    p = S.workload(name)
    code = p.dtype | (T.TCM_B_COLMAJOR if p.b_col else 0)
    q = _entry(p.M, p.N, p.K, code)
    say(f"[case] shipped entry for {name}: {q}")
    g = S.generate(p)
    C, plan = run_tcm(p, g)
    say(f"       plan: {plan}")
    assert " tuned=" in plan
    assert f"config={q['config']} " in plan and f"grid={q['grid']} " in plan
    ii, jj = S.sample_entries(p)
    err = check(p, g, C, ii, jj)
    assert err <= FULL_SIZE_GUARD


def test_shipped_entry_fixes_the_small_product():
    p = S.small_problem(S.F16, 1024, 1024, 1024, seed=120, bias=True, relu=True)
    g = S.generate(p)
    say(f"[case] shipped entry for {p.name} with bias + ReLU (another class: the nearest is not used across epilogues)")
    C, plan = run_tcm(p, g)
    say(f"       plan: {plan}")
    check(p, g, C)
    p = S.small_problem(S.F16, 1024, 1024, 1024, seed=121)
    g = S.generate(p)
    say(f"[case] shipped entry for {p.name}")
    C, plan = run_tcm(p, g)
    say(f"       plan: {plan}")
    assert " tuned=20,20,20" in plan and "mode=dp" in plan
    check(p, g, C)


def test_nearest_shipped_class():
    # 896 x 896 x 1024 is class (19, 19, 20): the nearest held class is 1024^3's
    # (20, 20, 20); 512^3's (18, 18, 18) is two half octaves away in K
    p = S.small_problem(S.F16, 896, 896, 1024, seed=122)
    g = S.generate(p)
    say(f"[case] nearest shipped class for {p.name}")
    C, plan = run_tcm(p, g)
    say(f"       plan: {plan}")
    assert " tuned=20,20,20" in plan
    check(p, g, C)
