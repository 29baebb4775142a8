"""The tuning table shipped with the library (tensor_core_mixed_amd/tuned/mi355x.txt):
well formed, loaded by the library on its own, and used by the planner for
the classes it holds (CPU only: planning needs no device)."""
import os
import subprocess
import sys

import pytest

import tensor_core_mixed_amd as T

SHIPPED = os.path.join(os.path.dirname(T.__file__), "tuned", "mi355x.txt")


def _entries():
    out = []
    for line in open(SHIPPED):
        if line.strip() and not line.startswith("#"):
            f = line.split()
            assert f[0] == "tcm-tune-2" and len(f) == 21, line
            out.append([int(x) for x in f[1:17]] + [float(f[17])] + [int(x) for x in f[18:21]])
    return out


@pytest.fixture(autouse=True)
def _shipped_table_loaded():
    """Each test starts from exactly the shipped table (other tests may have
    changed the process's table) and leaves the table as it found it."""
    before = T.tcm_tune_table()
    T.tcm_tune_clear()
    assert T.tcm_tune_load(open(SHIPPED).read()) == T.TCM_OK
    T.tcm_set_option("tuned", 1)
    yield
    T.tcm_tune_clear()
    assert T.tcm_tune_load(before) == T.TCM_OK


def test_shipped_table_is_well_formed_and_loads():
    assert os.path.exists(SHIPPED)
    text = open(SHIPPED).read()
    lines = [l for l in text.splitlines() if l.strip() and not l.startswith("#")]
    assert sorted(T.tcm_tune_table().splitlines()) == sorted(lines)
    # a fresh process loads the same file by itself, before its first plan
    code = ("import sys; sys.path.insert(0, %r); import tensor_core_mixed_amd as T; "
            "T.tcm_plan(64, 64, 64, 64, 64, 64, 0); print(T.tcm_tune_table(), end='')" % os.path.dirname(os.path.dirname(T.__file__)))
    env = dict(os.environ)
    env.pop("TCM_TUNE_FILE", None)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, check=True).stdout
    assert sorted(out.splitlines()) == sorted(lines)
    # an empty TCM_TUNE_FILE ships nothing
    env["TCM_TUNE_FILE"] = ""
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, check=True).stdout
    assert out == ""
    ents = _entries()
    assert len(ents) >= 12
    # it covers the headline (f16, B column-major, 8192^3) and the workload set's classes
    assert any(e[0:10] == [0, 0, 1, 0, 0, 1, 0, 26, 26, 26] for e in ents)


@pytest.mark.parametrize("i", range(len(_entries())))
def test_planner_uses_every_shipped_entry(i):
    e = _entries()[i]
    dtype, a_col, b_col, c_type, epi, aligned, batched = e[0:7]
    config, mode = e[10], e[11]
    M, N, K = e[17], e[18], e[19]
    code = dtype | (T.TCM_A_COLMAJOR if a_col else 0) | (T.TCM_B_COLMAJOR if b_col else 0)
    code |= {0: 0, 1: T.TCM_C_F16, 2: T.TCM_C_BF16}[c_type]
    lda, ldb = (M if a_col else K), (K if b_col else N)
    q = T.tcm_plan(M, N, K, lda, ldb, N, code, epi, bool(aligned))
    if config in (100, 101):  # a split-k GEMV kernel (the planner picks its own k ranges)
        assert q["kernel"] == 2 and q["config"] == -1, (e, q)
        if config == 100:  # the 4x4x4 row-major-B kernel (256 columns a workgroup) or the column-major-B one
            assert M <= 16 and (b_col or q["bn"] == 256), (e, q)
        else:  # the 16x16x32 row-major-B kernel
            assert M <= 64 and not b_col and q["bn"] == 128, (e, q)
        return
    assert q["kernel"] == 1 and (q["config"], q["mode"]) == (config, mode), (e, q)
    if e[12] == 2:  # equal shares of every tile
        assert q["grid"] % q["tiles"] == 0 and q["grid"] <= e[13] * q["tiles"]
    T.tcm_set_option("tuned", 0)
    q0 = T.tcm_plan(M, N, K, lda, ldb, N, code, epi, bool(aligned))
    T.tcm_set_option("tuned", 1)
    # the model's plan is a tiled one as well, or the GEMV for a few rows
    assert q0["kernel"] == 1 or (q0["kernel"] == 2 and M <= 32)
