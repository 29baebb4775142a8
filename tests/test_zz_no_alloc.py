"""tcm_gemm_noalloc (no allocation: Stream-K scratch in a fixed device
array) against tcm_gemm on the same inputs, through the C ABI.  Each case
runs two calls in a row, the second on a smaller problem, so the second
reuses the array the first left behind (counters cleared, partial slots
overwritten).  The bar is the parity bar of the other GPU tests (bit-exact
int8, normalised error for floats), and where both entry points launch the
same plan their outputs must agree bit for bit."""
import numpy as np
import pytest
import torch

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import check, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    T.tcm_set_option("force_mode", 0)
    T.tcm_set_option("force_config", -1)
    T.tcm_set_option("sk_grid", 0)
    T.tcm_set_option("sk_fixup", 0)
    T.tcm_set_option("gemv", 0)


def _call(fn, p, g):
    ka, pa = to_device(g["A"], p.dtype)
    kb, pb = to_device(g["B"], p.dtype)
    kbias = torch.from_numpy(g["bias"].copy()).cuda() if g["bias"] is not None else None
    C = torch.full((p.M, p.LDC), -7 if p.dtype == S.I8 else float("nan"),
                   dtype=torch.int32 if p.dtype == S.I8 else torch.float32, device="cuda")
    epi = (T.TCM_EPI_BIAS if p.bias else 0) | (T.TCM_EPI_RELU if p.relu else 0)
    code = p.dtype | (T.TCM_B_COLMAJOR if p.b_col else 0)
    st = fn(p.M, p.N, p.K, pa, p.LDA, pb, p.LDB, C.data_ptr(), p.LDC, code,
            kbias.data_ptr() if kbias is not None else None, epi, torch.cuda.current_stream().cuda_stream)
    plan = T.tcm_last_plan()
    torch.cuda.synchronize()
    out = C.cpu().numpy()
    del ka, kb, kbias
    return st, out, plan


# (config, mode, fixup, first problem, second smaller problem)
CASES = [
    (4, 2, 1, (512, 512, 4096), (130, 200, 1024)),     # Stream-K, last arrival: counters in the scratch
    (4, 2, 2, (512, 512, 4096), (130, 200, 1024)),     # Stream-K, fix-up kernel: partials only
    (1, 2, 1, (1024, 768, 2048), (300, 264, 512)),     # 128x128 units, larger partial slots
    (6, 2, 2, (16, 4096, 4096), (1, 1024, 2048)),      # skinny Stream-K units
    (-1, 0, 0, (1536, 1536, 4096), (520, 264, 640)),   # the planner's choice
    (0, 1, 0, (600, 520, 512), (260, 136, 256)),       # data-parallel: no scratch used
    (0, 2, 0, (1024, 768, 2048), (520, 264, 640)),     # equal shares of the eight-wave tile: one partial a workgroup
]


@pytest.mark.parametrize("dtype", [S.F16, S.BF16, S.F32, S.I8])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"cfg{c[0]}-mode{c[1]}-fix{c[2]}")
def test_noalloc_matches_tcm_gemm_two_calls(dtype, case):
    config, mode, fixup, first, second = case
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", mode)
    T.tcm_set_option("sk_fixup", fixup)
    for i, (M, N, K) in enumerate((first, second)):
        N, K = max(ce, N // ce * ce), max(ce, K // ce * ce)
        p = S.small_problem(dtype, M, N, K, seed=500 + i, bias=True, relu=(i == 1))
        say(f"[case] noalloc call {i + 1}: {p.name} dtype={dtype} config={config} mode={mode} fixup={fixup}")
        g = S.generate(p)
        st0, ref, plan0 = _call(T.tcm_gemm, p, g)
        assert st0 == T.TCM_OK, T.tcm_status_string(st0)
        st1, got, plan1 = _call(T.tcm_gemm_noalloc, p, g)
        assert st1 == T.TCM_OK, T.tcm_status_string(st1)
        say(f"       tcm_gemm:         {plan0}")
        say(f"       tcm_gemm_noalloc: {plan1}")
        assert "scratch=static" in plan1
        check(p, g, got)
        if plan1.replace(" scratch=static", "") == plan0:
            assert np.array_equal(np.nan_to_num(got, nan=1e30), np.nan_to_num(ref, nan=1e30)), "same plan, different bits"
        else:
            check(p, g, ref)


@pytest.mark.parametrize("shapes", [((8, 4096, 4096), (3, 1028, 1000)), ((40, 4096, 4096), (17, 2048, 1000))],
                         ids=["both_kernels", "wide"])
@pytest.mark.parametrize("dtype", [S.F16, S.BF16])
def test_noalloc_gemv_two_calls(dtype, shapes):
    """The split-k GEMV kernels keep their partial sums in the same array:
    two calls in a row, the second smaller, bit-identical to tcm_gemm's (the
    16x16x32 kernel then the 4x4x4 one; the 16x16x32 kernel twice)."""
    T.tcm_set_option("gemv", 2)
    for i, (M, N, K) in enumerate(shapes):
        p = S.small_problem(dtype, M, N, K, seed=520 + i, bias=True, relu=(i == 1))
        say(f"[case] noalloc gemv call {i + 1}: {p.name} dtype={dtype}")
        g = S.generate(p)
        st0, ref, plan0 = _call(T.tcm_gemm, p, g)
        st1, got, plan1 = _call(T.tcm_gemm_noalloc, p, g)
        assert st0 == T.TCM_OK and st1 == T.TCM_OK
        say(f"       {plan1}")
        assert "kernel=gemv" in plan0 and plan1 == plan0 + " scratch=static"
        check(p, g, got)
        assert np.array_equal(got, ref), "same plan, different bits"


def test_noalloc_forced_streamk_beyond_the_scratch_is_refused():
    """A forced Stream-K grid whose partial slots exceed the fixed array is
    refused with TCM_ERR_NOT_SUPPORTED (nothing launched, C untouched); left
    to the planner, the same call runs data-parallel and is correct."""
    p = S.small_problem(S.F16, 1024, 1024, 8192, seed=510, bias=True)
    g = S.generate(p)
    T.tcm_set_option("force_config", 1)  # 128 x 128 tiles: 128 KiB of partial slots per workgroup
    T.tcm_set_option("sk_grid", 2048)    # 256 MiB of slots > the 64 MiB array
    T.tcm_set_option("force_mode", 2)
    say(f"[case] noalloc forced Stream-K beyond the scratch ({T.tcm_noalloc_scratch_bytes()} bytes)")
    st, C, plan = _call(T.tcm_gemm_noalloc, p, g)
    say(f"       {T.tcm_status_string(st)}: {plan}")
    assert st == T.TCM_ERR_NOT_SUPPORTED
    assert np.all(np.isnan(C)), "a refused call wrote C"
    T.tcm_set_option("force_mode", 0)
    st, C, plan = _call(T.tcm_gemm_noalloc, p, g)
    say(f"       planner's choice: {plan}")
    assert st == T.TCM_OK and "mode=dp" in plan
    check(p, g, C)
