"""Stream-K against data-parallel, bit for bit, on int8 (exact arithmetic):
at the two split-k shapes of the workload set and, repeated, on problems
whose tiles are split over many workgroups.

Split tiles are finished by their last arriving workgroup, which reads the
other segments' partial tiles after an arrival counter says they are stored
(device-coherent loads and stores plus a relaxed device-scope counter).  A
partial read too early, or a stale cached copy of one, changes the int8
result; the repeated runs stop at the first call that differs from the
data-parallel result and name it."""
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
    for k, v in (("force_mode", 0), ("force_config", -1), ("sk_grid", 0), ("sk_fixup", 0)):
        T.tcm_set_option(k, v)


class _Resident:
    """One problem's inputs uploaded once; `run()` computes C into a buffer
    first filled with a sentinel and returns it (on the device)."""

    def __init__(self, p):
        self.p = p
        self.g = S.generate(p)
        self.ka, self.pa = to_device(self.g["A"], p.dtype)
        self.kb, self.pb = to_device(self.g["B"], p.dtype)
        self.bias = torch.from_numpy(self.g["bias"].copy()).cuda() if p.bias else None
        ct = torch.int32 if p.dtype == S.I8 else torch.float32
        self.C = torch.empty(p.M * p.LDC, dtype=ct, device="cuda")
        self.code = p.dtype | (T.TCM_B_COLMAJOR if p.b_col else 0)
        self.epi = (T.TCM_EPI_BIAS if p.bias else 0) | (T.TCM_EPI_RELU if p.relu else 0)

    def run(self):
        p = self.p
        self.C.fill_(-7 if p.dtype == S.I8 else float("nan"))
        st = T.tcm_gemm(p.M, p.N, p.K, self.pa, p.LDA, self.pb, p.LDB, self.C.data_ptr(), p.LDC, self.code,
                        None if self.bias is None else self.bias.data_ptr(), self.epi,
                        torch.cuda.current_stream().cuda_stream)
        assert st == T.TCM_OK, T.tcm_status_string(st)
        return self.C


def _mode(mode, config=-1, sk_grid=0, fixup=0):
    T.tcm_set_option("force_mode", mode)
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("sk_grid", sk_grid)
    T.tcm_set_option("sk_fixup", fixup)


@pytest.mark.parametrize("M,N,K", [(3840, 3840, 4096), (1536, 1536, 16384)])
def test_int8_dp_and_streamk_bit_exact_at_split_k_shapes(M, N, K):
    """The split-k shapes of the workload set, in int8: the planner's
    data-parallel and Stream-K plans give identical int32 results, and both
    match the oracle on sampled entries."""
    p = S.small_problem(S.I8, M, N, K, seed=71, b_col=True, bias=True, relu=True)
    say(f"[case] int8 {M}x{N}x{K} data-parallel against Stream-K")
    r = _Resident(p)
    _mode(1)
    C_dp = r.run().clone()
    plan_dp = T.tcm_last_plan()
    _mode(2)
    C_sk = r.run().clone()
    plan_sk = T.tcm_last_plan()
    say(f"       dp: {plan_dp}\n       sk: {plan_sk}")
    assert "mode=dp" in plan_dp and "mode=streamk" in plan_sk
    assert torch.equal(C_dp, C_sk), "int8 data-parallel and Stream-K results differ"
    ii, jj = S.sample_entries(p)
    check(p, r.g, C_sk.cpu().numpy().reshape(M, p.LDC), ii, jj)


# (M, N, K-steps of 128 int8, config, grid): 8 to 32 segments per split tile,
# some segments shorter than the pipeline depth
MANY = [(256, 512, 96, 1, 256, 1), (64, 4096, 32, 5, 512, 1), (32, 4096, 32, 6, 512, 1), (256, 512, 96, 1, 256, 2)]


@pytest.mark.parametrize("M,N,ksteps,config,grid,fixup", MANY)
def test_int8_streamk_repeated_against_data_parallel(M, N, ksteps, config, grid, fixup):
    """200 back-to-back Stream-K calls, each compared with the data-parallel
    result before the next; the first mismatch fails the test and names its
    call.  fixup 1: the last arrival sums each split tile; 2: a second kernel
    does."""
    p = S.small_problem(S.I8, M, N, 128 * ksteps, seed=72 + config, b_col=(config != 1), bias=True)
    say(f"[case] int8 {M}x{N}x{p.K} config={config} grid={grid} fixup={fixup}, 200 Stream-K calls")
    r = _Resident(p)
    _mode(1, config)
    C_dp = r.run().clone()
    check(p, r.g, C_dp.cpu().numpy().reshape(M, p.LDC))
    _mode(2, config, grid, fixup)
    for i in range(200):
        C = r.run()
        if i == 0:
            plan = T.tcm_last_plan()
            say(f"       sk: {plan}")
            assert "mode=streamk" in plan and f"grid={grid}" in plan
        if not torch.equal(C, C_dp):
            bad = int((C != C_dp).sum())
            pytest.fail(f"Stream-K call {i} differs from data-parallel in {bad} entries")


@pytest.mark.parametrize("dtype", [S.F16, S.BF16])
def test_float_streamk_repeated_is_deterministic(dtype):
    """The last arrival adds the partials in workgroup order whichever
    workgroup arrives last, so 100 Stream-K calls give the same bits."""
    p = S.small_problem(dtype, 256, 512, 64 * 96, seed=74, b_col=True, bias=True)
    say(f"[case] dtype={dtype} {p.M}x{p.N}x{p.K} config=1 grid=256, 100 Stream-K calls")
    r = _Resident(p)
    _mode(2, 1, 256, 1)
    first = r.run().clone()
    check(p, r.g, first.cpu().numpy().reshape(p.M, p.LDC))
    for i in range(1, 100):
        C = r.run()
        if not torch.equal(C, first):
            pytest.fail(f"Stream-K call {i} differs from the first call")
