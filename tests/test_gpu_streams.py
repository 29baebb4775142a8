"""Streams and graphs: calls on two streams at once (each stream has its own
split-k workspace), and a captured HIP graph replayed several times with
eager work in between, each replay checked against the oracle."""
import numpy as np
import pytest
import torch

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import check, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    T.tcm_set_option("gemv", 0)
    T.tcm_set_option("gemv_wide", 0)
    T.tcm_set_option("force_mode", 0)
    T.tcm_set_option("force_config", -1)
    T.tcm_set_option("sk_grid", 0)
    T.tcm_set_option("sk_fixup", 0)


def _dev(x):
    return torch.from_numpy(x.view(np.int16).copy() if x.dtype == np.uint16 else x.copy()).cuda()


class Call:
    """One problem resident on the device, callable on a given stream."""

    def __init__(self, p):
        self.p, self.g = p, S.generate(p)
        self.A, self.B = _dev(self.g["A"]), _dev(self.g["B"])
        self.bias = _dev(self.g["bias"]) if self.g["bias"] is not None else None
        self.C = torch.full((p.M, p.LDC), float("nan"), device="cuda")
        self.code = p.dtype | (T.TCM_B_COLMAJOR if p.b_col else 0)
        self.epi = (T.TCM_EPI_BIAS if p.bias else 0) | (T.TCM_EPI_RELU if p.relu else 0)

    def __call__(self, stream):
        p = self.p
        st = T.tcm_gemm(p.M, p.N, p.K, self.A.data_ptr(), p.LDA, self.B.data_ptr(), p.LDB, self.C.data_ptr(), p.LDC,
                        self.code, self.bias.data_ptr() if self.bias is not None else None, self.epi, stream.cuda_stream)
        assert st == T.TCM_OK, T.tcm_status_string(st)

    def check(self):
        return check(self.p, self.g, self.C.cpu().numpy())


@pytest.mark.parametrize("mode", [1, 2])
def test_two_streams_at_once(mode):
    T.tcm_set_option("force_mode", mode)
    T.tcm_set_option("force_config", 4)
    a = Call(S.small_problem(S.F16, 96, 320, 2048, seed=400, bias=True, relu=True))
    b = Call(S.small_problem(S.F16, 160, 128, 1536, seed=401, bias=True))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    say(f"[case] two streams, mode {mode}")
    for _ in range(3):  # several rounds, no synchronisation between the streams
        a(s1)
        b(s2)
    torch.cuda.synchronize()
    say(f"       plan: {T.tcm_last_plan()}")
    a.check()
    b.check()


@pytest.mark.parametrize("mode,fixup,config", [(1, 0, 4), (2, 1, 4), (2, 2, 4), (2, 0, 0)])
def test_graph_capture_replays(mode, fixup, config):
    """A call captured into a HIP graph (the split-k workspace already exists
    for the stream, so capture allocates nothing) gives the eager result on
    every replay; eager work and synchronisations run between the replays.
    With fixup 2 the call is two launches: Stream-K and its fix-up kernel;
    on the eight-wave config (config 0) the equal shares and their sum."""
    T.tcm_set_option("force_mode", mode)
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("sk_fixup", fixup)
    c = Call(S.small_problem(S.F16, 128 if config else 520, 256 if config else 272, 1024, seed=402, bias=True,
                             relu=True))
    s = torch.cuda.Stream()
    c(s)  # warm-up: plans, and creates this stream's workspace
    torch.cuda.synchronize()
    eager = c.C.clone()
    c.check()
    say(f"[case] graph capture, mode {mode}, fixup {fixup}, config {config}: {T.tcm_last_plan()}")
    if mode == 2 and config == 0:
        assert "split=8" in T.tcm_last_plan()
    elif mode == 2:
        assert ("fixup=kernel" in T.tcm_last_plan()) == (fixup == 2)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        c(s)
    for i in range(3):
        c.C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.nan_to_num(c.C, nan=1e9), torch.nan_to_num(eager, nan=1e9)), f"replay {i} differs"
        x = torch.randn(1024, device="cuda")  # unrelated eager work between the replays
        (x @ x).item()
    c.check()


def test_graph_replay_after_the_workspace_grew():
    """A graph captured on a stream keeps pointing at that stream's Stream-K
    workspace.  A later, larger call on the stream grows the workspace: the
    outgrown buffers are kept (not freed), so replays stay correct.  A call
    that would grow a workspace while its stream is capturing is refused
    with TCM_ERR_NOT_SUPPORTED instead of allocating inside the capture."""
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("force_config", 4)
    T.tcm_set_option("sk_fixup", 1)
    small = Call(S.small_problem(S.F16, 128, 256, 1024, seed=403, bias=True, relu=True))
    big = Call(S.small_problem(S.F16, 1024, 1024, 2048, seed=404, bias=True))
    s = torch.cuda.Stream()
    T.tcm_set_option("sk_grid", 16)
    small(s)  # this stream's workspace: 16 workgroups' partial slots
    torch.cuda.synchronize()
    eager = small.C.clone()
    small.check()
    say(f"[case] capture before growth: {T.tcm_last_plan()}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        small(s)
    T.tcm_set_option("sk_grid", 0)
    big(s)  # full co-resident grid: the workspace grows
    torch.cuda.synchronize()
    say(f"       growth: {T.tcm_last_plan()}")
    big.check()
    for i in range(3):
        small.C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.nan_to_num(small.C, nan=1e9), torch.nan_to_num(eager, nan=1e9)), f"replay {i} differs"
        big(s)  # eager calls on the same stream between the replays
        torch.cuda.synchronize()
    big.check()
    # a fresh stream has no workspace yet: capturing a Stream-K call there is refused
    s2 = torch.cuda.Stream()
    p = small.p
    g2 = torch.cuda.CUDAGraph()
    status = []
    with torch.cuda.graph(g2, stream=s2):
        status.append(T.tcm_gemm(p.M, p.N, p.K, small.A.data_ptr(), p.LDA, small.B.data_ptr(), p.LDB,
                                 small.C.data_ptr(), p.LDC, small.code, small.bias.data_ptr(), small.epi,
                                 s2.cuda_stream))
    say(f"       growth under capture: {T.tcm_status_string(status[0])}")
    assert status == [T.TCM_ERR_NOT_SUPPORTED]


@pytest.mark.parametrize("form", ["b_row", "b_wide", "b_col"])
def test_graph_capture_replays_gemv(form):
    """The split-k GEMV kernels (two launches: the k ranges, then their sum)
    captured into a graph after an eager call made the stream's workspace:
    every replay gives the eager bits."""
    b_col = form == "b_col"
    T.tcm_set_option("gemv", 2)
    T.tcm_set_option("gemv_wide", 2 if form == "b_wide" else 1)
    c = Call(S.small_problem(S.F16, 5 if form != "b_wide" else 40, 1024, 2048, seed=405, bias=True, relu=True,
                             b_col=b_col))
    s = torch.cuda.Stream()
    c(s)
    torch.cuda.synchronize()
    eager = c.C.clone()
    c.check()
    say(f"[case] graph capture, gemv {form}: {T.tcm_last_plan()}")
    assert "kernel=gemv" in T.tcm_last_plan() and "fixup=kernel" in T.tcm_last_plan()
    assert ("mfma=16x16x32" in T.tcm_last_plan()) == (form != "b_row")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        c(s)
    for i in range(3):
        c.C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.nan_to_num(c.C, nan=1e9), torch.nan_to_num(eager, nan=1e9)), f"replay {i} differs"
        x = torch.randn(1024, device="cuda")
        (x @ x).item()
    c.check()
