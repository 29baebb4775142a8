"""GPU parity of tcm_gemm_batched: every entry of a strided batch against the
CPU oracle run on that entry alone.  Entries sit at padded strides with
sentinels in the gaps, so an indexing mistake reads or writes the wrong
element and shows up."""
import numpy as np
import pytest
import torch

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import check, say

pytestmark = pytest.mark.gpu

DTYPES = [S.F16, S.BF16, S.F32, S.I8]
_T = {S.F16: torch.int16, S.BF16: torch.int16, S.F32: torch.float32, S.I8: torch.int8}
_C_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    T.tcm_set_option("force_mode", 0)
    T.tcm_set_option("force_config", -1)
    T.tcm_set_option("sk_grid", 0)
    T.tcm_set_option("generic", 0)
    T.tcm_set_option("sk_fixup", 0)
    T.tcm_set_option("grid_shares", 0)


def _pack(arr, n_entries, pad, fill):
    """Entries of arr (n_entries, ...) flattened at a stride of entry size + pad."""
    flat = np.ascontiguousarray(arr).reshape(n_entries, -1)
    stride = flat.shape[1] + pad
    out = np.full((n_entries, stride), fill, dtype=flat.dtype)
    out[:, :flat.shape[1]] = flat
    return out.reshape(-1), stride


def _dev(flat, dtype):
    if flat.dtype == np.uint16:
        return torch.from_numpy(flat.view(np.int16).copy()).cuda()
    return torch.from_numpy(flat.copy()).cuda()


def run_batched(p, g, pads=(64, 128, 32), shared_bias=False):
    """Call tcm_gemm_batched through the C ABI; returns C as (batch, M, ldc) float/int arrays and the plan.
    The default padding keeps every entry 16-byte aligned for any element type (the fast path)."""
    pa, pb, pc = pads
    nb = 1 if p.b_shared else p.batch
    sent = {S.F16: np.float16(np.nan).view(np.uint16), S.BF16: np.uint16(0x7FC0), S.F32: np.float32(np.nan),
            S.I8: np.int8(99)}[p.dtype]
    A, sa = _pack(g["A"], p.batch, pa, sent)
    B, sb = _pack(g["B"], nb, pb, sent)
    sb = 0 if p.b_shared else sb
    kA, kB = _dev(A, p.dtype), _dev(B, p.dtype)
    bias_ptr, sbias, kbias = None, 0, None
    if g["bias"] is not None:
        bias = g["bias"][:1] if shared_bias else g["bias"]
        bflat, sbias = _pack(bias, bias.shape[0], 4, 0)
        sbias = 0 if shared_bias else sbias
        kbias = torch.from_numpy(bflat.copy()).cuda()
        bias_ptr = kbias.data_ptr()
    c_t = _C_TORCH.get(p.c_type, torch.int32 if p.dtype == S.I8 else torch.float32)
    entry_c = p.M * p.LDC
    sc = entry_c + pc
    C = torch.full((p.batch * sc,), -7 if p.dtype == S.I8 else float("nan"), dtype=c_t, device="cuda")
    if p.accum:
        for e in range(p.batch):
            cin = g["C_in"][e].reshape(-1)
            src = torch.from_numpy(cin.view(np.int16).copy()).view(c_t) if cin.dtype == np.uint16 else torch.from_numpy(cin.copy())
            C[e * sc:e * sc + entry_c] = src.cuda()
    code = p.dtype | (T.TCM_A_COLMAJOR if p.a_col else 0) | (T.TCM_B_COLMAJOR if p.b_col else 0)
    code |= {"acc": 0, "f16": T.TCM_C_F16, "bf16": T.TCM_C_BF16}[p.c_type]
    epi = (T.TCM_EPI_BIAS if p.bias else 0) | (T.TCM_EPI_RELU if p.relu else 0) | (T.TCM_EPI_ACCUM if p.accum else 0)
    st = T.tcm_gemm_batched(p.batch, p.M, p.N, p.K, kA.data_ptr(), p.LDA, sa, kB.data_ptr(), p.LDB, sb,
                            C.data_ptr(), p.LDC, sc, code, bias_ptr, sbias, epi,
                            torch.cuda.current_stream().cuda_stream)
    assert st == T.TCM_OK, T.tcm_status_string(st)
    plan = T.tcm_last_plan()
    torch.cuda.synchronize()
    Cc = C.float() if c_t in (torch.float16, torch.bfloat16) else C
    out = Cc.cpu().numpy().reshape(p.batch, sc)
    gap = out[:, entry_c:]
    assert np.all(np.isnan(gap)) if p.dtype != S.I8 else np.all(gap == -7), "wrote between batch entries"
    return out[:, :entry_c].reshape(p.batch, p.M, p.LDC), plan


def check_batch(p, g, C, shared_bias=False):
    errs = []
    for e in range(p.batch):
        ge = S.entry_inputs(p, g, e)
        if shared_bias and ge["bias"] is not None:
            ge = dict(ge, bias=g["bias"][0])
        errs.append(check(p.entry(e), ge, C[e]))
    return max(errs)


def _case(p, **kw):
    say(f"[case] batched {p.name} batch={p.batch} M={p.M} N={p.N} K={p.K} dtype={p.dtype} b_col={p.b_col} "
        f"b_shared={p.b_shared} bias={p.bias} c_type={p.c_type} accum={p.accum} seed={p.seed} "
        f"force_mode={T.tcm_get_option('force_mode')} force_config={T.tcm_get_option('force_config')} {kw}")
    g = S.generate(p)
    C, plan = run_batched(p, g, **{k: v for k, v in kw.items() if k in ("pads", "shared_bias")})
    say(f"       plan: {plan}")
    return g, C, plan


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("config", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("mode", [1, 2])
def test_batched_every_config_and_mode(dtype, config, mode):
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", mode)
    p = S.small_problem(dtype, 40, 144, 208, seed=90 + config, bias=True, relu=True, batch=3)
    g, C, plan = _case(p)
    assert f"config={config}" in plan and "batch=3" in plan
    check_batch(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("a_col", [False, True])
@pytest.mark.parametrize("b_shared", [False, True])
def test_batched_equal_shares(dtype, a_col, b_shared):
    """Equal shares of the eight-wave tile across a batch: the entries' tiles
    form one list (3 entries x 2 x 2 tiles), every tile cut into 5 k shares
    (the last holding the K tail), each share and the sum on its entry's
    operands, B shared or not, both layouts of A."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    bk = {S.F16: 64, S.BF16: 64, S.F32: 32, S.I8: 128}[dtype]
    T.tcm_set_option("force_config", 0)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("grid_shares", 5)
    p = S.small_problem(dtype, 272, 272, 25 * bk + ce, seed=120, a_col=a_col, bias=True, relu=True, batch=3,
                        b_shared=b_shared, lda=272 + ce if a_col else 0)
    g, C, plan = _case(p)
    assert "config=0" in plan and "split=5" in plan and "grid=60" in plan and "batch=3" in plan
    check_batch(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("config", [1, 4])
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("b_col", [False, True])
def test_batched_column_major_a(dtype, config, mode, b_col):
    """Column-major A on the tiles across a batch: each entry's A at its own
    stride, Stream-K segments crossing entries."""
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", mode)
    p = S.small_problem(dtype, 80, 144, 208, seed=99 + config, a_col=True, b_col=b_col, bias=True, relu=True, batch=3)
    g, C, plan = _case(p)
    assert "kernel=tile" in plan and f"config={config}" in plan and "a_col=1" in plan
    check_batch(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
def test_batched_shared_b_and_bias(dtype):
    """Stride 0 shares B (and the bias) across the batch."""
    p = S.small_problem(dtype, 33, 80, 96, seed=95, bias=True, batch=5, b_shared=True, b_col=True)
    g, C, plan = _case(p, shared_bias=True)
    check_batch(p, g, C, shared_bias=True)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("sk_grid", [5, 37, 200])
@pytest.mark.parametrize("config", [4, 5, 6])
@pytest.mark.parametrize("fixup", [1, 2])
def test_batched_streamk_splits_across_entries(dtype, sk_grid, config, fixup):
    """One Stream-K grid over the tiles of all entries; segments cross entry
    boundaries; split tiles summed by their last arrival or a second kernel."""
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("sk_grid", sk_grid)
    T.tcm_set_option("sk_fixup", fixup)
    p = S.small_problem(dtype, 16, 192, 1024, seed=96, bias=True, batch=7)
    g, C, plan = _case(p)
    assert "mode=streamk" in plan
    check_batch(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", ["odd_k", "a_col"])
def test_batched_generic_path(dtype, layout):
    if layout == "odd_k":
        p = S.small_problem(dtype, 50, 70, 37, seed=97, bias=True, relu=True, batch=4)
    else:
        p = S.small_problem(dtype, 50, 72, 48, seed=98, a_col=True, bias=True, batch=4)
    g, C, plan = _case(p, pads=(3, 5, 7))  # odd padding: misaligned entries as well
    assert "kernel=generic" in plan
    check_batch(p, g, C)


@pytest.mark.parametrize("variant", [(S.F16, "f16", True), (S.BF16, "bf16", False), (S.I8, "acc", True)],
                         ids=["f16-Cf16-accum", "bf16-Cbf16", "i8-accum"])
@pytest.mark.parametrize("mode", [1, 2])
def test_batched_wider_epilogue(variant, mode):
    dtype, c_type, accum = variant
    T.tcm_set_option("force_mode", mode)
    p = S.small_problem(dtype, 64, 128, 256, seed=99, bias=True, relu=True, batch=3, c_type=c_type, accum=accum)
    g, C, plan = _case(p)
    check_batch(p, g, C)


def test_batched_int8_dp_and_streamk_bit_exact():
    p = S.small_problem(S.I8, 48, 256, 2048, seed=100, bias=True, batch=6)
    g = S.generate(p)
    outs = []
    for mode in (1, 2):
        T.tcm_set_option("force_mode", mode)
        C, plan = run_batched(p, g)
        check_batch(p, g, C)
        outs.append(C)
    assert np.array_equal(outs[0], outs[1])


def test_batch_of_one_matches_single_call():
    """tcm_gemm_batched with batch 1 is tcm_gemm: identical bits."""
    p = S.small_problem(S.F16, 100, 136, 200, seed=101, bias=True, relu=True)
    g = S.generate(p)
    from gpu_util import run_tcm
    C1, _ = run_tcm(p, g)
    q = S.small_problem(S.F16, 100, 136, 200, seed=101, bias=True, relu=True)
    gb = {k: (None if v is None else v[None]) for k, v in g.items()}
    qb = S.Problem(**{**q.__dict__, "batch": 1})
    Cb, _ = run_batched(qb, gb, pads=(0, 0, 0))
    assert np.array_equal(np.nan_to_num(C1, nan=1234.5), np.nan_to_num(Cb[0], nan=1234.5))


def test_empty_batch_is_a_no_op():
    C = torch.full((16,), 3.0, device="cuda")
    A = torch.zeros(16, dtype=torch.float16, device="cuda")
    st = T.tcm_gemm_batched(0, 4, 4, 4, A.data_ptr(), 4, 16, A.data_ptr(), 4, 16, C.data_ptr(), 4, 16, 0, None, 0, 0,
                            None)
    assert st == T.TCM_OK
    torch.cuda.synchronize()
    assert torch.all(C == 3.0)


def test_torch_convenience_batched():
    torch.manual_seed(1)
    A = torch.randn(4, 24, 64, device="cuda").half()
    W = torch.randn(4, 64, 40, device="cuda").half()
    C = T.gemm_batched(A, W)
    ref = torch.stack([A[e].float() @ W[e].float() for e in range(4)])
    assert torch.allclose(C, ref, atol=1e-2, rtol=1e-3)
    # one shared (expanded) B and a per-entry bias
    Wb = torch.randn(64, 40, device="cuda").half()
    bias = torch.randn(4, 40, device="cuda")
    C2 = T.gemm_batched(A, Wb.expand(4, 64, 40), bias=bias)
    ref2 = torch.stack([A[e].float() @ Wb.float() + bias[e] for e in range(4)])
    assert torch.allclose(C2, ref2, atol=1e-2, rtol=1e-3)
