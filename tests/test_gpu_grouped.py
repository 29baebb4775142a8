"""GPU parity of tcm_gemm_grouped: every entry of a group (its own M, N,
operands and leading dimensions, a shared K) against the CPU oracle run on
that entry alone.  Each C sits in a buffer with a sentinel tail, so a store
past an entry's C shows up."""
import numpy as np
import pytest
import torch

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import check, say, to_device

pytestmark = pytest.mark.gpu

DTYPES = [S.F16, S.BF16, S.F32, S.I8]
_C_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}
TAIL = 32


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    T.tcm_set_option("force_mode", 0)
    T.tcm_set_option("force_config", -1)
    T.tcm_set_option("sk_grid", 0)
    T.tcm_set_option("generic", 0)
    T.tcm_set_option("sk_fixup", 0)


def make_group(dtype, shapes, K, seed, b_col=False, bias=False, relu=False, c_type="acc", accum=False, ld_pad=0):
    """One small problem per (M, N) entry, each drawn from its own seed."""
    return [S.small_problem(dtype, M, N, K, seed=seed + i, b_col=b_col, bias=bias, relu=relu, c_type=c_type, accum=accum,
                            lda=(K + ld_pad) if ld_pad else 0, ldc=(N + ld_pad) if ld_pad else 0)
            for i, (M, N) in enumerate(shapes)]


def run_group(ps, a_offset=0):
    """tcm_gemm_grouped over problems ps (same dtype, K, flags); returns each C (M x ldc) and the plan."""
    gs = [S.generate(p) for p in ps]
    p0 = ps[0]
    c_t = _C_TORCH.get(p0.c_type, torch.int32 if p0.dtype == S.I8 else torch.float32)
    fill = -7 if p0.dtype == S.I8 else float("nan")
    keep, ents, Cs = [], [], []
    for i, (p, g) in enumerate(zip(ps, gs)):
        ka, pa = to_device(g["A"], p.dtype, a_offset if i == 0 else 0)
        kb, pb = to_device(g["B"], p.dtype)
        kbias = torch.from_numpy(g["bias"].copy()).cuda() if g["bias"] is not None else None
        C = torch.full((max(p.M, 1) * p.LDC + TAIL,), fill, dtype=c_t, device="cuda")
        if p.accum and p.M:
            cin = g["C_in"].reshape(-1)
            src = torch.from_numpy(cin.view(np.int16).copy()).view(c_t) if p.c_type != "acc" else torch.from_numpy(cin.copy())
            C[:cin.size] = src.cuda()
        keep += [ka, kb, kbias]
        Cs.append(C)
        ents.append((p.M, p.N, pa, p.LDA, pb, p.LDB, C.data_ptr(), p.LDC, kbias.data_ptr() if kbias is not None else None))
    code = p0.dtype | (T.TCM_B_COLMAJOR if p0.b_col else 0) | {"acc": 0, "f16": T.TCM_C_F16, "bf16": T.TCM_C_BF16}[p0.c_type]
    epi = (T.TCM_EPI_BIAS if p0.bias else 0) | (T.TCM_EPI_RELU if p0.relu else 0) | (T.TCM_EPI_ACCUM if p0.accum else 0)
    say(f"[case] grouped {len(ps)} entries {[(p.M, p.N) for p in ps]} K={p0.K} dtype={p0.dtype} b_col={p0.b_col} "
        f"bias={p0.bias} c_type={p0.c_type} accum={p0.accum} force_config={T.tcm_get_option('force_config')} "
        f"force_mode={T.tcm_get_option('force_mode')} sk_grid={T.tcm_get_option('sk_grid')}")
    st = T.tcm_gemm_grouped(ents, p0.K, code, epi, torch.cuda.current_stream().cuda_stream)
    assert st == T.TCM_OK, T.tcm_status_string(st)
    plan = T.tcm_last_plan()
    say(f"       plan: {plan}")
    torch.cuda.synchronize()
    outs = []
    for p, C in zip(ps, Cs):
        h = (C.float() if c_t in (torch.float16, torch.bfloat16) else C).cpu().numpy()
        tail = h[max(p.M, 1) * p.LDC:]
        assert np.all(np.isnan(tail)) if p.dtype != S.I8 else np.all(tail == -7), "wrote past an entry's C"
        outs.append(h[:p.M * p.LDC].reshape(p.M, p.LDC))
    del keep
    return gs, outs, plan


def check_group(ps, gs, outs):
    for p, g, C in zip(ps, gs, outs):
        if p.M and p.N:
            check(p, g, C)


SHAPES = [(37, 64), (0, 128), (130, 48), (1, 208), (64, 64), (200, 96)]  # ragged M, N multiples of 16, an empty entry


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("config", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("mode", [1, 2])
def test_grouped_every_config_and_mode(dtype, config, mode):
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", mode)
    ps = make_group(dtype, SHAPES, 208, seed=200 + config, b_col=(config % 2 == 1), bias=True, relu=True)
    gs, outs, plan = run_group(ps)
    assert f"config={config}" in plan and "group=6" in plan
    assert ("mode=dp" if mode == 1 else "mode=streamk") in plan
    check_group(ps, gs, outs)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("config", [4, 5, 6])
@pytest.mark.parametrize("sk_grid", [3, 37, 200])
@pytest.mark.parametrize("fixup", [1, 2])
def test_grouped_streamk_splits_across_entries(dtype, config, sk_grid, fixup):
    """One Stream-K grid over the tiles of every entry; segments cross entry
    boundaries; split tiles summed by their last arrival or a second kernel."""
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("sk_grid", sk_grid)
    T.tcm_set_option("sk_fixup", fixup)
    K = 1024 if dtype != S.I8 else 2048
    ps = make_group(dtype, [(16, 192), (5, 64), (48, 128), (1, 256)], K, seed=210, bias=True)
    gs, outs, plan = run_group(ps)
    assert "mode=streamk" in plan
    check_group(ps, gs, outs)


@pytest.mark.parametrize("variant", [(S.F16, "f16", True), (S.BF16, "bf16", False), (S.F32, "acc", True),
                                     (S.I8, "acc", True)], ids=["f16-Cf16-accum", "bf16-Cbf16", "f32-accum", "i8-accum"])
@pytest.mark.parametrize("mode", [1, 2])
def test_grouped_wider_epilogue_and_padded_ld(variant, mode):
    dtype, c_type, accum = variant
    T.tcm_set_option("force_mode", mode)
    ps = make_group(dtype, [(70, 80), (33, 160), (128, 32)], 256, seed=220, bias=True, relu=True, c_type=c_type,
                    accum=accum, ld_pad=16)
    gs, outs, plan = run_group(ps)
    assert "kernel=tile" in plan
    check_group(ps, gs, outs)


@pytest.mark.parametrize("dtype", DTYPES)
def test_grouped_falls_back_entry_by_entry(dtype):
    """An entry no tile config can take (unaligned A): every entry runs on its own, same results."""
    ps = make_group(dtype, [(40, 64), (20, 32)], 96, seed=230, bias=True)
    gs, outs, plan = run_group(ps, a_offset=1)
    assert "entries one by one" in plan
    check_group(ps, gs, outs)


def test_grouped_int8_dp_and_streamk_bit_exact():
    ps = make_group(S.I8, [(48, 256), (7, 128), (96, 64)], 2048, seed=240, bias=True, relu=True)
    results = []
    for mode in (1, 2):
        T.tcm_set_option("force_mode", mode)
        T.tcm_set_option("force_config", 4)
        gs, outs, plan = run_group(ps)
        check_group(ps, gs, outs)
        results.append(outs)
    for a, b in zip(*results):
        assert np.array_equal(a, b)


def test_grouped_single_entry_matches_tcm_gemm():
    """A group of one is tcm_gemm on the same plan: identical bits."""
    from gpu_util import run_tcm
    p = S.small_problem(S.F16, 100, 144, 208, seed=250, bias=True, relu=True)
    T.tcm_set_option("force_config", 1)
    T.tcm_set_option("force_mode", 1)
    g = S.generate(p)
    C1, _ = run_tcm(p, g)
    gs, outs, plan = run_group([p])
    assert np.array_equal(C1[:, :p.N], outs[0][:, :p.N])
    check(p, gs[0], outs[0])


def test_torch_convenience_grouped():
    torch.manual_seed(2)
    As = [torch.randn(m, 64, device="cuda").half() for m in (5, 40, 17)]
    Bs = [torch.randn(64, n, device="cuda").half() for n in (48, 32, 80)]
    bs = [torch.randn(n, device="cuda") for n in (48, 32, 80)]
    Cs = T.gemm_grouped(As, Bs, biases=bs, relu=True)
    for A, B, b, C in zip(As, Bs, bs, Cs):
        ref = (A.float() @ B.float() + b).relu()
        assert torch.allclose(C, ref, atol=1e-2, rtol=1e-3)


N_RANDOM = 60


def draw_group(seed):
    """Random group `seed`: 1 to 12 entries sharing K and the type, each with
    its own M (0 to 300) and N (on the 16-byte grid, or not: such groups run
    entry by entry), either layout of B, padded leading dimensions, any
    epilogue, and now and then a forced tile config, mode or Stream-K grid."""
    rng = np.random.default_rng(66000 + seed)
    dtype = DTYPES[int(rng.integers(len(DTYPES)))]
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    on_grid = rng.random() < 0.8
    count = int(rng.integers(1, 13))
    shapes = []
    for _ in range(count):
        M = int(rng.integers(0, 301)) if rng.random() < 0.9 else 0
        N = int(rng.integers(1, 300))
        shapes.append((M, max(ce, N // ce * ce) if on_grid else N))
    K = int(rng.integers(1, 1200))
    K = max(ce, K // ce * ce) if on_grid else K
    c_type = "acc" if dtype in (S.I8, S.F32) else ["acc", "f16", "bf16"][int(rng.integers(3))]
    if c_type == "bf16" and dtype == S.F16:
        c_type = "f16"
    if c_type == "f16" and dtype == S.BF16:
        c_type = "bf16"
    ps = make_group(dtype, shapes, K, seed=3000 + 20 * seed, b_col=bool(rng.integers(2)), bias=bool(rng.integers(2)),
                    relu=bool(rng.integers(2)), c_type=c_type, accum=rng.random() < 0.25,
                    ld_pad=int(rng.integers(0, 3)) * ce)
    opts = {}
    r = rng.random()
    if r < 0.25:
        opts = {"force_config": int(rng.integers(0, T.tcm_config_count())), "force_mode": int(rng.integers(1, 3))}
    elif r < 0.4:
        opts = {"force_mode": 2, "sk_grid": int(rng.integers(1, 400))}
    return ps, opts


@pytest.mark.parametrize("seed", range(N_RANDOM))
def test_random_group_case(seed):
    ps, opts = draw_group(seed)
    for k, v in opts.items():
        assert T.tcm_set_option(k, v) == T.TCM_OK
    if all(p.M == 0 for p in ps):
        ps[0] = S.small_problem(ps[0].dtype, 7, ps[0].N, ps[0].K, seed=ps[0].seed, b_col=ps[0].b_col, bias=ps[0].bias,
                                relu=ps[0].relu, c_type=ps[0].c_type, accum=ps[0].accum)
    gs, outs, plan = run_group(ps)
    check_group(ps, gs, outs)
