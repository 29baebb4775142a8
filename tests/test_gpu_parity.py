"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs (bars in gpu_util.py).  Each case prints its name, shape
and seed before touching the GPU."""
import numpy as np
import pytest
import torch

import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import check, check_padding_untouched, run_tcm, say

pytestmark = pytest.mark.gpu

DTYPES = [S.F16, S.BF16, S.F32, S.I8]


@pytest.fixture(autouse=True)
def _reset_options():
    # these cases are about the tiled and generic kernels: products of a few
    # rows stay on the tiles (the split-k GEMV has tests of its own)
    T.tcm_set_option("gemv", 1)
    yield
    T.tcm_set_option("gemv", 0)
    T.tcm_set_option("force_mode", 0)
    T.tcm_set_option("force_config", -1)
    T.tcm_set_option("sk_grid", 0)
    T.tcm_set_option("generic", 0)
    T.tcm_set_option("sk_fixup", 0)
    T.tcm_set_option("grid_shares", 0)


def _run(p, **kw):
    say(f"[case] {p.name} M={p.M} N={p.N} K={p.K} dtype={p.dtype} a_col={p.a_col} b_col={p.b_col} "
        f"bias={p.bias} relu={p.relu} lda={p.LDA} ldb={p.LDB} ldc={p.LDC} seed={p.seed} "
        f"force_mode={T.tcm_get_option('force_mode')} force_config={T.tcm_get_option('force_config')} "
        f"sk_grid={T.tcm_get_option('sk_grid')} generic={T.tcm_get_option('generic')}")
    g = S.generate(p)
    C, plan = run_tcm(p, g, **kw)
    say(f"       plan: {plan}")
    return g, C, plan


# ------------------------------------------------------------ small cases, all entries

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("b_col", [False, True])
def test_first_slice_512(dtype, b_col):
    """512^3 (several tiles, all entries) for every type and both B layouts."""
    p = S.small_problem(dtype, 512, 512, 512, seed=0, b_col=b_col)
    g, C, plan = _run(p)
    assert "kernel=tile" in plan
    check(p, g, C)


RAGGED = [(300, 264, 200), (257, 136, 72), (33, 520, 136), (1, 8, 64), (17, 40, 8), (600, 96, 392)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("b_col", [False, True])
def test_ragged_tiles_and_k_tail(dtype, shape, b_col):
    """Ragged M and N edges and a K tail, on the tiled kernel, with bias + ReLU."""
    M, N, K = shape
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    K = max(ce, K // ce * ce)
    if not b_col:
        N = max(ce, N // ce * ce)
    p = S.small_problem(dtype, M, N, K, seed=11, b_col=b_col, bias=True, relu=True)
    g, C, plan = _run(p)
    assert "kernel=tile" in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("config", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("mode", [1, 2])
def test_every_config_and_mode(dtype, config, mode):
    """Each tile config, data-parallel and Stream-K, on a shape with edges in M, N and K."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 190, 304, 53 * ce, seed=config * 10 + mode, bias=True, relu=(mode == 2))
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", mode)
    g, C, plan = _run(p)
    assert f"config={config}" in plan and ("mode=dp" if mode == 1 else "mode=streamk") in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("config", [0, 1, 3, 4, 5])
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("b_col", [False, True])
def test_column_major_a_every_config_and_mode(dtype, config, mode, b_col):
    """A stored column-major (m contiguous) on the tiles: each config of at
    least 64 rows, data-parallel and Stream-K, both B layouts, on a shape
    with edges in M (208: a partial tile of every height), N and K, bias and
    ReLU, and A's columns padded (lda past M)."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 208, 304, 53 * ce, seed=config * 10 + mode + 3, a_col=True, b_col=b_col, bias=True,
                        relu=(mode == 2), lda=208 + ce)
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", mode)
    g, C, plan = _run(p)
    assert "kernel=tile" in plan and f"config={config}" in plan
    assert ("mode=dp" if mode == 1 else "mode=streamk") in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(512, 512, 512), (64, 520, 136), (1024, 96, 392), (16, 4096, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("b_col", [False, True])
def test_column_major_a_planned(dtype, shape, b_col):
    """The planner's own plan for column-major A: the tiles (M is a whole
    number of 16-byte pieces here), with ragged N and a K tail."""
    M, N, K = shape
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    K = max(ce, K // ce * ce)
    if not b_col:
        N = max(ce, N // ce * ce)
    p = S.small_problem(dtype, M, N, K, seed=sum(shape) % 97, a_col=True, b_col=b_col, bias=True, relu=True)
    g, C, plan = _run(p)
    assert "kernel=tile" in plan, plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", [S.F16, S.I8])
def test_column_major_a_off_the_piece_grid_is_generic(dtype):
    """M not a whole number of 16-byte pieces: the generic kernel, correct."""
    ce = {S.F16: 8, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 4 * ce + 1, 256, 8 * ce, seed=41, a_col=True, b_col=True, bias=True)
    g, C, plan = _run(p)
    assert "kernel=generic" in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", [S.F16, S.BF16])
@pytest.mark.parametrize("ksteps", [1, 2, 3, 33])
@pytest.mark.parametrize("mode", [1, 2, 3])
@pytest.mark.parametrize("layout", ["b_row", "a_col_b_col", "a_col_b_row"])
def test_pingpong_loop_step_counts(dtype, ksteps, mode, layout):
    """The eight-wave kernel with row-major B or column-major A (operands
    read back with transposing LDS reads) runs its wave groups one phase
    apart, each group copying one operand, group B two K-steps ahead: one,
    two and three K-steps exercise the prologue and the steps that issue no
    copies, 33 the steady state (with a ragged k tail), on ragged M and N.
    Stream-K runs the same loop on segments that start mid-tile (mode 2, a
    given grid) and on equal shares (mode 3 here: Stream-K without a grid)."""
    K = 64 * ksteps - (24 if ksteps == 33 else 0)
    a_col, b_col = layout.startswith("a_col"), layout.endswith("b_col")
    p = S.small_problem(dtype, 520, 264, K, seed=70 + ksteps, bias=True, relu=(mode == 1), a_col=a_col, b_col=b_col,
                        lda=520 + 8 if a_col else 0)
    T.tcm_set_option("force_config", 0)
    T.tcm_set_option("force_mode", min(mode, 2))
    if mode == 2:
        T.tcm_set_option("sk_grid", 5)
    g, C, plan = _run(p)
    assert "config=0" in plan and f"b_col={int(b_col)}" in plan and (("a_col=1" in plan) == a_col)
    assert ("mode=dp" if mode == 1 else "mode=streamk") in plan
    if mode == 3 and ksteps > 1:
        assert f"split={min(8, ksteps)}" in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("sk_grid", [3, 7, 64, 301])
@pytest.mark.parametrize("config", [1, 5, 6])
@pytest.mark.parametrize("fixup", [1, 2])
def test_streamk_many_segments_per_tile(dtype, sk_grid, config, fixup):
    """Small persistent grids split each tile over several workgroups (and
    large ones give workgroups a few iterations each: segments shorter than
    the pipeline depth).  Split tiles are summed by their last arrival
    (fixup 1) or by a second kernel (fixup 2)."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 260, 208, 40 * ce, seed=sk_grid, b_col=(sk_grid % 2 == 1), bias=True)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("sk_grid", sk_grid)
    T.tcm_set_option("sk_fixup", fixup)
    g, C, plan = _run(p)
    grid = int(plan.split("grid=")[1].split()[0])
    assert "mode=streamk" in plan and 1 <= grid <= sk_grid
    assert ("fixup=kernel" in plan) == (fixup == 2)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("config", [1, 4, 5, 6])
def test_fixup_kernel_bit_identical_to_last_arrival(dtype, config):
    """Both ways of finishing a split tile add the same partials in the same
    order: the outputs agree bit for bit, floats included."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 150, 272, 96 * ce, seed=60 + config, bias=True, relu=True)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("sk_grid", 37)
    outs = []
    for fixup in (1, 2):
        T.tcm_set_option("sk_fixup", fixup)
        g, C, plan = _run(p)
        outs.append(C)
    check(p, g, outs[1])
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("dtype", DTYPES)
def test_int8_and_float_dp_vs_streamk_agree(dtype):
    """Data-parallel and Stream-K give the same int8 result bit-for-bit, and
    Stream-K's float result is the same bits on every run (fixed sum order)."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 384, 384, 48 * ce, seed=5, bias=True, relu=True)
    T.tcm_set_option("force_config", 1)
    T.tcm_set_option("force_mode", 1)
    g, C_dp, _ = _run(p)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("sk_grid", 29)
    _, C_sk1, _ = _run(p)
    _, C_sk2, _ = _run(p)
    check(p, g, C_sk1)
    assert np.array_equal(C_sk1, C_sk2), "Stream-K result differs between runs"
    if dtype == S.I8:
        assert np.array_equal(C_dp, C_sk1), "int8 data-parallel and Stream-K differ"


# ------------------------------------------- equal shares (the eight-wave tile's Stream-K)

BK = {S.F16: 64, S.BF16: 64, S.F32: 32, S.I8: 128}  # elements of one K-step


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shares", [2, 3, 5, 8])
@pytest.mark.parametrize("b_col", [False, True])
def test_equal_shares_every_count(dtype, shares, b_col):
    """Every tile of the eight-wave 256x256 config cut into 2 to 8 equal k
    shares, each on the data-parallel loop, summed by the wave-per-block
    kernel: partial tiles at the M and N edges (520 x 272: 3 x 2 tiles), 42
    K-steps with a partial last one (shares of 5 to 21 steps, the last share
    holding the tail), bias + ReLU (the bias in share 0 only)."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 520, 272, 41 * BK[dtype] + ce, seed=60 + shares, b_col=b_col, bias=True, relu=True)
    T.tcm_set_option("force_config", 0)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("grid_shares", shares)
    g, C, plan = _run(p)
    assert "config=0" in plan and f"split={shares}" in plan and f"grid={6 * shares}" in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("b_col", [False, True])
def test_equal_shares_column_major_a(dtype, b_col):
    """The equal shares with A stored column-major (the [k][m] staging), the
    planner's share count (two tiles: eight shares), padded lda."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 208, 304, 29 * BK[dtype] + ce, seed=70, a_col=True, b_col=b_col, bias=True,
                        lda=208 + ce)
    T.tcm_set_option("force_config", 0)
    T.tcm_set_option("force_mode", 2)
    g, C, plan = _run(p)
    assert "config=0" in plan and "split=8" in plan and "a_col=1" in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
def test_equal_shares_fixed_sum_order(dtype):
    """The shares are added in share order: the float result is the same bits
    on every call, and int8 (exact integer sums) equals the data-parallel
    result bit for bit."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 512, 512, 48 * BK[dtype], seed=6, bias=True, relu=True)
    T.tcm_set_option("force_config", 0)
    T.tcm_set_option("force_mode", 1)
    g, C_dp, _ = _run(p)
    T.tcm_set_option("force_mode", 2)
    _, C_s1, plan = _run(p)
    _, C_s2, _ = _run(p)
    assert "split=8" in plan
    check(p, g, C_s1)
    assert np.array_equal(C_s1, C_s2), "equal-shares result differs between calls"
    if dtype == S.I8:
        assert np.array_equal(C_dp, C_s1), "int8 data-parallel and equal shares differ"


@pytest.mark.parametrize("dtype", DTYPES)
def test_eight_wave_persistent_streamk_when_grid_given(dtype):
    """A given Stream-K grid keeps the eight-wave config's persistent kernel
    (segments cross tile boundaries; last arrival or fix-up kernel)."""
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 300, 528, 20 * BK[dtype] + ce, seed=8, bias=True, relu=True)
    T.tcm_set_option("force_config", 0)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("sk_grid", 7)
    g, C, plan = _run(p)
    assert "config=0" in plan and "mode=streamk" in plan and "split=" not in plan
    check(p, g, C)


# ------------------------------------------------------------ generic kernel

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("layout", ["odd_k", "a_col", "both_col", "padded_ld", "unaligned"])
def test_generic_path(dtype, layout):
    """Shapes and layouts the tiled kernel does not take: same results, slower."""
    kw = {}
    if layout == "odd_k":
        p = S.small_problem(dtype, 70, 90, 37, seed=3, bias=True, relu=True)
    elif layout == "a_col":
        p = S.small_problem(dtype, 130, 72, 96, seed=4, a_col=True, bias=True)
    elif layout == "both_col":
        p = S.small_problem(dtype, 65, 129, 100, seed=5, a_col=True, b_col=True, relu=True)
    elif layout == "padded_ld":
        p = S.small_problem(dtype, 100, 60, 75, seed=6, lda=81, ldb=67, ldc=70, bias=True)
    else:
        p = S.small_problem(dtype, 128, 128, 128, seed=7, bias=True)
        kw = dict(a_offset=1, b_offset=3, c_offset=1)
    g, C, plan = _run(p, **kw)
    assert "kernel=generic" in plan
    check(p, g, C)
    if layout == "padded_ld":
        check_padding_untouched(p, C, -7 if dtype == S.I8 else float("nan"))


BYTE_OFFSETS = [dict(A=2), dict(B=3), dict(C=1), dict(bias=1), dict(A=1, B=1, C=3, bias=2)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("offs", BYTE_OFFSETS, ids=lambda d: "-".join(f"{k}{v}" for k, v in d.items()))
def test_generic_path_pointers_not_aligned_to_their_element(dtype, offs):
    """Pointers at any byte address (e.g. an f32 A two bytes in, a C one
    byte in) are served, not rejected: the generic kernel's byte-access
    instance against the oracle, with bias + ReLU and ragged edges."""
    from gpu_util import run_tcm_bytes
    p = S.small_problem(dtype, 70, 66, 100, seed=8, bias=True, relu=True)
    say(f"[case] byte offsets {offs} {p.name} dtype={dtype}")
    g = S.generate(p)
    C, plan = run_tcm_bytes(p, g, offs)
    say(f"       plan: {plan}")
    assert "kernel=generic" in plan
    check(p, g, C)


@pytest.mark.parametrize("variant", [(S.F16, "f16", True), (S.BF16, "bf16", True), (S.F32, "acc", True)],
                         ids=["f16-Cf16", "bf16-Cbf16", "f32-Cf32"])
def test_generic_path_unaligned_16bit_c_with_c_in(variant):
    """A 16-bit C (read as C_in, then written) one byte past its element boundary."""
    from gpu_util import run_tcm_bytes
    dtype, c_type, accum = variant
    p = S.small_problem(dtype, 40, 34, 48, seed=9, bias=True, c_type=c_type, accum=accum, ldc=37)
    say(f"[case] unaligned C with C_in {p.name} c_type={c_type}")
    g = S.generate(p)
    C, plan = run_tcm_bytes(p, g, dict(C=1))
    assert "kernel=generic" in plan
    check(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
def test_forced_generic_matches_tiled(dtype):
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    p = S.small_problem(dtype, 200, 144, 20 * ce, seed=9, bias=True, relu=True)
    g, C_tile, plan = _run(p)
    assert "kernel=tile" in plan
    T.tcm_set_option("generic", 1)
    _, C_gen, plan = _run(p)
    assert "kernel=generic" in plan
    check(p, g, C_gen)
    if dtype == S.I8:
        assert np.array_equal(C_tile, C_gen)


# ------------------------------------------------------------ degenerate cases

@pytest.mark.parametrize("dtype", DTYPES)
def test_k_zero_gives_epilogue_of_bias(dtype):
    p = S.small_problem(dtype, 5, 7, 0, seed=1, bias=True, relu=True, lda=1)
    g, C, _ = _run(p)
    check(p, g, C)


@pytest.mark.parametrize("dtype", DTYPES)
def test_one_by_one(dtype):
    ce = {S.F16: 8, S.BF16: 8, S.F32: 4, S.I8: 16}[dtype]
    for K in (1, ce):
        p = S.small_problem(dtype, 1, 1, K, seed=2, bias=True)
        g, C, _ = _run(p)
        check(p, g, C)


def test_empty_problem_leaves_c_untouched():
    C = torch.full((16,), 3.0, device="cuda")
    A = torch.zeros(16, dtype=torch.float16, device="cuda")
    st = T.tcm_gemm(0, 4, 4, A.data_ptr(), 4, A.data_ptr(), 4, C.data_ptr(), 4, 0, None, 0, None)
    assert st == T.TCM_OK
    torch.cuda.synchronize()
    assert torch.all(C == 3.0)


def test_block_sum_printed_value_on_gpu():
    """The pages' worked example, through the engine: sum(arange(256)) = 32640."""
    for dtype, tdt in ((S.F16, torch.float16), (S.BF16, torch.bfloat16), (S.F32, torch.float32)):
        a = torch.arange(256, dtype=tdt, device="cuda").reshape(1, 256)
        b = torch.ones((256, 8), dtype=tdt, device="cuda")
        say(f"[case] block sum dtype={dtype}")
        C = T.gemm(a, b)
        torch.cuda.synchronize()
        assert torch.all(C == 32640.0), C
    a = (torch.arange(256, device="cuda") - 128).to(torch.int8).reshape(1, 256)
    C = T.gemm(a, torch.ones((256, 16), dtype=torch.int8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(C == -128)


def test_torch_convenience_layouts():
    """gemm() reads row/column-major views from strides."""
    torch.manual_seed(0)
    A = torch.randn(96, 64, device="cuda").half()
    Bt = torch.randn(80, 64, device="cuda").half()
    say("[case] torch convenience: B as transposed view")
    C = T.gemm(A, Bt.t())
    ref = A.float().cpu() @ Bt.float().cpu().t()
    assert torch.allclose(C.cpu(), ref, atol=1e-2, rtol=1e-3)
    C2 = T.gemm(A.t().contiguous().t(), Bt.t())  # column-major A view -> generic kernel
    assert torch.allclose(C2.cpu(), ref, atol=1e-2, rtol=1e-3)


# ------------------------------------------------------- wider epilogues: C_in and a 16-bit C

# (element type, C type, accumulate) combinations; int8 keeps an int32 C
EPI_VARIANTS = [(S.F16, "f16", True), (S.F16, "bf16", False), (S.BF16, "bf16", True), (S.BF16, "acc", True),
                (S.F32, "f16", True), (S.F32, "acc", True), (S.I8, "acc", True)]


def _epi_id(v):
    return f"{S.DTYPE_NAMES[v[0]]}-C{v[1]}-{'accum' if v[2] else 'store'}"


@pytest.mark.parametrize("variant", EPI_VARIANTS, ids=_epi_id)
@pytest.mark.parametrize("config", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("mode", [1, 2])
def test_init_tensor_and_16bit_c_every_config_and_mode(variant, config, mode):
    """C_in as the initial value and/or C stored in f16 / bf16, on every tile
    config in both modes, ragged edges, bias + ReLU, padded ldc (whose padding
    must keep C_in's values)."""
    dtype, c_type, accum = variant
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", mode)
    # N and K multiples of the 16-byte chunk so every config can take the row-major B
    p = S.small_problem(dtype, 300, 272, 208, seed=40 + config, bias=True, relu=True, ldc=280, c_type=c_type,
                        accum=accum)
    g, C, plan = _run(p)
    assert f"config={config}" in plan and ("mode=dp" if mode == 1 else "mode=streamk") in plan
    err = check(p, g, C)
    say(f"       normalised error {err:.3e}")
    if accum:
        cin = g["C_in"].reshape(p.M, p.LDC)[:, p.N:]
        pad = C[:, p.N:]
        if c_type != "acc":
            code = S.C_TYPE_CODE[c_type]
            want = (cin.view(np.float16).astype(np.float32) if code == S.F16 else
                    torch.from_numpy(cin.view(np.int16).copy()).view(torch.bfloat16).float().numpy())
        else:
            want = cin
        assert np.array_equal(pad, want), "C's padding columns changed"


@pytest.mark.parametrize("variant", EPI_VARIANTS, ids=_epi_id)
@pytest.mark.parametrize("config", [4, 5, 6])
@pytest.mark.parametrize("fixup", [1, 2])
def test_init_tensor_streamk_many_segments(variant, config, fixup):
    """Only the k = 0 segment of a split tile may add C_in (and the bias),
    whichever way the split tile is summed."""
    dtype, c_type, accum = variant
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("sk_fixup", fixup)
    T.tcm_set_option("sk_grid", 37)
    K = 1024 if dtype != S.I8 else 2048
    p = S.small_problem(dtype, 96, 128, K, seed=50, bias=True, c_type=c_type, accum=accum)
    g, C, plan = _run(p)
    assert "mode=streamk" in plan
    check(p, g, C)


@pytest.mark.parametrize("variant", EPI_VARIANTS, ids=_epi_id)
@pytest.mark.parametrize("layout", ["a_col", "odd_ld", "unaligned_c"])
def test_init_tensor_generic_path(variant, layout):
    """The generic kernel's C_in read and 16-bit store (any layout, ld, alignment)."""
    dtype, c_type, accum = variant
    kw = {}
    if layout == "a_col":
        p = S.small_problem(dtype, 70, 50, 37, seed=60, a_col=True, bias=True, relu=True, c_type=c_type, accum=accum)
    elif layout == "odd_ld":
        p = S.small_problem(dtype, 65, 33, 41, seed=61, lda=43, ldb=35, ldc=37, c_type=c_type, accum=accum)
    else:
        p = S.small_problem(dtype, 64, 64, 64, seed=62, bias=True, c_type=c_type, accum=accum)
        kw = {"c_offset": 1}
    g, C, plan = _run(p, **kw)
    assert "kernel=generic" in plan
    check(p, g, C)


@pytest.mark.parametrize("variant", EPI_VARIANTS, ids=_epi_id)
def test_init_tensor_k_zero(variant):
    """K = 0: C = epi(C_in + bias), exactly (up to the 16-bit output rounding)."""
    dtype, c_type, accum = variant
    p = S.small_problem(dtype, 40, 24, 0, seed=70, bias=True, relu=True, lda=1, ldc=27, c_type=c_type, accum=accum)
    g, C, plan = _run(p)
    check(p, g, C)


def test_init_tensor_dp_and_streamk_bit_exact_int8():
    """int8 with C_in: data-parallel and Stream-K give identical C."""
    p = S.small_problem(S.I8, 256, 256, 4096, seed=80, bias=True, relu=True, accum=True)
    out = []
    for mode in (1, 2):
        T.tcm_set_option("force_mode", mode)
        g, C, plan = _run(p)
        check(p, g, C)
        out.append(C)
    assert np.array_equal(out[0], out[1])


def test_torch_convenience_accumulate_and_16bit_out():
    """gemm(..., accumulate=True) adds into C; out_dtype picks a 16-bit C."""
    torch.manual_seed(0)
    A = torch.randn(130, 96, device="cuda").half()
    B = torch.randn(96, 72, device="cuda").half()
    C0 = torch.randn(130, 72, device="cuda")
    C = C0.clone()
    T.gemm(A, B, C, accumulate=True)
    ref = C0 + A.float() @ B.float()
    assert torch.allclose(C, ref, atol=1e-2, rtol=1e-3)
    Ch = T.gemm(A, B, out_dtype=torch.bfloat16)
    assert Ch.dtype == torch.bfloat16
    assert torch.allclose(Ch.float(), (A.float() @ B.float()), atol=0.05, rtol=2 ** -7)


# ------------------------------------------------------------ auto-tuning

@pytest.mark.parametrize("dtype", [S.F16, S.I8])
def test_autotune_choice_is_used_and_correct(dtype):
    """tcm_tune times the candidates, records the fastest; the next tcm_gemm on
    the same signature launches exactly that plan and stays correct."""
    from gpu_util import to_device
    saved = T.tcm_tune_table()  # the shipped table, restored afterwards
    T.tcm_tune_clear()
    try:
        p = S.small_problem(dtype, 768, 512, 1024, seed=110, bias=True, relu=True)
        g = S.generate(p)
        say(f"[case] autotune {p.name}")
        ka, pa = to_device(g["A"], dtype)
        kb, pb = to_device(g["B"], dtype)
        kbias = torch.from_numpy(g["bias"].copy()).cuda()
        C = torch.empty((p.M, p.LDC), dtype=torch.int32 if dtype == S.I8 else torch.float32, device="cuda")
        epi = T.TCM_EPI_BIAS | T.TCM_EPI_RELU
        st, best = T.tcm_tune(p.M, p.N, p.K, pa, p.LDA, pb, p.LDB, C.data_ptr(), p.LDC, dtype, kbias.data_ptr(), epi, 3,
                              torch.cuda.current_stream().cuda_stream)
        assert st == T.TCM_OK and best["kernel"] == 1
        table = T.tcm_tune_table().strip().splitlines()
        assert len(table) == 1 and table[0].startswith("tcm-tune-2 ") and table[0].endswith(f" {p.M} {p.N} {p.K}")
        say(f"       tuned: {table[0]}")
        C2, plan = run_tcm(p, g)
        assert f"config={best['config']} " in plan and " tuned=" in plan
        assert ("mode=dp" if best["mode"] == 1 else "mode=streamk") in plan
        check(p, g, C2)
    finally:
        T.tcm_tune_clear()
        assert T.tcm_tune_load(saved) == T.TCM_OK
