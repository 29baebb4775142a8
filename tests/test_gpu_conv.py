"""GPU parity of tcm_conv2d (the implicit-GEMM Conv2d + bias + ReLU) against
the CPU oracle's direct convolution, through the C ABI.

Bars as for the GEMM, with the GEMM's K being R*S*C: int8 bit-exact; float
types max|y - y_ref| / (R*S*C * max|x| * max|f| + max|bias|) <= 1e-3 (f16,
bf16) or 1e-5 (f32), plus half an output ulp for a 16-bit y.  Outputs sit in
a buffer with sentinels after the end, so a store past y shows up."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
import tensor_core_mixed_amd as T
from gpu_util import OUT_U, TOL, say, to_device, value_range

pytestmark = pytest.mark.gpu

DTYPES = [S.F16, S.BF16, S.F32, S.I8]
BKE = {S.F16: 64, S.BF16: 64, S.F32: 32, S.I8: 128}   # K-step in elements: channels the tiled gather needs
_C_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}
TAIL = 64


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    T.tcm_set_option("force_mode", 0)
    T.tcm_set_option("force_config", -1)
    T.tcm_set_option("sk_grid", 0)
    T.tcm_set_option("generic", 0)
    T.tcm_set_option("sk_fixup", 0)


def run_conv(p, g, x_offset=0, x_byte_offset=0):
    """tcm_conv2d on p's inputs; returns y as an (N*P*Q, K) float / int array and the plan.
    x_offset shifts x by elements, x_byte_offset by bytes (any address)."""
    dt = p.dtype
    if x_byte_offset:
        from gpu_util import _bytes_on_device
        kx, px = _bytes_on_device(g["x"], x_byte_offset)
    else:
        kx, px = to_device(g["x"], dt, x_offset)
    kf, pf = to_device(g["f"], dt)
    kb = torch.from_numpy(g["bias"].copy()).cuda() if g["bias"] is not None else None
    c_t = _C_TORCH.get(p.c_type, torch.int32 if dt == S.I8 else torch.float32)
    M = p.N * p.P * p.Q
    y = torch.full((M * p.K + TAIL,), -7 if dt == S.I8 else float("nan"), dtype=c_t, device="cuda")
    code = dt | {"acc": 0, "f16": T.TCM_C_F16, "bf16": T.TCM_C_BF16}[p.c_type]
    epi = (T.TCM_EPI_BIAS if p.bias else 0) | (T.TCM_EPI_RELU if p.relu else 0)
    say(f"[case] conv {p.name} pad={p.pad} stride={p.stride} dil={p.dil} c_type={p.c_type} bias={p.bias} "
        f"relu={p.relu} x_offset={x_offset} x_byte_offset={x_byte_offset} force_config={T.tcm_get_option('force_config')} "
        f"force_mode={T.tcm_get_option('force_mode')} generic={T.tcm_get_option('generic')}")
    st = T.tcm_conv2d(p.N, p.H, p.W, p.C, p.K, p.R, p.S, p.pad[0], p.pad[1], p.stride[0], p.stride[1], p.dil[0],
                      p.dil[1], px, pf, y.data_ptr(), code, kb.data_ptr() if kb is not None else None, epi,
                      torch.cuda.current_stream().cuda_stream)
    assert st == T.TCM_OK, T.tcm_status_string(st)
    plan = T.tcm_last_plan()
    say(f"       plan: {plan}")
    torch.cuda.synchronize()
    out = (y.float() if c_t in (torch.float16, torch.bfloat16) else y).cpu().numpy()
    tail = out[M * p.K:]
    assert np.all(np.isnan(tail)) if dt != S.I8 else np.all(tail == -7), "wrote past the end of y"
    del kx, kf, kb
    return out[:M * p.K].reshape(M, p.K), plan


def check_conv(p, g, y, mm=None, kk=None):
    """Compare y with the oracle on all outputs or at (mm, kk); returns the normalised error."""
    o = oracle.get()
    kw = dict(pad=p.pad, stride=p.stride, dil=p.dil, bias=g["bias"], relu=p.relu)
    if mm is None:
        ref = o.conv2d(g["x"], g["f"], p.dtype, **kw).reshape(y.shape)
        got = y
        assert p.dtype == S.I8 or np.all(np.isfinite(got)), "unwritten or non-finite outputs"
    else:
        ref = o.conv2d_entries(g["x"], g["f"], p.dtype, mm, kk, **kw)
        got = y[mm, kk]
    if p.dtype == S.I8:
        bad = np.flatnonzero(got.reshape(-1) != ref.reshape(-1))
        assert bad.size == 0, f"{p.name}: {bad.size} int8 mismatches, first at {bad[0]}"
        return 0.0
    diff = np.abs(got.astype(np.float64) - ref)
    u = OUT_U[p.c_type]
    taps = p.R * p.S * p.C
    if taps == 0:
        assert np.all(diff <= u * np.abs(ref)), f"{p.name}: no taps must give epi(bias)"
        return 0.0
    denom = taps * value_range(g["x"], p.dtype) * value_range(g["f"], p.dtype)
    if g["bias"] is not None:
        denom += float(np.max(np.abs(g["bias"])))
    err = float(np.max(diff - u * np.abs(ref))) / denom if diff.size else 0.0
    assert err <= TOL[p.dtype], f"{p.name}: normalised error {err:.3e} > {TOL[p.dtype]:.0e}"
    return max(err, 0.0)


def _run_check(p, **kw):
    g = S.generate_conv(p)
    y, plan = run_conv(p, g, **kw)
    check_conv(p, g, y)
    return y, plan


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("config", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("mode", [1, 2])
def test_conv_every_config_and_mode(dtype, config, mode):
    """Every tile config in both modes: 3x3, padding 1, ragged pixel count and channel count."""
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", mode)
    p = S.small_conv(dtype, 2, 9, 7, 2 * BKE[dtype], 40, 3, 3, pad=(1, 1), seed=120 + config, bias=True, relu=True)
    _, plan = _run_check(p)
    assert "kernel=conv" in plan and f"config={config}" in plan


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("config", [1, 4, 5, 6])
def test_conv_streamk_fixup_kernel(dtype, config):
    """Stream-K convolution with many segments per tile, split tiles summed
    by the second kernel."""
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("sk_grid", 41)
    T.tcm_set_option("sk_fixup", 2)
    p = S.small_conv(dtype, 2, 9, 7, 2 * BKE[dtype], 40, 3, 3, pad=(1, 1), seed=140 + config, bias=True, relu=True)
    _, plan = _run_check(p)
    assert "kernel=conv" in plan and "mode=streamk" in plan and "fixup=kernel" in plan


GEOMETRIES = [  # (N, H, W, K, R, S, pad, stride, dil)
    (1, 8, 8, 64, 1, 1, (0, 0), (1, 1), (1, 1)),      # 1x1: a plain product
    (2, 11, 13, 48, 3, 3, (0, 0), (1, 1), (1, 1)),    # no padding
    (2, 12, 12, 32, 3, 3, (1, 1), (2, 2), (1, 1)),    # stride 2
    (1, 15, 14, 24, 3, 3, (2, 2), (1, 1), (2, 2)),    # dilation 2
    (1, 9, 16, 20, 1, 7, (0, 3), (1, 1), (1, 1)),     # 1x7
    (1, 16, 9, 20, 7, 1, (3, 0), (1, 1), (1, 1)),     # 7x1
    (2, 17, 19, 33, 5, 5, (2, 1), (3, 2), (1, 2)),    # everything at once, odd K
    (1, 3, 3, 16, 3, 3, (4, 4), (1, 1), (1, 1)),      # padding wider than the input: border pixels see only zeros
    (1, 5, 5, 8, 5, 5, (0, 0), (1, 1), (1, 1)),       # one output pixel
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("geo", GEOMETRIES, ids=[f"g{i}" for i in range(len(GEOMETRIES))])
def test_conv_geometry(dtype, geo):
    N, H, W, K, R, S_, pad, stride, dil = geo
    p = S.small_conv(dtype, N, H, W, BKE[dtype], K, R, S_, pad=pad, stride=stride, dil=dil, seed=130, bias=True,
                     relu=True)
    _, plan = _run_check(p)
    assert "kernel=conv" in plan


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("C", [3, 8, 40, 200])
def test_conv_generic_channels(dtype, C):
    """Channel counts that are not a multiple of the K-step run on the generic kernel."""
    if C == 200 and dtype == S.F32:
        C = 52
    p = S.small_conv(dtype, 2, 10, 9, C, 36, 3, 3, pad=(1, 1), stride=(1, 2), seed=140, bias=True, relu=True)
    _, plan = _run_check(p)
    assert "kernel=generic" in plan and "conv=1" in plan


@pytest.mark.parametrize("dtype", DTYPES)
def test_conv_generic_matches_tiled(dtype):
    """The same call on both kernels: int8 identical, floats both within the bar."""
    p = S.small_conv(dtype, 2, 10, 10, BKE[dtype], 72, 3, 3, pad=(1, 1), seed=141, bias=True, relu=True)
    g = S.generate_conv(p)
    y1, plan1 = run_conv(p, g)
    check_conv(p, g, y1)
    T.tcm_set_option("generic", 1)
    y2, plan2 = run_conv(p, g)
    check_conv(p, g, y2)
    assert "kernel=conv" in plan1 and "kernel=generic" in plan2
    if dtype == S.I8:
        assert np.array_equal(y1, y2)


@pytest.mark.parametrize("dtype", DTYPES)
def test_conv_unaligned_input_goes_generic(dtype):
    p = S.small_conv(dtype, 1, 8, 8, BKE[dtype], 16, 3, 3, pad=(1, 1), seed=142, bias=True)
    g = S.generate_conv(p)
    y, plan = run_conv(p, g, x_offset=1)
    assert "kernel=generic" in plan
    check_conv(p, g, y)


@pytest.mark.parametrize("dtype", DTYPES)
def test_conv_input_not_aligned_to_its_element(dtype):
    """x one byte past an element boundary (three for f32): served by the
    generic kernel's byte-access instance, not rejected."""
    p = S.small_conv(dtype, 1, 7, 9, 5, 12, 3, 3, pad=(1, 0), seed=143, bias=True, relu=True)
    g = S.generate_conv(p)
    y, plan = run_conv(p, g, x_byte_offset=3 if dtype == S.F32 else 1)
    assert "kernel=generic" in plan
    check_conv(p, g, y)


@pytest.mark.parametrize("variant", [(S.F16, "f16"), (S.BF16, "bf16"), (S.F32, "bf16")], ids=["f16", "bf16", "f32-bf16"])
@pytest.mark.parametrize("mode", [1, 2])
def test_conv_16bit_output(variant, mode):
    dtype, c_type = variant
    T.tcm_set_option("force_mode", mode)
    p = S.small_conv(dtype, 2, 9, 9, BKE[dtype], 64, 3, 3, pad=(1, 1), seed=143, bias=True, relu=True, c_type=c_type)
    _run_check(p)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("sk_grid", [3, 50, 300])
@pytest.mark.parametrize("config", [4, 5, 6])
def test_conv_streamk_split_tiles(dtype, sk_grid, config):
    """Stream-K with grids that split tiles at arbitrary taps."""
    T.tcm_set_option("force_config", config)
    T.tcm_set_option("force_mode", 2)
    T.tcm_set_option("sk_grid", sk_grid)
    p = S.small_conv(dtype, 2, 8, 8, 2 * BKE[dtype], 64, 3, 3, pad=(1, 1), seed=144, bias=True, relu=True)
    _, plan = _run_check(p)
    assert "mode=streamk" in plan


def test_conv_int8_dp_and_streamk_bit_exact():
    p = S.small_conv(S.I8, 2, 14, 14, 256, 128, 3, 3, pad=(1, 1), seed=145, bias=True, relu=True)
    g = S.generate_conv(p)
    outs = []
    for mode in (1, 2):
        T.tcm_set_option("force_mode", mode)
        y, plan = run_conv(p, g)
        check_conv(p, g, y)
        outs.append(y)
    assert np.array_equal(outs[0], outs[1])


def test_conv_no_channels_gives_the_bias():
    p = S.small_conv(S.F32, 1, 4, 4, 0, 8, 3, 3, pad=(1, 1), seed=146, bias=True, relu=False)
    _run_check(p)


def test_conv_empty_outputs():
    x = torch.zeros(64, dtype=torch.float16, device="cuda")
    assert T.tcm_conv2d(0, 4, 4, 64, 8, 3, 3, 1, 1, 1, 1, 1, 1, x.data_ptr(), x.data_ptr(), x.data_ptr(), 0, None, 0,
                        None) == T.TCM_OK
    assert T.tcm_conv2d(1, 4, 4, 64, 0, 3, 3, 1, 1, 1, 1, 1, 1, x.data_ptr(), x.data_ptr(), None, 0, None, 0,
                        None) == T.TCM_OK


def test_torch_convenience_conv2d():
    torch.manual_seed(3)
    x = torch.randn(2, 10, 12, 64, device="cuda").half()
    f = torch.randn(32, 3, 3, 64, device="cuda").half()
    b = torch.randn(32, device="cuda")
    y = T.conv2d(x, f, bias=b, relu=True, padding=1, stride=(1, 2))
    ref = torch.nn.functional.conv2d(x.float().permute(0, 3, 1, 2), f.float().permute(0, 3, 1, 2), b, padding=1,
                                     stride=(1, 2)).relu().permute(0, 2, 3, 1)
    assert y.shape == ref.shape
    assert torch.allclose(y, ref, atol=2e-2, rtol=1e-3)
    y16 = T.conv2d(x, f, bias=b, relu=True, padding=1, stride=(1, 2), out_dtype=torch.float16)
    assert torch.allclose(y16.float(), ref, atol=5e-2, rtol=2e-3)


@pytest.mark.parametrize("name", list(S.CONV_WORKLOADS))
def test_conv_full_size_sampled(name):
    """The measured convolutions at full size, in the planner's launch: sampled outputs against the oracle."""
    p = S.CONV_WORKLOADS[name]
    g = S.generate_conv(p)
    y, plan = run_conv(p, g)
    assert "kernel=conv" in plan
    mm, kk = S.sample_conv_entries(p)
    check_conv(p, g, y, mm, kk)
    assert p.dtype == S.I8 or np.all(np.isfinite(y)), "unwritten outputs"


N_RANDOM = 100


def draw_conv(seed):
    """Random convolution `seed`: element type, channels on the K-step grid
    (the tiled gather) or off it (the generic kernel), 1x1 to 3x3 filters,
    padding, stride and dilation up to 2, 1 to 159 output channels, bias,
    ReLU, C's type, and now and then a forced tile config and mode."""
    rng = np.random.default_rng(55000 + seed)
    dt = [S.F16, S.BF16, S.F32, S.I8][int(rng.integers(4))]
    C = BKE[dt] * int(rng.integers(1, 4)) if rng.random() < 0.8 else int(rng.integers(1, 40))
    R, Sd = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    pad = (int(rng.integers(0, R)), int(rng.integers(0, Sd)))
    stride = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
    dil = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
    H, W = int(rng.integers(R * dil[0], 16)), int(rng.integers(Sd * dil[1], 16))
    N, K = int(rng.integers(1, 5)), int(rng.integers(1, 160))
    c_type = "acc" if dt in (S.I8, S.F32) else ["acc", "f16", "bf16"][int(rng.integers(3))]
    if c_type == "bf16" and dt == S.F16:
        c_type = "f16"
    if c_type == "f16" and dt == S.BF16:
        c_type = "bf16"
    p = S.small_conv(dt, N, H, W, C, K, R, Sd, pad=pad, stride=stride, dil=dil, seed=700 + seed,
                     bias=bool(rng.integers(2)), relu=bool(rng.integers(2)), c_type=c_type)
    opts = {}
    r = rng.random()
    if r < 0.3:
        opts = {"force_config": int(rng.integers(0, T.tcm_config_count())), "force_mode": int(rng.integers(1, 3))}
    elif r < 0.4:
        opts = {"force_mode": 2}
    return p, opts


@pytest.mark.parametrize("seed", range(N_RANDOM))
def test_random_conv_case(seed):
    p, opts = draw_conv(seed)
    for k, v in opts.items():
        assert T.tcm_set_option(k, v) == T.TCM_OK
    _run_check(p)
