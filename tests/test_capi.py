"""The C-ABI library on the CPU: exports, argument checks, the planner and the
Stream-K partition.  No kernel runs here (no GPU in this process)."""
import os
import re
import subprocess

import numpy as np
import pytest

import tensor_core_mixed_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tcm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tcm_[a-z_]+)\s*\(", text)))


@pytest.fixture(autouse=True)
def _planner_model_without_the_table():
    """The planner tests here check the cost model itself: the tuning table
    (the shipped one included) is off unless a test turns it on; a test that
    edits the table gets the process's table back afterwards."""
    T.tcm_plan(64, 64, 64, 64, 64, 64, 0)  # the first plan loads the shipped table
    before = T.tcm_tune_table()
    T.tcm_set_option("tuned", 0)
    yield
    T.tcm_set_option("tuned", 1)
    T.tcm_tune_clear()
    assert T.tcm_tune_load(before) == T.TCM_OK


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "tcm_gemm" in names and len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", T.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tcm_[a-z_]+)\b", out))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    lib = T.lib()
    for n in names:
        getattr(lib, n)


def test_status_strings_and_version():
    for s in range(5):
        assert T.tcm_status_string(s).startswith("TCM_")
    assert "unknown" in T.tcm_status_string(99)
    assert "gfx950" in T.tcm_version()


BAD = [  # (M, N, K, lda, ldb, ldc, dtype, epilogue, A, B, C, bias)
    (-1, 4, 4, 4, 4, 4, 0, 0, 16, 16, 16, 0),           # negative size
    (4, 4, 4, 3, 4, 4, 0, 0, 16, 16, 16, 0),            # lda < K
    (4, 4, 4, 4, 3, 4, 0, 0, 16, 16, 16, 0),            # ldb < N
    (4, 4, 8, 8, 4, 4, T.TCM_B_COLMAJOR, 0, 16, 16, 16, 0),  # col-major B needs ldb >= K
    (4, 4, 4, 4, 4, 3, 0, 0, 16, 16, 16, 0),            # ldc < N
    (4, 4, 4, 4, 4, 4, 7, 0, 16, 16, 16, 0),            # unknown element type
    (4, 4, 4, 4, 4, 4, 1 << 12, 0, 16, 16, 16, 0),      # unknown flag
    (4, 4, 4, 4, 4, 4, 0, 8, 16, 16, 16, 0),            # unknown epilogue
    (4, 4, 4, 4, 4, 4, T.TCM_C_F16 | T.TCM_C_BF16, 0, 16, 16, 16, 0),  # two output types
    (4, 4, 4, 4, 4, 4, T.TCM_I8_I32 | T.TCM_C_F16, 0, 16, 16, 16, 0),  # 16-bit C for int8
    (4, 4, 4, 4, 4, 4, 0, 1, 16, 16, 16, 0),            # bias flag without bias
    (4, 4, 4, 4, 4, 4, 0, 0, 0, 16, 16, 0),             # NULL A
    (4, 4, 4, 4, 4, 4, 0, 0, 16, 0, 16, 0),             # NULL B
    (4, 4, 4, 4, 4, 4, 0, 0, 16, 16, 0, 0),             # NULL C
    (4, 4, 4, 4, 4, 4, 0, 0, 4096, 16, 4100, 0),        # C overlaps A
    (4, 4, 4, 4, 4, 4, 0, 0, 16, 4096, 4100, 0),        # C overlaps B
    (4, 4, 4, 4, 4, 4, 0, 1, 16, 256, 4096, 4100),      # C overlaps bias
]


@pytest.mark.parametrize("args", BAD)
def test_invalid_arguments_rejected_before_any_hip_call(args):
    M, N, K, lda, ldb, ldc, dt, epi, A, B, C, bias = args
    st = T.tcm_gemm(M, N, K, A or None, lda, B or None, ldb, C or None, ldc, dt, bias or None, epi, None)
    assert st == T.TCM_ERR_INVALID_VALUE


def test_empty_problem_is_ok_without_device():
    # nothing is read or written for M == 0 or N == 0, so NULL pointers are fine
    assert T.tcm_gemm(0, 5, 3, None, 3, None, 5, None, 5, 0, None, 0, None) == T.TCM_OK
    assert T.tcm_gemm(0, 5, 3, 16, 3, 16, 5, 4096, 5, 0, None, 0, None) == T.TCM_OK
    assert T.tcm_gemm(5, 0, 3, 16, 3, 16, 5, 4096, 5, 0, None, 0, None) == T.TCM_OK


def test_valid_call_without_device_reports_hip_error():
    # real-looking (fake) pointers: checks pass, the first HIP call fails
    st = T.tcm_gemm(64, 64, 64, 1 << 20, 64, 2 << 20, 64, 3 << 20, 64, 0, None, 0, None)
    assert st == T.TCM_ERR_HIP
    # every epilogue combination, and C at any address: element-misaligned
    # pointers are served (single-byte accesses on the generic kernel)
    for epi in range(8):
        for flags in (0, T.TCM_C_F16, T.TCM_C_BF16):
            st = T.tcm_gemm(64, 64, 64, 1 << 20, 64, 2 << 20, 64, (3 << 20) + 2, 64, T.TCM_BF16_F32 | flags,
                            4 << 20, epi, None)
            assert st == T.TCM_ERR_HIP, (epi, flags)


@pytest.mark.parametrize("ptrs", [dict(A=(1 << 20) + 1), dict(B=(2 << 20) + 3), dict(C=(3 << 20) + 1),
                                  dict(C=(3 << 20) + 2), dict(bias=(4 << 20) + 1)],
                         ids=lambda d: ",".join(f"{k}+{v & 0xff}" for k, v in d.items()))
@pytest.mark.parametrize("dtype", [T.TCM_F16_F32, T.TCM_F32_F32, T.TCM_I8_I32, T.TCM_BF16_F32 | T.TCM_C_BF16])
def test_misaligned_pointers_are_valid_requests(ptrs, dtype):
    """No pointer needs any alignment: the checks pass and the call reaches its first HIP call."""
    a = dict(A=1 << 20, B=2 << 20, C=3 << 20, bias=4 << 20)
    a.update(ptrs)
    st = T.tcm_gemm(64, 64, 64, a["A"], 64, a["B"], 64, a["C"], 64, dtype, a["bias"], T.TCM_EPI_BIAS, None)
    assert st == T.TCM_ERR_HIP


def test_options():
    assert T.tcm_get_option("force_mode") == 0
    assert T.tcm_set_option("force_mode", 2) == T.TCM_OK and T.tcm_get_option("force_mode") == 2
    assert T.tcm_set_option("force_mode", 3) == T.TCM_ERR_INVALID_VALUE
    assert T.tcm_set_option("no_such_key", 1) == T.TCM_ERR_INVALID_VALUE
    assert T.tcm_get_option("no_such_key") == -2
    assert T.tcm_set_option("force_config", T.tcm_config_count()) == T.TCM_ERR_INVALID_VALUE
    assert T.tcm_set_option("force_mode", 0) == T.TCM_OK
    assert T.tcm_get_option("sk_fixup") == 0
    assert T.tcm_set_option("sk_fixup", 2) == T.TCM_OK and T.tcm_get_option("sk_fixup") == 2
    assert T.tcm_set_option("sk_fixup", 3) == T.TCM_ERR_INVALID_VALUE
    assert T.tcm_set_option("sk_fixup", 0) == T.TCM_OK


def test_config_table():
    n = T.tcm_config_count()
    assert n >= 3
    for i in range(n):
        for dt, bk in ((0, 64), (1, 64), (2, 32), (3, 128)):
            bm, bn, k, waves = T.tcm_config_info(i, dt)
            assert k == bk and waves in (2, 4, 8) and bm % 32 == 0 and bn % 32 == 0
            assert 2 * (bm + bn) * 128 <= 160 * 1024  # two LDS stages fit one CU


def test_planner_headline_shape_is_data_parallel_big_tiles():
    p = T.tcm_plan(8192, 8192, 8192, 8192, 8192, 8192, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)
    assert p["kernel"] == 1 and (p["bm"], p["bn"]) == (256, 256) and p["mode"] == 1
    assert p["tiles"] == 1024 and p["iters_per_tile"] == 128 and p["grid"] == 1024


@pytest.fixture
def tiles_only():
    """The tiled kernel for every call (no split-k GEMV)."""
    T.tcm_set_option("gemv", 1)
    yield
    T.tcm_set_option("gemv", 0)


@pytest.mark.parametrize("M", [1, 16, 64])
def test_planner_skinny_uses_streamk(M, tiles_only):
    p = T.tcm_plan(M, 4096, 4096, 4096, 4096, 4096, T.TCM_F16_F32)
    assert p["kernel"] == 1 and p["mode"] == 2
    assert p["sk_tiles"] > 0 and p["workspace_bytes"] > 0
    # a few K-steps per workgroup: a small tile with a deep Stream-K pipeline
    assert p["config"] in (5, 6) and p["bm"] <= 64 and p["bn"] == 64


@pytest.mark.parametrize("M,N,K,fixup,config", [(1, 4096, 4096, 1, -1), (16, 4096, 4096, 1, -1), (64, 4096, 4096, None, -1),
                                                (256, 4096, 4096, None, -1), (1536, 1536, 16384, 0, 1)])
def test_planner_fixup_kernel_for_many_segments(M, N, K, fixup, config, tiles_only):
    """Split tiles with five or more segments are summed by a second kernel;
    with fewer, by their last arrival.  The option overrides either way.
    (1536^2 x 16384 on 128x128 units: three aligned shares a tile.)"""
    T.tcm_set_option("force_config", config)
    try:
        p = T.tcm_plan(M, N, K, K, N, N, T.TCM_F16_F32)
        per_wg = -(-p["sk_tiles"] * p["iters_per_tile"] // p["grid"])
        assert p["mode"] == 2 and p["split"] == 0 and p["fixup_kernel"] == int(p["iters_per_tile"] >= 5 * per_wg)
        if fixup is not None:
            assert p["fixup_kernel"] == fixup
        for opt, want in ((1, 0), (2, 1)):
            assert T.tcm_set_option("sk_fixup", opt) == T.TCM_OK
            assert T.tcm_plan(M, N, K, K, N, N, T.TCM_F16_F32)["fixup_kernel"] == want
    finally:
        T.tcm_set_option("sk_fixup", 0)
        T.tcm_set_option("force_config", -1)
    # data-parallel plans have nothing to sum
    assert T.tcm_plan(8192, 8192, 8192, 8192, 8192, 8192, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)["fixup_kernel"] == 0


def test_streamk_grid_aligned_to_the_tiles():
    """When the tiles fit the co-resident grid two or more times over, the
    Stream-K grid is an exact multiple of the tile count (every tile's shares
    start at the same k); otherwise it is the co-resident grid."""
    try:
        T.tcm_set_option("force_config", 1)
        p = T.tcm_plan(1536, 1536, 16384, 16384, 1536, 1536, T.TCM_F16_F32)
        assert p["mode"] == 2 and (p["bm"], p["bn"]) == (128, 128) and p["split"] == 0
        assert p["sk_tiles"] == 144 and p["grid"] == 432  # 144 x 3 of 512 slots
        p = T.tcm_plan(2048, 2048, 8192, 8192, 2048, 2048, T.TCM_F16_F32)
        assert p["mode"] == 2 and p["grid"] % p["sk_tiles"] == 0
        T.tcm_set_option("force_config", -1)
        T.tcm_set_option("sk_grid", 500)  # an explicit grid is kept
        p = T.tcm_plan(1536, 1536, 16384, 16384, 1536, 1536, T.TCM_F16_F32)
        assert p["grid"] == 500 and p["split"] == 0
    finally:
        T.tcm_set_option("sk_grid", 0)
        T.tcm_set_option("force_config", -1)


@pytest.fixture
def model_only():
    """Plans from the cost model alone (the shipped tuning table ignored)."""
    T.tcm_set_option("tuned", 0)
    yield
    T.tcm_set_option("tuned", 1)
    for k, v in (("force_config", -1), ("force_mode", 0), ("grid_shares", 0), ("sk_grid", 0), ("grid_per_cu8", 0)):
        T.tcm_set_option(k, v)


def test_equal_shares_of_the_eight_wave_tile(model_only):
    """The eight-wave 256x256 config's Stream-K is equal shares: every tile cut
    into S k ranges (S fills the 256 CUs, at most 8, each share at least one
    K-step), grid T x S, one partial tile a workgroup (no arrival counters),
    always summed by the second kernel."""
    p = T.tcm_plan(1536, 1536, 16384, 16384, 1536, 1536, T.TCM_F16_F32)  # 36 tiles: 7 shares fill 252 CUs
    assert (p["config"], p["mode"], p["sk_tiles"], p["split"], p["grid"]) == (0, 2, 36, 7, 252)
    assert p["dp_tiles"] == 0 and p["fixup_kernel"] == 1
    assert p["workspace_bytes"] == 252 * 256 * 256 * 4
    T.tcm_set_option("force_config", 0)
    T.tcm_set_option("force_mode", 2)
    for M, N, K, dt, want in ((256, 256, 16384, T.TCM_F16_F32, 8),      # one tile: at most 8 shares
                              (256, 256, 192, T.TCM_F16_F32, 3),        # three K-steps: three shares
                              (512, 1024, 4096, T.TCM_I8_I32, 8),       # int8: 128-element K-steps
                              (2048, 2048, 8192, T.TCM_BF16_F32, 4),    # 64 tiles x 4
                              (1024, 8192, 8192, T.TCM_F16_F32, 2)):    # 128 tiles x 2
        p = T.tcm_plan(M, N, K, K, N, N, dt)
        assert p["split"] == want and p["grid"] == p["sk_tiles"] * want, (M, N, K, p)
    T.tcm_set_option("grid_shares", 3)  # the equal-shares option gives S
    p = T.tcm_plan(1536, 1536, 16384, 16384, 1536, 1536, T.TCM_F16_F32)
    assert (p["split"], p["grid"], p["workspace_bytes"]) == (3, 108, 108 * 256 * 256 * 4)
    # more shares than fill the CUs once are capped (64 tiles: at most 4)
    T.tcm_set_option("grid_shares", 5)
    p = T.tcm_plan(2048, 2048, 4096, 4096, 2048, 2048, T.TCM_F16_F32)
    assert (p["config"], p["split"], p["grid"]) == (0, 4, 256)
    T.tcm_set_option("grid_shares", 0)
    # a forced Stream-K without a forced config may take the equal shares
    T.tcm_set_option("force_config", -1)
    p = T.tcm_plan(1536, 1536, 16384, 16384, 1536, 1536, T.TCM_F16_F32)
    assert (p["config"], p["mode"], p["split"]) == (0, 2, 7)
    T.tcm_set_option("force_config", 0)
    # a given grid keeps the persistent Stream-K kernel
    T.tcm_set_option("sk_grid", 200)
    p = T.tcm_plan(1536, 1536, 16384, 16384, 1536, 1536, T.TCM_F16_F32)
    assert p["config"] == 0 and p["mode"] == 2 and p["split"] == 0 and p["grid"] == 200
    T.tcm_set_option("sk_grid", 0)
    # tiles that fill half the CUs or more: no second share, the persistent kernel
    p = T.tcm_plan(3840, 3840, 4096, 4096, 3840, 3840, T.TCM_F16_F32)
    assert p["config"] == 0 and p["mode"] == 2 and p["split"] == 0
    # a batch's tiles form one list: two entries of 36 tiles, 3 shares each
    p = T.tcm_plan_batched(2, 1536, 1536, 16384, 16384, 1536, 1536, T.TCM_F16_F32)
    assert (p["sk_tiles"], p["split"], p["grid"]) == (72, 3, 216)


def test_forced_streamk_skips_the_eight_wave_config():
    """Where the eight-wave config's equal shares cannot serve (225 tiles fill
    more than half the CUs), its Stream-K would be the persistent kernel: a
    forced Stream-K plan uses another config unless that one is forced too."""
    try:
        T.tcm_set_option("force_mode", 2)
        p = T.tcm_plan(3840, 3840, 4096, 4096, 3840, 3840, T.TCM_F16_F32)
        assert p["mode"] == 2 and (p["bm"], p["bn"]) != (256, 256)
        T.tcm_set_option("force_config", 0)
        p = T.tcm_plan(3840, 3840, 4096, 4096, 3840, 3840, T.TCM_F16_F32)
        assert p["mode"] == 2 and p["config"] == 0
    finally:
        T.tcm_set_option("force_mode", 0)
        T.tcm_set_option("force_config", -1)


def test_deep_config_is_the_small_tile_with_more_stages():
    assert T.tcm_config_count() == 7
    for dt in range(4):
        assert T.tcm_config_info(5, dt)[:2] == T.tcm_config_info(4, dt)[:2] == (64, 64)
        # the skinny unit: 32 x 64, two waves
        bm, bn, _, waves = T.tcm_config_info(6, dt)
        assert (bm, bn, waves) == (32, 64, 2)
    # it serves products of few rows only, and as Stream-K (the split-k GEMV
    # left out, which takes such products where it can)
    T.tcm_set_option("gemv", 1)
    try:
        p = T.tcm_plan(16, 4096, 4096, 4096, 4096, 4096, T.TCM_F16_F32)
        assert p["config"] == 6 and p["mode"] == 2
        assert T.tcm_plan(64, 4096, 4096, 4096, 4096, 4096, T.TCM_F16_F32)["config"] != 6
        assert T.tcm_plan(512, 512, 512, 512, 512, 512, T.TCM_F16_F32)["config"] != 6
    finally:
        T.tcm_set_option("gemv", 0)


def test_planner_keeps_split_128_tiles_for_phase_aligned_shapes():
    # 3840^2 x 4096 (900 tiles of 128x128 on 512 slots): a split-k plan would
    # read shared operand panels out of phase, so the 256x256 data-parallel
    # plan stays; and 1536^2 x 16384 (too few tiles for one wave) splits k.
    p = T.tcm_plan(3840, 3840, 4096, 4096, 3840, 3840, T.TCM_F16_F32)
    assert p["mode"] == 1 and (p["bm"], p["bn"]) == (256, 256)
    p = T.tcm_plan(1536, 1536, 16384, 16384, 1536, 1536, T.TCM_F16_F32)
    assert p["mode"] == 2


def test_planner_generic_fallbacks():
    # K not a multiple of the 16-byte chunk, unaligned pointers, column-major A
    assert T.tcm_plan(100, 100, 17, 17, 100, 100, 0)["kernel"] == 0
    assert T.tcm_plan(100, 100, 64, 64, 100, 100, 0, aligned=False)["kernel"] == 0
    assert T.tcm_plan(100, 100, 64, 100, 100, 100, T.TCM_A_COLMAJOR)["kernel"] == 0
    assert T.tcm_plan(100, 100, 64, 64, 100, 100, 0)["kernel"] == 0  # row-major B, N % 8 != 0
    assert T.tcm_plan(100, 104, 64, 64, 104, 104, 0)["kernel"] == 1
    assert T.tcm_plan(100, 100, 64, 64, 64, 100, T.TCM_B_COLMAJOR)["kernel"] == 1
    assert T.tcm_plan(100, 100, 0, 1, 100, 100, 0)["kernel"] == 0  # K == 0


def test_planner_forced_modes():
    try:
        assert T.tcm_set_option("force_mode", 2) == 0
        p = T.tcm_plan(1024, 1024, 1024, 1024, 1024, 1024, 0)
        assert p["mode"] == 2 and p["sk_tiles"] + p["dp_tiles"] == p["tiles"]
        assert T.tcm_set_option("force_mode", 1) == 0
        p = T.tcm_plan(1, 4096, 4096, 4096, 4096, 4096, 0)
        assert p["mode"] == 1 and p["dp_tiles"] == p["tiles"]
        assert T.tcm_set_option("force_config", 1) == 0
        p = T.tcm_plan(1000, 1000, 512, 512, 1000, 1000, 0)
        assert (p["bm"], p["bn"]) == (128, 128)
    finally:
        T.tcm_set_option("force_mode", 0)
        T.tcm_set_option("force_config", -1)


SK_SHAPES = [(9, 16, 256), (36, 256, 256), (225, 64, 256), (144, 256, 512), (1, 7, 300), (5, 3, 2), (300, 1, 1000),
             (17, 13, 64)]


@pytest.mark.parametrize("sk_tiles,iters,grid", SK_SHAPES)
def test_streamk_partition_covers_each_iteration_once(sk_tiles, iters, grid):
    W = sk_tiles * iters
    ranges = [T.tcm_streamk_range(sk_tiles, iters, grid, w) for w in range(grid)]
    assert ranges[0][0] == 0 and ranges[-1][1] == W
    for (b0, e0), (b1, e1) in zip(ranges, ranges[1:]):
        assert e0 == b1  # contiguous, in workgroup order
    sizes = [e - b for b, e in ranges]
    assert max(sizes) - min(sizes) <= 1  # even split
    # each workgroup stores at most two partial tiles (its first and last segment)
    for b, e in ranges:
        if e > b:
            assert (e - 1) // iters - b // iters + 1 >= 1


def _segments(sk_tiles, iters, grid):
    """(wg, tile, k_lo, k_hi) segments in workgroup order, as the kernel walks them."""
    segs = []
    for w in range(grid):
        b, e = T.tcm_streamk_range(sk_tiles, iters, grid, w)
        it = b
        while it < e:
            t = it // iters
            k_lo = it - t * iters
            k_hi = min(iters, k_lo + (e - it))
            segs.append((w, t, k_lo, k_hi))
            it += k_hi - k_lo
    return segs


@pytest.mark.parametrize("sk_tiles,iters,grid", [(4, 8, 3), (2, 5, 7), (3, 16, 16), (6, 4, 5)])
def test_streamk_cpu_simulation_matches_oracle_int8(oracle_lib, sk_tiles, iters, grid):
    """Run the Stream-K decomposition on the CPU: each segment's partial is the
    oracle's exact int8 sum over its k range (bias only in the k = 0 segment),
    partials are summed in workgroup order; the result equals the oracle's
    full product bit-for-bit."""
    import oracle
    rng = np.random.default_rng(7)
    bm, bn, bk = 8, 8, 16
    tiles_n = 2 if sk_tiles % 2 == 0 else 1
    tiles_m = sk_tiles // tiles_n
    M, N, K = tiles_m * bm, tiles_n * bn, iters * bk
    A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    B = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
    bias = rng.integers(-2 ** 20, 2 ** 20, size=N).astype(np.int32)
    full = oracle_lib.gemm(M, N, K, A, K, False, B, N, False, oracle.I8, bias=bias)
    out = np.zeros((M, N), dtype=np.int64)
    seen = {}
    for w, t, k_lo, k_hi in _segments(sk_tiles, iters, grid):
        tm, tn = divmod(t, tiles_n)
        rows, cols = slice(tm * bm, tm * bm + bm), slice(tn * bm, tn * bn + bn)
        a = np.ascontiguousarray(A[rows, k_lo * bk:k_hi * bk])
        b = np.ascontiguousarray(B[k_lo * bk:k_hi * bk, cols])
        part = oracle_lib.gemm(bm, bn, (k_hi - k_lo) * bk, a, a.shape[1], False, b, bn, False, oracle.I8,
                               bias=bias[cols] if k_lo == 0 else None)
        out[rows, cols] += part
        seen.setdefault(t, []).append((w, k_lo, k_hi))
    assert np.array_equal(out.astype(np.int32), full)
    for t, parts in seen.items():  # every tile's segments tile its k range exactly once, in order
        ks = sorted(parts)
        assert ks[0][1] == 0 and ks[-1][2] == iters
        assert all(a[2] == b[1] for a, b in zip(ks, ks[1:]))


@pytest.mark.parametrize("tiles_m,tiles_n", [(32, 32), (15, 15), (1, 16), (16, 1), (6, 6), (2, 32), (33, 7),
                                             (8, 8), (1, 1), (3, 5), (100, 3), (17, 64)])
def test_tile_order_is_a_bijection(tiles_m, tiles_n):
    seen = set()
    for t in range(tiles_m * tiles_n):
        tm, tn = T.tcm_tile_order(t, tiles_m, tiles_n)
        assert 0 <= tm < tiles_m and 0 <= tn < tiles_n
        seen.add((tm, tn))
    assert len(seen) == tiles_m * tiles_n
    with pytest.raises(T.TcmError):
        T.tcm_tile_order(tiles_m * tiles_n, tiles_m, tiles_n)


def test_tile_order_gives_each_xcd_one_block():
    """32 x 32 tiles (8192^2 at 256x256): XCD x = workgroup id mod 8 gets an 8 x 16
    block, and the 32 workgroups it runs first form a 4 x 8 block."""
    for x in range(8):
        tiles = [T.tcm_tile_order(t, 32, 32) for t in range(x, 1024, 8)]
        rows = {tm for tm, _ in tiles}
        cols = {tn for _, tn in tiles}
        assert len(rows) == 8 and len(cols) == 16
        first = tiles[:32]
        assert len({tm for tm, _ in first}) == 4 and len({tn for _, tn in first}) == 8


BAD_BATCHED = [  # (batch, sa, sb, sc, sbias, C address)
    (-1, 16, 16, 16, 0, 4096),     # negative batch
    (2, -1, 16, 16, 0, 4096),      # negative stride
    (2, 16, 16, 15, 0, 4096),      # C entries overlap (stride_c < (M-1)*ldc + N = 16)
    (2, 1 << 40, 16, 16, 0, 4096), # stride beyond the limit
    (3, 2048, 16, 16, 0, 4096 + 2 * 2048 * 2 - 8),  # C overlaps the last entry of A
]


@pytest.mark.parametrize("args", BAD_BATCHED)
def test_invalid_batched_arguments(args):
    batch, sa, sb, sc, sbias, cptr = args
    st = T.tcm_gemm_batched(batch, 4, 4, 4, 4096, 4, sa, 1 << 20, 4, sb, cptr, 4, sc, T.TCM_F16_F32, None, sbias, 0, None)
    assert st == T.TCM_ERR_INVALID_VALUE


def test_batched_empty_and_valid_without_device():
    # batch 0 is a no-op even with NULL pointers; a valid batch reaches the first HIP call
    assert T.tcm_gemm_batched(0, 4, 4, 4, None, 4, 0, None, 4, 0, None, 4, 0, 0, None, 0, 0, None) == T.TCM_OK
    st = T.tcm_gemm_batched(4, 64, 64, 64, 1 << 20, 64, 4096, 2 << 20, 64, 0, 3 << 20, 64, 4096, 0, None, 0, 0, None)
    assert st == T.TCM_ERR_HIP


# class key of the headline: dtype a_col b_col c_type epilogue aligned batched mclass nclass kclass
HEADLINE_KEY = (0, 0, 1, 0, 0, 1, 0, 26, 26, 26)


def _line(key, config, mode, grid_kind=0, grid_param=0, fixup=0, group_m=0, us=12.5, shape=(8192, 8192, 8192)):
    return ("tcm-tune-2 " + " ".join(str(v) for v in key) +
            f" {config} {mode} {grid_kind} {grid_param} {fixup} {group_m} {us:.3f} " + " ".join(map(str, shape)))


def test_half_octave_classes():
    """The class of a size is floor(2 log2 x): one class spans [2^(c/2), 2^((c+1)/2))."""
    T.tcm_tune_clear()
    T.tcm_set_option("tuned", 1)
    try:
        # an entry for the class of 4096 (24) in M, N, K, int8: config 1 Stream-K
        key = (3, 0, 0, 0, 3, 1, 0, 24, 24, 24)
        assert T.tcm_tune_load(_line(key, 1, 2, shape=(4096, 4096, 4096))) == T.TCM_OK
        for k in (4096, 5008, 5792):  # inside the class (K: the tile count stays)
            q = T.tcm_plan(4096, 4096, k, k, 4096, 4096, T.TCM_I8_I32, T.TCM_EPI_BIAS_RELU)
            assert (q["config"], q["mode"]) == (1, 2), k
        for k in (2048, 2896, 8192, 12000):  # two or more half octaves away (22, 22, 26, 27)
            q = T.tcm_plan(4096, 4096, k, k, 4096, 4096, T.TCM_I8_I32, T.TCM_EPI_BIAS_RELU)
            assert (q["config"], q["mode"]) != (1, 2), k
        # another epilogue is another class
        q = T.tcm_plan(4096, 4096, 4096, 4096, 4096, 4096, T.TCM_I8_I32, 0)
        assert (q["config"], q["mode"]) != (1, 2)
        # a class without an entry takes the nearest one within a half octave in every size
        # (K here, so that the tile count stays that of the tuned shape)
        for m, n, k, near in ((4096, 4096, 3008, True), (4096, 4096, 8000, True), (4096, 4096, 12000, False),
                              (4096, 4096, 16384, False)):
            q = T.tcm_plan(m, n, k, k, n, n, T.TCM_I8_I32, T.TCM_EPI_BIAS_RELU)
            assert ((q["config"], q["mode"]) == (1, 2)) == near, (m, n, k)
        # an entry applies only in the wave regime it was tuned in: 4096^2 on 128x128
        # units is 1024 tiles, two waves of the 512 split-k slots; 5800 x 4096
        # (the nearest class) is 1472 tiles, three waves
        q = T.tcm_plan(5800, 4096, 4096, 4096, 4096, 4096, T.TCM_I8_I32, T.TCM_EPI_BIAS_RELU)
        assert (q["config"], q["mode"]) != (1, 2)
    finally:
        T.tcm_tune_clear()


def test_tune_table_round_trip_and_use_by_the_planner():
    T.tcm_tune_clear()
    T.tcm_set_option("tuned", 1)
    model = T.tcm_plan(8192, 8192, 8192, 8192, 8192, 8192, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)
    assert model["config"] == 0
    text = (_line(HEADLINE_KEY, 1, 2, grid_kind=2, grid_param=3, fixup=2, group_m=8) + "\n" +
            _line((3, 0, 0, 0, 3, 1, 0, 12, 12, 12), 4, 1, shape=(64, 64, 64)) + "\n")
    assert T.tcm_tune_load("# a comment\n\n" + text) == T.TCM_OK
    out = T.tcm_tune_table()
    assert sorted(out.strip().splitlines()) == sorted(text.strip().splitlines())
    tuned = T.tcm_plan(8192, 8192, 8192, 8192, 8192, 8192, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)
    # config 1 split-k in equal shares per tile (up to 3, as many as fit the co-resident grid),
    # split tiles summed by the fix-up kernel
    assert (tuned["config"], tuned["mode"]) == (1, 2)
    assert tuned["grid"] % tuned["tiles"] == 0 and tuned["fixup_kernel"] == 1
    # another class (unaligned) is untouched
    assert T.tcm_plan(8192, 8192, 8192, 8192, 8192, 8192, T.TCM_F16_F32 | T.TCM_B_COLMAJOR, aligned=False)["kernel"] == 0
    T.tcm_set_option("tuned", 0)
    try:
        assert T.tcm_plan(8192, 8192, 8192, 8192, 8192, 8192, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)["config"] == 0
    finally:
        T.tcm_set_option("tuned", 1)
    # an explicit switch wins over the table
    T.tcm_set_option("force_config", 2)
    try:
        assert T.tcm_plan(8192, 8192, 8192, 8192, 8192, 8192, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)["config"] == 2
    finally:
        T.tcm_set_option("force_config", -1)
    # a switch the caller set keeps its value (here: the fix-up)
    T.tcm_set_option("sk_fixup", 1)
    try:
        assert T.tcm_plan(8192, 8192, 8192, 8192, 8192, 8192, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)["fixup_kernel"] == 0
    finally:
        T.tcm_set_option("sk_fixup", 0)
    T.tcm_tune_clear()
    assert T.tcm_tune_table() == ""
    assert T.tcm_plan(8192, 8192, 8192, 8192, 8192, 8192, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)["config"] == 0


GOOD_TAIL = " 1 1 0 0 0 0 1.0 8 8 8"


@pytest.mark.parametrize("bad", [
    "tcm-tune-1 0 0 1 0 0 1 0 26 26 26" + GOOD_TAIL,           # unknown version tag
    "tcm-tune-2 0 0 1 0 0 1 0 26 26 26 99 1 0 0 0 0 1.0 8 8 8",  # no such config
    "tcm-tune-2 0 0 1 0 0 1 0 26 26 26 1 3 0 0 0 0 1.0 8 8 8",   # no such mode
    "tcm-tune-2 0 0 1 0 0 1 0 26 26 26 1 2 3 1 0 0 1.0 8 8 8",   # no such grid kind
    "tcm-tune-2 0 0 1 0 0 1 0 26 26 26 1 2 1 0 0 0 1.0 8 8 8",   # a grid kind without its parameter
    "tcm-tune-2 0 0 1 0 0 1 0 26 26 26 1 2 0 0 3 0 1.0 8 8 8",   # no such fix-up
    "tcm-tune-2 0 0 1 0 0 1 0 26 26 26 1 2 0 0 0 17 1.0 8 8 8",  # group rows beyond 16
    "tcm-tune-2 7 0 1 0 0 1 0 26 26 26" + GOOD_TAIL,           # no such element type
    "tcm-tune-2 0 2 1 0 0 1 0 26 26 26" + GOOD_TAIL,           # a flag that is not 0 / 1
    "tcm-tune-2 0 0 1 0 0 1 0 26 26 26 1 1 0 0 0 0 1.0 8 8",   # missing field
    "tcm-tune-2 0 0 1 0 0 1 0 26 26 26" + GOOD_TAIL + " extra",  # trailing text
    "tcm-tune-2 0 0 1 0 0 1 0 26 26 26 1 1 0 0 0 0 1.0 0 8 8",   # an empty tuned shape
])
def test_tune_load_rejects_malformed_text_all_or_nothing(bad):
    T.tcm_tune_clear()
    good = _line(HEADLINE_KEY, 1, 1)
    assert T.tcm_tune_load(good + "\n" + bad + "\n") == T.TCM_ERR_INVALID_VALUE
    assert T.tcm_tune_table() == ""  # the good line was not applied either
    assert T.tcm_tune_load("") == T.TCM_OK  # empty text: nothing to do


def test_tune_invalid_arguments_without_device():
    assert T.tcm_tune(64, 64, 64, 1 << 20, 64, 2 << 20, 64, 3 << 20, 64, 0, None, 0, 0, None)[0] == T.TCM_ERR_INVALID_VALUE
    assert T.tcm_tune(64, 64, 64, 1 << 20, 3, 2 << 20, 64, 3 << 20, 64, 0, None, 0, 5, None)[0] == T.TCM_ERR_INVALID_VALUE
    assert T.tcm_tune(64, 64, 64, 1 << 20, 64, 2 << 20, 64, 3 << 20, 64, 0, None, 0, 5, None)[0] == T.TCM_ERR_HIP


# convolution: (N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, dtype, epilogue, x, f, y, bias)
CONV_OK = (2, 8, 8, 64, 32, 3, 3, 1, 1, 1, 1, 1, 1, T.TCM_F16_F32, 0, 1 << 20, 2 << 20, 3 << 20, 0)
_CONV_FIELDS = "N H W C K R S pad_h pad_w stride_h stride_w dil_h dil_w dtype epilogue x f y bias".split()


def _conv(**kw):
    a = dict(zip(_CONV_FIELDS, CONV_OK), **kw)
    return T.tcm_conv2d(*(a[k] for k in _CONV_FIELDS[:13]), a["x"] or None, a["f"] or None, a["y"] or None, a["dtype"],
                        a["bias"] or None, a["epilogue"], None)


def test_planner_column_major_a():
    """Column-major A (m contiguous) runs on the tiles of at least 64 rows when
    M and lda are whole numbers of 16-byte pieces (the split-k GEMV and the
    32-row configs take row-major A only); otherwise the generic kernel."""
    code = T.TCM_F16_F32 | T.TCM_A_COLMAJOR
    p = T.tcm_plan(4096, 4096, 4096, 4096, 4096, 4096, code | T.TCM_B_COLMAJOR)
    assert p["kernel"] == 1 and (p["bm"], p["bn"]) == (256, 256)
    p = T.tcm_plan(16, 4096, 4096, 16, 4096, 4096, code)
    assert p["kernel"] == 1 and p["bm"] >= 64
    assert T.tcm_plan(1000, 1000, 512, 1000, 1000, 1000, code)["kernel"] == 1
    assert T.tcm_plan(1004, 1000, 512, 1004, 1000, 1000, code)["kernel"] == 0  # M % 8 != 0
    assert T.tcm_plan(1000, 1000, 512, 1004, 1000, 1000, code)["kernel"] == 0  # lda % 8 != 0
    assert T.tcm_plan(1024, 1024, 1024, 1024, 1024, 1024, T.TCM_I8_I32 | T.TCM_A_COLMAJOR)["kernel"] == 1
    assert T.tcm_plan(1000, 1024, 1024, 1000, 1024, 1024, T.TCM_I8_I32 | T.TCM_A_COLMAJOR)["kernel"] == 0  # 1000 % 16
    for cfg in (2, 6):  # 32-row tiles: not for column-major A
        T.tcm_set_option("force_config", cfg)
        try:
            q = T.tcm_plan(64, 4096, 4096, 64, 4096, 4096, code)
        finally:
            T.tcm_set_option("force_config", -1)
        assert q["kernel"] != 1 or q["config"] != cfg


BAD_CONV = [
    dict(N=-1), dict(H=-1), dict(C=-1), dict(K=-1), dict(R=0), dict(S=0),  # negative / empty filter
    dict(pad_h=-1), dict(stride_w=0), dict(dil_h=0),
    dict(H=2, R=5),                              # dilated filter larger than the padded input
    dict(W=1, pad_w=0, S=2),
    dict(H=3, R=2, dil_h=3, pad_h=0),           # dilation pushes the filter past the input
    dict(H=1 << 31),                             # beyond the dimension limit
    dict(dtype=T.TCM_F16_F32 | T.TCM_A_COLMAJOR),  # layouts are fixed
    dict(dtype=T.TCM_F16_F32 | T.TCM_B_COLMAJOR),
    dict(dtype=T.TCM_I8_I32 | T.TCM_C_F16),      # 16-bit output for int8
    dict(dtype=7),                               # unknown element type
    dict(epilogue=T.TCM_EPI_ACCUM),              # accumulate is not offered
    dict(epilogue=T.TCM_EPI_BIAS),               # bias flag without bias
    dict(x=0), dict(f=0), dict(y=0),             # NULL operands
    dict(y=(1 << 20) + 64),                      # y overlaps x
    dict(y=(2 << 20) - 64),                      # y overlaps f (f starts inside y)
    dict(epilogue=T.TCM_EPI_BIAS, bias=(3 << 20) + 256),  # bias inside y
]


@pytest.mark.parametrize("kw", BAD_CONV, ids=[",".join(f"{k}={v}" for k, v in d.items()) for d in BAD_CONV])
def test_invalid_conv_arguments_rejected(kw):
    assert _conv(**kw) == T.TCM_ERR_INVALID_VALUE


def test_conv_empty_and_valid_without_device():
    # no output pixel or no output channel: nothing to do, NULL pointers allowed
    assert _conv(N=0, x=0, f=0, y=0) == T.TCM_OK
    assert _conv(K=0, x=0, f=0, y=0) == T.TCM_OK
    # valid requests reach the first HIP call: fast-path shapes, a channel count
    # the tiled gather does not take, strides and dilations, 16-bit outputs
    for kw in (dict(), dict(C=3), dict(stride_h=2, stride_w=3, dil_h=2, dil_w=2), dict(dtype=T.TCM_BF16_F32 | T.TCM_C_BF16),
               dict(epilogue=T.TCM_EPI_BIAS | T.TCM_EPI_RELU, bias=4 << 20), dict(dtype=T.TCM_I8_I32), dict(C=0),
               dict(x=(1 << 20) + 1), dict(y=(3 << 20) + 2)):  # element-misaligned pointers are served too
        assert _conv(**kw) == T.TCM_ERR_HIP, kw


def _gentry(M=64, N=64, A=1 << 20, lda=64, B=2 << 20, ldb=64, C=3 << 20, ldc=64, bias=0):
    return T.GroupEntry(M, N, A or None, lda, B or None, ldb, C or None, ldc, bias or None)


def test_grouped_invalid_arguments():
    ok = [_gentry(), _gentry(A=4 << 20, B=5 << 20, C=6 << 20)]
    assert T.tcm_gemm_grouped([_gentry()] * 33, 64, 0, 0, None) == T.TCM_ERR_INVALID_VALUE  # beyond the limit
    assert T.lib().tcm_gemm_grouped(-1, None, 64, 0, 0, None) == T.TCM_ERR_INVALID_VALUE
    assert T.lib().tcm_gemm_grouped(2, None, 64, 0, 0, None) == T.TCM_ERR_INVALID_VALUE
    bad = [
        [_gentry(lda=32)],                                   # lda < K
        [_gentry(N=-1)],                                     # negative size
        [_gentry(C=0)],                                      # NULL C
        [_gentry(), _gentry(A=4 << 20, B=5 << 20, C=(3 << 20) + 64)],  # two C overlap
        [_gentry(), _gentry(A=(3 << 20) + 128, B=5 << 20, C=6 << 20)],  # C of entry 0 overlaps A of entry 1
    ]
    for ents in bad:
        assert T.tcm_gemm_grouped(ents, 64, 0, 0, None) == T.TCM_ERR_INVALID_VALUE, ents
    assert T.tcm_gemm_grouped(ok, 64, 0, T.TCM_EPI_BIAS, None) == T.TCM_ERR_INVALID_VALUE  # bias flag, no bias
    assert T.tcm_gemm_grouped(ok, -1, 0, 0, None) == T.TCM_ERR_INVALID_VALUE


def test_grouped_empty_and_valid_without_device():
    assert T.tcm_gemm_grouped([], 64, 0, 0, None) == T.TCM_OK
    # entries without rows or columns are skipped, NULL pointers and all
    assert T.tcm_gemm_grouped([_gentry(M=0, A=0, B=0, C=0), _gentry(N=0, A=0, B=0, C=0)], 64, 0, 0, None) == T.TCM_OK
    ok = [_gentry(), _gentry(M=17, A=4 << 20, B=5 << 20, C=6 << 20), _gentry(M=0, A=0, B=0, C=0)]
    assert T.tcm_gemm_grouped(ok, 64, 0, 0, None) == T.TCM_ERR_HIP
    assert T.tcm_gemm_grouped([_gentry(C=(3 << 20) + 2)], 64, 0, 0, None) == T.TCM_ERR_HIP  # any alignment


def test_plan_batched_counts_every_entry():
    """tcm_plan_batched plans one work list over all entries; batch 1 is tcm_plan."""
    one = T.tcm_plan(16, 4096, 4096, 4096, 4096, 4096, T.TCM_F16_F32)
    assert T.tcm_plan_batched(1, 16, 4096, 4096, 4096, 4096, 4096, T.TCM_F16_F32) == one
    b8 = T.tcm_plan_batched(8, 16, 4096, 4096, 4096, 4096, 4096, T.TCM_F16_F32)
    assert b8["kernel"] == 1
    assert b8["tiles"] == 8 * ((16 + b8["bm"] - 1) // b8["bm"]) * ((4096 + b8["bn"] - 1) // b8["bn"])
    assert b8["dp_tiles"] + b8["sk_tiles"] == b8["tiles"]
    for bad in (0, -1, 1 << 31):
        with pytest.raises(T.TcmError):
            T.tcm_plan_batched(bad, 16, 4096, 4096, 4096, 4096, 4096, T.TCM_F16_F32)


def test_data_parallel_entries_carry_over_to_fewer_waves_only():
    """A data-parallel class entry applies to problems of as many waves or
    fewer on its tile config, not to ones that need more."""
    T.tcm_tune_clear()
    T.tcm_set_option("tuned", 1)
    try:
        # f16, B row-major: 2048^3 on 64x64 tiles (config 4) with group rows 8, one wave of 1024 slots
        assert T.tcm_tune_load(_line((0, 0, 0, 0, 0, 1, 0, 22, 22, 22), 4, 1, group_m=8, shape=(2048, 2048, 2048))) == 0
        q = T.tcm_plan(2048, 2048, 2048, 2048, 2048, 2048, T.TCM_F16_F32)
        assert (q["config"], q["mode"]) == (4, 1)
        q = T.tcm_plan(1600, 1600, 2048, 2048, 1600, 1600, T.TCM_F16_F32)  # nearest class, under one wave
        assert (q["config"], q["mode"]) == (4, 1)
        q = T.tcm_plan(2816, 2816, 2816, 2816, 2816, 2816, T.TCM_F16_F32)  # same class, two waves
        assert q["config"] != 4 or q["mode"] != 1
    finally:
        T.tcm_tune_clear()


# ------------------------------------------------------------ split-k GEMV

@pytest.mark.parametrize("tuned", [0, 1])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
def test_planner_gemv_for_few_rows(M, tuned):
    """Row-major f16 products of at most 32 rows run on a split-k GEMV, with
    or without the shipped table (whose entries for those classes name one):
    the 16x16x32 kernel (128 columns, ranges of a multiple of 128 rows, one
    workgroup per CU without the table) or, as a table entry may say, the
    4x4x4 one (256 columns a workgroup, k ranges of a multiple of 64 rows);
    k ranges cover K, their partial sums (ranges x M x N floats) added by a
    second kernel."""
    T.tcm_set_option("tuned", tuned)
    try:
        p = T.tcm_plan(M, 4096, 4096, 4096, 4096, 4096, T.TCM_F16_F32)
    finally:
        T.tcm_set_option("tuned", 1)
    assert p["kernel"] == 2 and p["config"] == -1
    if p["bn"] == 256:
        assert p["bk"] % 64 == 0 and p["bm"] == {1: 1, 2: 2, 3: 4, 4: 4, 5: 8, 8: 8}[M]
    else:
        assert p["bn"] == 128 and p["bk"] % 128 == 0 and p["bm"] == (16 if M <= 16 else 32)
    assert p["bk"] * p["iters_per_tile"] >= 4096 and p["grid"] == 4096 // p["bn"] * p["iters_per_tile"]
    assert p["workspace_bytes"] == p["iters_per_tile"] * M * 4096 * 4 and p["fixup_kernel"] == 1
    if not tuned:
        assert p["bn"] == 128 and p["iters_per_tile"] == 8 and p["bk"] == 512


def test_planner_gemv_not_taken_when_ineligible():
    """More than 32 rows, row-major B with N not a multiple of 4,
    column-major B with K not a multiple of 8, a padded A row off 16 bytes,
    int8 or f32, a forced tile config or mode: tiles."""
    code = T.TCM_F16_F32
    assert T.tcm_plan(8, 4096, 4096, 4096, 4096, 4096, code)["kernel"] == 2
    assert T.tcm_plan(33, 4096, 4096, 4096, 4096, 4096, code)["kernel"] == 1
    assert T.tcm_plan(8, 4096, 4100, 4104, 4104, 4096, code | T.TCM_B_COLMAJOR)["kernel"] != 2
    assert T.tcm_plan(8, 4094, 4096, 4096, 4094, 4094, code)["kernel"] != 2
    assert T.tcm_plan(8, 4096, 4096, 4100, 4096, 4096, code)["kernel"] != 2
    assert T.tcm_plan(8, 4096, 4096, 4096, 4096, 4096, T.TCM_F32_F32)["kernel"] != 2
    assert T.tcm_plan(8, 4096, 4096, 4096, 4096, 4096, T.TCM_I8_I32)["kernel"] != 2
    assert T.tcm_plan(8, 4096, 4096, 4096, 4096, 4096, code, aligned=False)["kernel"] != 2
    for key, val in (("force_config", 4), ("force_mode", 2), ("gemv", 1)):
        T.tcm_set_option(key, val)
        try:
            assert T.tcm_plan(8, 4096, 4096, 4096, 4096, 4096, code)["kernel"] == 1
        finally:
            T.tcm_set_option(key, -1 if key == "force_config" else 0)


def test_planner_gemv_rows_limits():
    """Without the table the planner takes the GEMV up to 32 rows (row-major
    B, 16-byte rows of B); option gemv = 2 takes it for any eligible call (64
    rows on the 16x16x32 kernel; 16 with gemv_wide = 1, which leaves only the
    4x4x4 kernel); column-major B stops at 8 rows, or 16 forced."""
    code = T.TCM_F16_F32
    T.tcm_set_option("tuned", 0)
    try:
        assert T.tcm_plan(32, 4096, 4096, 4096, 4096, 4096, code)["kernel"] == 2
        assert T.tcm_plan(33, 4096, 4096, 4096, 4096, 4096, code)["kernel"] == 1
        assert T.tcm_plan(9, 4096, 4096, 4096, 4096, 4096, code | T.TCM_B_COLMAJOR)["kernel"] == 1
        T.tcm_set_option("gemv", 2)
        p = T.tcm_plan(64, 4096, 4096, 4096, 4096, 4096, code)
        assert p["kernel"] == 2 and p["bm"] == 64 and p["bn"] == 128
        assert T.tcm_plan(65, 4096, 4096, 4096, 4096, 4096, code)["kernel"] == 1
        assert T.tcm_plan(16, 4096, 4096, 4096, 4096, 4096, code | T.TCM_B_COLMAJOR)["kernel"] == 2
        assert T.tcm_plan(17, 4096, 4096, 4096, 4096, 4096, code | T.TCM_B_COLMAJOR)["kernel"] == 1
        T.tcm_set_option("gemv_wide", 1)
        p = T.tcm_plan(16, 4096, 4096, 4096, 4096, 4096, code)
        assert p["kernel"] == 2 and p["bn"] == 256
        assert T.tcm_plan(17, 4096, 4096, 4096, 4096, 4096, code)["kernel"] == 1
        T.tcm_set_option("gemv_wide", 2)
        p = T.tcm_plan(1, 4096, 4096, 4096, 4096, 4096, code)
        assert p["kernel"] == 2 and p["bn"] == 128 and p["bm"] == 16
    finally:
        T.tcm_set_option("gemv", 0)
        T.tcm_set_option("gemv_wide", 0)
        T.tcm_set_option("tuned", 1)


@pytest.mark.parametrize("K,splits", [(8, 0), (1000, 0), (4096, 0), (4096, 3), (70000, 0), (70000, 7)])
@pytest.mark.parametrize("M", [12, 24, 64])
def test_planner_gemv_wide_k_ranges(M, K, splits):
    """16x16x32 row-major kernel: one workgroup per CU (N = 1024: 8 column
    blocks, 32 ranges), ranges of a multiple of 512 rows (16-row bucket) or
    256 (32 and 64) where K allows, an asked-for count rounded to ranges of a
    multiple of 128 rows; together they cover K."""
    T.tcm_set_option("gemv", 2)
    T.tcm_set_option("gemv_splits", splits)
    try:
        p = T.tcm_plan(M, 1024, K, -(-K // 8) * 8, 1024, 1024, T.TCM_F16_F32)
    finally:
        T.tcm_set_option("gemv", 0)
        T.tcm_set_option("gemv_splits", 0)
    kw, ranges = p["bk"], p["iters_per_tile"]
    assert p["kernel"] == 2 and p["bn"] == 128 and p["tiles"] == 8 and p["grid"] == 8 * ranges
    assert kw * ranges >= K and kw * (ranges - 1) < K
    if splits:
        assert kw == -(-(-(-K // splits)) // 128) * 128
    else:
        align = 512 if M <= 16 else 256
        assert kw == -(-(-(-K // 32)) // align) * align
    assert p["fixup_kernel"] == (ranges > 1)
    assert p["workspace_bytes"] == (ranges * M * 1024 * 4 if ranges > 1 else 0)


@pytest.mark.parametrize("K,splits", [(64, 1), (100, 1), (4096, 5), (70000, 0)])
def test_planner_gemv_k_ranges(K, splits):
    """The 4x4x4 kernel's k ranges: multiples of 64 rows, at most 1024 each,
    together covering K; an asked-for count is rounded to that grid."""
    T.tcm_set_option("gemv_splits", splits)
    T.tcm_set_option("gemv_wide", 1)
    try:
        p = T.tcm_plan(2, 1024, K, -(-K // 8) * 8, 1024, 1024, T.TCM_BF16_F32)
    finally:
        T.tcm_set_option("gemv_splits", 0)
        T.tcm_set_option("gemv_wide", 0)
    kw, ranges = p["bk"], p["iters_per_tile"]
    assert p["kernel"] == 2 and kw % 64 == 0 and kw <= 1024
    assert kw * ranges >= K and kw * (ranges - 1) < K
    if splits:
        assert kw == min(1024, -(-(-(-K // splits)) // 64) * 64)
    assert p["fixup_kernel"] == (ranges > 1)
    assert p["workspace_bytes"] == (ranges * 2 * 1024 * 4 if ranges > 1 else 0)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_planner_gemv_column_major_b(M):
    """Column-major B (k contiguous): 128 columns a workgroup, k ranges of
    256 rows, 16 rows computed whatever M is; K must be a multiple of 8."""
    T.tcm_set_option("tuned", 0)
    try:
        p = T.tcm_plan(M, 4096, 4096, 4096, 4096, 4096, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)
        q = T.tcm_plan(M, 4096, 4100, 4104, 4104, 4096, T.TCM_F16_F32 | T.TCM_B_COLMAJOR)
    finally:
        T.tcm_set_option("tuned", 1)
    assert p["kernel"] == 2 and p["bn"] == 128 and p["bk"] == 256 and p["bm"] == 16
    assert p["iters_per_tile"] == 16 and p["grid"] == 32 * 16
    assert p["workspace_bytes"] == 16 * M * 4096 * 4
    assert q["kernel"] != 2  # K = 4100 is not a multiple of 8
