"""Host-side logic of bench.py: the one-GPU guard, plan parsing, and the
checks that keep stale HBM-traffic counters out of the roofline."""
import json
import os
import subprocess
import sys

import bench
import synthetic as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DP_PLAN = ("kernel=tile config=0 tile=256x256x64 mode=dp grid=1024 tiles=1024 iters=128 dp_tiles=1024 sk_tiles=0 "
           "M=8192 N=8192 K=8192 dtype=0 b_col=1 est_cycles=1")
SK_PLAN = ("kernel=tile config=4 tile=64x64x64 mode=streamk grid=768 tiles=576 iters=256 dp_tiles=0 sk_tiles=576 "
           "M=1536 N=1536 K=16384 dtype=0 b_col=0 est_cycles=1")
HYBRID_PLAN = ("kernel=tile config=1 tile=128x128x64 mode=streamk grid=256 tiles=900 iters=64 dp_tiles=512 "
               "sk_tiles=388 M=3840 N=3840 K=4096 dtype=0 b_col=0 est_cycles=1")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_plan_kernels_names_the_launched_kernels():
    assert bench.plan_kernels(DP_PLAN) == {"void tcm::tile_gemm_kernel<0, 0, true, false>(tcm::TileArgs)"}
    assert bench.plan_kernels(SK_PLAN) == {"void tcm::tile_gemm_kernel<0, 4, false, true>(tcm::TileArgs)"}
    assert bench.plan_kernels(HYBRID_PLAN) == {"void tcm::tile_gemm_kernel<0, 1, false, false>(tcm::TileArgs)",
                                               "void tcm::tile_gemm_kernel<0, 1, false, true>(tcm::TileArgs)"}
    assert bench.plan_kernels("kernel=generic tile=64x64 tiles=4 iters=2 M=1 N=1 K=1 dtype=0") == set()
    conv = HYBRID_PLAN.replace("kernel=tile", "kernel=conv").replace("b_col=0", "b_col=1")
    assert bench.plan_kernels(conv) == {"void tcm::tile_conv_kernel<0, 1, false>(tcm::TileArgs)",
                                        "void tcm::tile_conv_kernel<0, 1, true>(tcm::TileArgs)"}
    acol = HYBRID_PLAN + " fixup=kernel a_col=1"
    assert bench.plan_kernels(acol) == {"void tcm::tile_gemm_acol_kernel<0, 1, false, false>(tcm::TileArgs)",
                                        "void tcm::tile_gemm_acol_kernel<0, 1, false, true>(tcm::TileArgs)",
                                        "void tcm::tile_fixup_kernel<0, 1, false>(tcm::TileArgs)"}
    split = SK_PLAN.replace("config=4", "config=0").replace("grid=768", "grid=252") + " fixup=kernel split=7"
    assert bench.plan_kernels(split) == {"void tcm::tile_split_kernel<0, 0, false, false>(tcm::TileArgs)",
                                         "void tcm::tile_split_fixup_kernel<0, 0>(tcm::TileArgs)"}
    assert bench.plan_kernels(split + " a_col=1") == {"void tcm::tile_split_kernel<0, 0, false, true>(tcm::TileArgs)",
                                                      "void tcm::tile_split_fixup_kernel<0, 0>(tcm::TileArgs)"}
    group = HYBRID_PLAN + " group=8"
    assert bench.plan_kernels(group) == {"void tcm::tile_group_kernel<0, 1, false, false>(tcm::GroupArgs)",
                                         "void tcm::tile_group_kernel<0, 1, false, true>(tcm::GroupArgs)"}
    gemv = "kernel=gemv rows=8 cols_per_wg=256 k_per_wg=128 splits=32 grid=512 M=5 N=4096 K=4096 dtype=1 fixup=kernel"
    assert bench.plan_kernels(gemv) == {"void tcm::gemv::gemv_split_kernel<1, 8>(tcm::GemvArgs)",
                                        "tcm::gemv::gemv_reduce_kernel(tcm::GemvArgs)"}
    assert bench.plan_kernels(gemv.replace(" fixup=kernel", "").replace("splits=32", "splits=1")) == \
        {"void tcm::gemv::gemv_split_kernel<1, 8>(tcm::GemvArgs)"}


def test_gemv_counters_are_keyed_to_the_gemv_sources():
    """The split-k GEMV's stored counters follow its own sources, the tiled
    workloads' counters the tiled kernels' sources."""
    assert bench.kernel_source_hash(bench.GEMV_SOURCES) != bench.kernel_source_hash()
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic_skinny_m1.json")))
    if "gemv" in (t.get("dominant_kernel") or ""):
        if "gemv_r_kernel" in t["dominant_kernel"]:  # the 16x16x32 kernel's plan
            plan = ("kernel=gemv rows=16 cols_per_wg=128 k_per_wg=512 splits=8 grid=256 M=1 N=4096 K=4096 dtype=0 "
                    "b_col=0 mfma=16x16x32 fixup=kernel")
        else:
            plan = ("kernel=gemv rows=1 cols_per_wg=256 k_per_wg=128 splits=32 grid=512 M=1 N=4096 K=4096 dtype=0 "
                    "b_col=0 mfma=4x4x4 fixup=kernel")
        got = bench.load_traffic(S.workload("skinny_m1"), plan)
        if t["source_hash"] == bench.kernel_source_hash(bench.GEMV_SOURCES):
            assert got == t["hbm_bytes_per_launch"]
        else:  # counters taken on other GEMV code are not reported
            assert got is None


def _with_traffic(tmp_path, monkeypatch, record):
    d = tmp_path / "profiles"
    d.mkdir()
    (d / "traffic_f16_8192.json").write_text(json.dumps(record))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(d / "traffic_{name}.json"))


def test_traffic_used_only_for_the_profiled_kernel_and_sources(tmp_path, monkeypatch):
    p = S.workload("f16_8192")
    good = {"source_hash": bench.kernel_source_hash(),
            "dominant_kernel": "void tcm::tile_gemm_kernel<0, 0, true, false>(tcm::TileArgs)",
            "hbm_bytes_per_launch": 1.5e9}
    _with_traffic(tmp_path, monkeypatch, good)
    assert bench.load_traffic(p, DP_PLAN) == 1.5e9
    # the plan now launches another kernel: the counters do not describe it
    assert bench.load_traffic(p, SK_PLAN) is None


def test_traffic_dropped_when_kernel_sources_change(tmp_path, monkeypatch):
    p = S.workload("f16_8192")
    stale = {"source_hash": "0000000000000000",
             "dominant_kernel": "void tcm::tile_gemm_kernel<0, 0, true, false>(tcm::TileArgs)",
             "hbm_bytes_per_launch": 1.5e9}
    _with_traffic(tmp_path, monkeypatch, stale)
    assert bench.load_traffic(p, DP_PLAN) is None


def test_kernel_hash_covers_the_tiled_kernel_sources():
    """Every source of the tiled GEMM and convolution kernels (the kernels the
    stored counters describe) is in the hash: their instantiations, the
    template and the shared argument / tile-table header."""
    csrc = os.path.join(ROOT, "tensor_core_mixed_amd", "csrc")
    tiled = {f for f in os.listdir(csrc) if f.startswith(("tile_", "conv_", "group_"))} | {"tcm_internal.h"}
    assert tiled == set(bench.KERNEL_SOURCES)


def test_kernel_hash_ignores_comments_but_not_code():
    src = "int f(int x) {  // twice\n    /* a\n       block */\n    return 2 * x;\n}\n"
    assert bench._code_only(src) == bench._code_only(src.replace("twice", "double it").replace("a\n", "b\n"))
    assert bench._code_only(src) != bench._code_only(src.replace("2 * x", "3 * x"))


def test_roofline_bound_follows_the_intensity():
    big = S.workload("f16_8192")
    r = bench.roofline(big.dtype, big.flops, big.alg_bytes, 0.9, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and 0 < r["frac"] < 1
    skinny = S.workload("skinny_m16")
    r = bench.roofline(skinny.dtype, skinny.flops, skinny.alg_bytes, 0.015, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert abs(r["achieved"] - skinny.alg_bytes / 15e-6 / 1e9) < 1
