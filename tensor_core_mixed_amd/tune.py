"""Offline tuning of the tile table: writes the tuning table the library ships.

    python -m tensor_core_mixed_amd.tune                 # tune the shape set, write tuned/mi355x.txt
    python -m tensor_core_mixed_amd.tune --heldout R.md  # check held-out shapes against the table
    python -m tensor_core_mixed_amd.tune --only gemv     # re-tune the shapes the split-k GEMV can serve
    python -m tensor_core_mixed_amd.tune --only split    # re-tune the shapes equal shares of the 256x256 tile can serve

Tuning: for every shape of TUNE_SHAPES, tcm_tune searches the tile configs in
both modes (and the split-k GEMV where it can serve the shape), then the
group rows, Stream-K grid and fix-up around the three fastest tile plans, and records the winner for the shape's class (element type,
layouts, output type, epilogue, alignment, and the half octaves of M, N, K;
see include/tcm.h).  The table text is written to tuned/mi355x.txt beside
this package's build directory, where libtcm.so finds it.

Held-out check: for each shape of HELDOUT_SHAPES (none of them tuned), the
call's own plan (the shipped table where it covers the class, else the cost
model) is timed against the best point tcm_tune finds for that shape; the
report lists both and their ratio.

Operands are random device tensors: N(0,1) for floating point (the matrix
cores' clock depends on the data, and the benchmarked workloads use normal
and uniform values), uniform int8 with an int32 bias for int8 products.
"""
import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "tuned", "mi355x.txt")

F16, BF16, F32, I8 = 0, 1, 2, 3
NAMES = {F16: "f16", BF16: "bf16", F32: "f32", I8: "i8"}

# (dtype, M, N, K, B column-major, epilogue flags, C type flag)
# the benchmarked workloads and shapes the cost model once misplanned
WORKLOAD_SHAPES = [
    (F16, 8192, 8192, 8192, True, 0, 0),
    (BF16, 8192, 8192, 8192, True, 0, 0),
    (F16, 8192, 8192, 8192, False, 0, 0),
    (F16, 8192, 8192, 8192, True, 0, "f16"),
    (F16, 512, 512, 512, False, 0, 0),
    (F32, 2048, 2048, 2048, False, 0, 0),
    (F16, 1, 4096, 4096, False, 0, 0),
    (F16, 16, 4096, 4096, False, 0, 0),
    (F16, 64, 4096, 4096, False, 0, 0),
    (F16, 256, 4096, 4096, False, 0, 0),
    (F16, 1536, 1536, 16384, False, 0, 0),
    (F16, 3840, 3840, 4096, False, 0, 0),
    (I8, 4096, 4096, 4096, False, 3, 0),
    (BF16, 4096, 4096, 4096, True, 7, "bf16"),
    (F16, 1024, 1024, 1024, False, 0, 0),
    (F16, 2048, 2048, 8192, False, 0, 0),
    (F16, 2560, 4096, 4096, False, 0, 0),
    (F16, 2048, 2048, 2048, False, 0, 0),
    (F16, 4096, 4096, 4096, True, 0, 0),
    (F16, 4096, 4096, 4096, False, 0, 0),
]



def _grid(dt, b_col, epi=0, c_type=0, big=8192):
    """A grid over the shape families: square, long K, short K, skinny
    (few rows), and rectangles."""
    out = []
    for s in (512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192):
        if s <= big:
            out.append((dt, s, s, s, b_col, epi, c_type))
    for s in (768, 1536, 3072):
        out.append((dt, s, s, 4 * s, b_col, epi, c_type))
    for s in (2048, 4096, 8192):
        if s <= big:
            out.append((dt, s, s, s // 4, b_col, epi, c_type))
    for m in (1, 8, 32, 128, 256, 512):
        for nk in (4096, 8192):
            if nk <= big:
                out.append((dt, m, nk, nk, b_col, epi, c_type))
    for m, n, k in ((1024, 4096, 1024), (4096, 1024, 4096), (512, 8192, 2048), (2048, 6144, 2048)):
        out.append((dt, m, n, k, b_col, epi, c_type))
    return out


GRID_SHAPES = (_grid(F16, False) + _grid(F16, True) + _grid(BF16, True) + _grid(I8, False, epi=3, big=4096) +
               [x for x in _grid(F32, False, big=4096) if x[1] >= 256])


# shapes of other classes (or other sizes within one), never tuned
HELDOUT_SHAPES = [
    (F16, 768, 768, 768, False, 0, 0),
    (F16, 1280, 1280, 5120, False, 0, 0),
    (F16, 3072, 3072, 3072, True, 0, 0),
    (BF16, 6144, 6144, 2048, True, 0, 0),
    (F16, 32, 8192, 8192, False, 0, 0),
    (F16, 128, 4096, 4096, False, 0, 0),
    (F16, 512, 11008, 4096, False, 0, 0),
    (I8, 2048, 2048, 2048, False, 3, 0),
    (F32, 1024, 1024, 1024, False, 0, 0),
    (BF16, 8192, 1024, 8192, True, 0, 0),
    (F16, 2000, 2000, 2000, False, 0, 0),
    (F16, 4096, 4096, 1024, False, 0, 0),
]


# a second held-out set, drawn after the first had shaped two planner rules
# (the nearest-class fallback and the fix-up threshold)
HELDOUT2_SHAPES = [
    (F16, 640, 640, 2560, False, 0, 0),
    (F16, 1536, 1536, 1536, False, 0, 0),
    (F16, 2304, 2304, 9216, False, 0, 0),
    (BF16, 4096, 4096, 2048, True, 0, 0),
    (F16, 8, 4096, 11008, False, 0, 0),
    (F16, 192, 5120, 5120, False, 0, 0),
    (F16, 1024, 3072, 1024, False, 0, 0),
    (I8, 3072, 3072, 3072, False, 3, 0),
    (F32, 3072, 1024, 512, False, 0, 0),
    (BF16, 2048, 8192, 2048, True, 0, 0),
    (F16, 1000, 1504, 3000, False, 0, 0),
    (F16, 6144, 6144, 6144, True, 0, 0),
]


# a third held-out set, drawn after set 2 had shaped the wave-regime rule
HELDOUT3_SHAPES = [
    (F16, 896, 1792, 3584, False, 0, 0),
    (F16, 2816, 2816, 2816, False, 0, 0),
    (F16, 3584, 3584, 8192, True, 0, 0),
    (BF16, 5120, 5120, 5120, True, 0, 0),
    (F16, 4, 8192, 4096, False, 0, 0),
    (F16, 96, 3072, 3072, False, 0, 0),
    (F16, 1536, 6144, 1536, False, 0, 0),
    (I8, 5120, 5120, 2048, False, 3, 0),
    (F32, 1536, 1536, 1536, False, 0, 0),
    (BF16, 7168, 2048, 4096, True, 0, 0),
    (F16, 1200, 1200, 1200, False, 0, 0),
    (F16, 2048, 2048, 4096, False, 0, 0),
]


# every tuned shape, once; held-out shapes are never among them
TUNE_SHAPES = list(dict.fromkeys(WORKLOAD_SHAPES + GRID_SHAPES))
TUNE_SHAPES = [x for x in TUNE_SHAPES if x not in set(HELDOUT_SHAPES + HELDOUT2_SHAPES + HELDOUT3_SHAPES)]


def _tensors(dt, M, N, K, b_col, epi, c_type):
    import torch
    torch.manual_seed(M * 31 + N * 7 + K)
    tdt = {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}
    if dt == I8:
        A = torch.randint(-128, 128, (M, K), dtype=torch.int8, device="cuda")
        B = torch.randint(-128, 128, (N, K) if b_col else (K, N), dtype=torch.int8, device="cuda")
        bias = torch.randint(-2 ** 20, 2 ** 20, (N,), dtype=torch.int32, device="cuda")
        C = torch.zeros((M, N), dtype=torch.int32, device="cuda")
    else:
        A = torch.randn(M, K, device="cuda").to(tdt[dt])
        B = torch.randn(*((N, K) if b_col else (K, N)), device="cuda").to(tdt[dt])
        bias = torch.randn(N, device="cuda")
        cdt = {0: torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[c_type]
        C = torch.zeros((M, N), dtype=cdt, device="cuda")
    return A, B, C, bias


def _args(T, dt, M, N, K, b_col, epi, c_type, A, B, C, bias):
    code = dt | (T.TCM_B_COLMAJOR if b_col else 0) | {0: 0, "f16": T.TCM_C_F16, "bf16": T.TCM_C_BF16}[c_type]
    return (M, N, K, A.data_ptr(), K, B.data_ptr(), K if b_col else N, C.data_ptr(), N, code,
            bias.data_ptr() if epi & 1 else None, epi)


def _label(shape):
    dt, M, N, K, b_col, epi, c_type = shape
    out = f"{NAMES[dt]} {M}x{N}x{K} B {'col' if b_col else 'row'}-major"
    if epi:
        out += " epi=" + "+".join(n for b, n in ((1, "bias"), (2, "relu"), (4, "C_in")) if epi & b)
    if c_type:
        out += f" C {c_type}"
    return out


def gemv_shape(shape):
    """Shapes a split-k GEMV kernel can serve (f16 / bf16; at most 16 rows,
    or at most 64 with row-major B and rows of A and B 16-byte aligned)."""
    dt, M, N, K, b_col, epi, c_type = shape
    if dt not in (F16, BF16) or K % 8:
        return False
    return (M <= 16 and (b_col or N % 4 == 0)) or (not b_col and M <= 64 and N % 8 == 0)


def split_shape(shape):
    """Shapes the eight-wave config's equal shares may serve: 256x256 tiles
    that fill at most half the 256 CUs (two or more shares a tile), at least
    16 K-steps to share out, and at least 128 rows and columns (a product of
    fewer rows wastes most of a 256-row tile's matrix-core work)."""
    dt, M, N, K, b_col, epi, c_type = shape
    tiles = -(-M // 256) * -(-N // 256)
    steps = -(-K // {F16: 64, BF16: 64, F32: 32, I8: 128}[dt])
    return tiles <= 128 and steps >= 16 and M >= 128 and N >= 128


def tune(shapes, iters, out, merge=None):
    import torch
    import tensor_core_mixed_amd as T
    T.tcm_plan(64, 64, 64, 64, 64, 64, F16)  # the first plan loads the shipped table ...
    if merge is None:
        T.tcm_tune_clear()                    # ... which is dropped: tune from the cost model
    s = torch.cuda.current_stream().cuda_stream
    for shape in shapes:
        A, B, C, bias = _tensors(*shape)
        t0 = time.time()
        st, best = T.tcm_tune(*_args(T, *shape, A, B, C, bias), iters, s)
        assert st == T.TCM_OK, T.tcm_status_string(st)
        print(f"[tune] {_label(shape)}: config {best['config']} mode {best['mode']} grid {best['grid']} "
              f"({time.time() - t0:.1f} s)", flush=True)
        del A, B, C, bias
    text = T.tcm_tune_table()
    os.makedirs(os.path.dirname(out), exist_ok=True)
    props = torch.cuda.get_device_properties(0)
    with open(out, "w") as f:
        what = (f"{len(TUNE_SHAPES)} shapes ({len(shapes)} re-tuned with `--only {merge}`)" if merge else
                f"{len(shapes)} shapes")
        f.write(f"# tuning table of libtcm for {props.name} ({props.multi_processor_count} CUs), "
                f"written by tensor_core_mixed_amd/tune.py from {what}, {iters} timed calls per candidate\n")
        f.write("# tcm-tune-2 dtype a_col b_col c_type epilogue aligned batched mclass nclass kclass "
                "config mode grid_kind grid_param fixup group_m us M N K\n")
        f.write(text)
    print(f"[tune] wrote {out} ({len(text.splitlines())} classes)", flush=True)


def _block_us(call, reps, stream):
    import torch
    for _ in range(3):
        call()
    t0 = time.time()
    while time.time() - t0 < 0.1:
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def heldout(sets, iters, report):
    """sets: [(title, shapes)]; one table per set in the report."""
    import torch
    import tensor_core_mixed_amd as T
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    results = []
    for title, shapes in sets:
        results.append((title, _heldout_rows(T, shapes, iters, stream, s)))
    _write_report(report, results, iters)


def _heldout_rows(T, shapes, iters, stream, s):
    rows = []
    for shape in shapes:
        A, B, C, bias = _tensors(*shape)
        args = _args(T, *shape, A, B, C, bias)
        call = lambda: T.tcm_gemm(*args, s)
        assert call() == T.TCM_OK
        plan = T.tcm_last_plan()
        saved = T.tcm_tune_table()
        st, best = T.tcm_tune(*args, iters, s)
        assert st == T.TCM_OK, T.tcm_status_string(st)
        line = [l for l in T.tcm_tune_table().splitlines() if l not in saved.splitlines()]
        T.tcm_tune_clear()
        T.tcm_tune_load(saved)
        # the call's own plan and the search's best point, re-timed the same
        # way and alternately (blocks of back-to-back calls, median of five
        # each): the search's own minimum over many candidates reads low
        auto_t, best_t = [], []
        best_desc = "(generic kernel)"
        if line:
            f = line[0].split()
            best_desc = f"config {f[11]} mode {f[12]} grid {f[13]}/{f[14]} fixup {f[15]} group {f[16]}"
        for _ in range(5):
            auto_t.append(_block_us(call, iters, stream))
            if line:
                T.tcm_tune_load(line[0])
                best_t.append(_block_us(call, iters, stream))
                T.tcm_tune_clear()
                T.tcm_tune_load(saved)
        auto = sorted(auto_t)[2]
        best_us = sorted(best_t)[2] if best_t else auto
        ratio = auto / best_us
        rows.append((_label(shape), plan, auto, best_desc, best_us, ratio))
        print(f"[heldout] {_label(shape)}: auto {auto:.1f} us, best {best_us:.1f} us ({best_desc}), ratio {ratio:.3f}",
              flush=True)
        del A, B, C, bias
    return rows


def _write_report(report, results, iters):
    import torch
    with open(report, "w") as f:
        props = torch.cuda.get_device_properties(0)
        f.write("# Held-out shapes: the planner's plan against the best tuned point\n\n")
        f.write(f"Device: {props.name}, {props.multi_processor_count} CUs.  Command: "
                f"`python -m tensor_core_mixed_amd.tune --heldout {os.path.relpath(report)} --iters {iters}`.\n\n")
        f.write("For each shape (none of them in the tuning set), `auto` is the call's own plan (the shipped table "
                "`tensor_core_mixed_amd/tuned/mi355x.txt` where it holds the shape's class, else the cost model); "
                "`best` is the fastest point `tcm_tune` finds "
                "for the shape (two stages: every tile config in both modes and, where they can serve the shape, the split-k GEMV "
                "kernels (configs 100 and 101); then group rows, Stream-K grid and fix-up around the three fastest tile plans).  Both are then re-timed alternately, five blocks of back-to-back calls each, "
                "and the medians compared: `ratio` = auto / best (the search's own minimum over many candidates reads "
                "low, so it is not used).\n\n")
        for title, rows in results:
            f.write(f"## {title}\n\n")
            f.write("| shape | auto plan | auto us | best point | best us | ratio |\n|---|---|---|---|---|---|\n")
            for lab, plan, auto, bdesc, bus, ratio in rows:
                short = " ".join(kv for kv in plan.split() if kv.split("=")[0] in ("kernel", "config", "tile", "mode", "grid",
                                                                                   "fixup", "tuned"))
                f.write(f"| {lab} | `{short}` | {auto:.1f} | {bdesc} | {bus:.1f} | {ratio:.3f} |\n")
            within = sum(1 for r in rows if r[5] <= 1.05)
            f.write(f"\n{within} of {len(rows)} shapes run within 5% of their best tuned point.\n\n")
    print(f"[heldout] wrote {report}", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=TABLE)
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--heldout", default=None, help="write the held-out report here instead of tuning")
    ap.add_argument("--only", choices=["gemv", "split"], default=None,
                    help="re-tune only the shapes the split-k GEMV (gemv) or the equal shares of the 256x256 tile "
                         "(split) can serve, keeping the shipped entries of the others")
    a = ap.parse_args()
    sys.path.insert(0, os.path.dirname(HERE))
    import torch
    torch.cuda.set_device(0)
    if a.heldout:
        heldout([("Held-out set 1", HELDOUT_SHAPES),
                 ("Held-out set 2 (drawn after set 1 shaped the nearest-class fallback and the fix-up threshold)",
                  HELDOUT2_SHAPES),
                 ("Held-out set 3 (drawn after set 2 shaped the wave-regime rule)", HELDOUT3_SHAPES)],
                a.iters, a.heldout)
    elif a.only:
        pick = gemv_shape if a.only == "gemv" else split_shape
        tune([x for x in TUNE_SHAPES if pick(x)], a.iters, a.out, merge=a.only)
    else:
        tune(TUNE_SHAPES, a.iters, a.out)


if __name__ == "__main__":
    main()
