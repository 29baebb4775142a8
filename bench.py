#!/usr/bin/env python3
"""Benchmark of the GEMM engine on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one tcm_gemm call of the whole hot path on the workload (default:
f16 8192^3, A row-major, B column-major, f32 accumulate and output -- the
shape the headline TFLOP/s figure is quoted on), inputs resident in HBM.
A convolution workload (conv_*) times one tcm_conv2d call instead.
Prints one JSON line with the throughput, the roofline of the dominant
kernel (achieved algorithmic FLOP/s from HIP events on the launch stream vs
the dtype's dense MFMA peak) and the CPU oracle's rate on a bounded sample.

Extra modes (for profiling runs):
  --calibrate-copy            one 512 MiB device-to-device copy (counter calibration)
  --summarize-counters DIR    turn rocprofv3 --pmc output into profiles/ JSON
  --all                       also time every workload and write a table (stderr)
"""
import argparse
import hashlib
import json
import os
import sys
import time
import types

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "GEMM TFLOPS/TOPS on 1 MI355X and % of dtype MFMA peak (fp16 8192³)"
# dense MFMA peaks of MI355X (256 CUs at 2.4 GHz), TFLOP/s (TOP/s for int8)
PEAK = {0: 2516.6, 1: 2516.6, 2: 157.3, 3: 5033.2}
HBM_PEAK_GBS = 8000.0
DTYPE_NAME = {0: "f16", 1: "bf16", 2: "f32", 3: "i8"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{name}.json")


# the sources of the tiled GEMM, grouped and convolution kernels, whose launches the stored counters describe
KERNEL_SOURCES = ("tcm_internal.h", "tile_kernel.h", "tile_instances.h", "tile_f16.hip", "tile_bf16.hip",
                  "tile_f32.hip", "tile_i8.hip", "tile_acol_f16.hip", "tile_acol_bf16.hip", "tile_acol_f32.hip",
                  "tile_acol_i8.hip", "conv_f16.hip", "conv_bf16.hip", "conv_f32.hip", "conv_i8.hip",
                  "group_f16.hip", "group_bf16.hip", "group_f32.hip", "group_i8.hip")


def _code_only(text):
    """C++ source without comments, trailing spaces and blank lines."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


# the sources of the split-k GEMV (products of a few rows)
GEMV_SOURCES = ("gemv.h", "gemv_kernel.hip")


def kernel_source_hash(sources=KERNEL_SOURCES):
    """Hash of a kernel family's code (comments and layout excluded): counters
    taken on other code are stale."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "tensor_core_mixed_amd", "csrc")
    for f in sources:
        with open(os.path.join(d, f)) as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def plan_kernels(plan):
    """Kernel names a tcm_last_plan() string launches (tiled GEMM / convolution and GEMV kernels)."""
    f = dict(kv.split("=", 1) for kv in plan.split() if "=" in kv)
    if f.get("kernel") == "gemv":
        if f.get("b_col") == "1":
            names = {f"void tcm::gemv::gemv_t_kernel<{f['dtype']}>(tcm::GemvArgs)"}
        elif f.get("mfma") == "16x16x32":
            names = {f"void tcm::gemv::gemv_r_kernel<{f['dtype']}, {f['rows']}>(tcm::GemvArgs)"}
        else:
            names = {f"void tcm::gemv::gemv_split_kernel<{f['dtype']}, {f['rows']}>(tcm::GemvArgs)"}
        if f.get("fixup") == "kernel":
            names.add("tcm::gemv::gemv_reduce_kernel(tcm::GemvArgs)")
        return names
    if f.get("kernel") not in ("tile", "conv"):
        return set()
    b = "true" if f.get("b_col") == "1" else "false"
    if int(f.get("split", 0)) > 1:  # equal shares of every tile, then the wave-per-block sum
        a = "true" if f.get("a_col") == "1" else "false"
        return {f"void tcm::tile_split_kernel<{f['dtype']}, {f['config']}, {b}, {a}>(tcm::TileArgs)",
                f"void tcm::tile_split_fixup_kernel<{f['dtype']}, {f['config']}>(tcm::TileArgs)"}
    if f["kernel"] == "conv":
        head = f"void tcm::tile_conv_kernel<{f['dtype']}, {f['config']}, "
    elif "group" in f:
        head = f"void tcm::tile_group_kernel<{f['dtype']}, {f['config']}, {b}, "
    elif f.get("a_col") == "1":  # A column-major
        head = f"void tcm::tile_gemm_acol_kernel<{f['dtype']}, {f['config']}, {b}, "
    else:
        head = f"void tcm::tile_gemm_kernel<{f['dtype']}, {f['config']}, {b}, "
    args = "(tcm::GroupArgs)" if "group" in f else "(tcm::TileArgs)"
    names = set()
    if int(f.get("dp_tiles", 0)) > 0:
        names.add(head + "false>" + args)
    if int(f.get("sk_tiles", 0)) > 0:
        names.add(head + "true>" + args)
        if f.get("fixup") == "kernel":  # split tiles summed by a second kernel
            kind = "conv" if f["kernel"] == "conv" else ("group" if "group" in f else "tile")
            tail = f"{f['dtype']}, {f['config']}>" if kind == "conv" else f"{f['dtype']}, {f['config']}, {b}>"
            names.add(f"void tcm::{kind}_fixup_kernel<{tail}{args}")
    return names


def describe(p):
    acc = "int32" if p.dtype == 3 else "f32"
    out = acc if p.c_type == "acc" else p.c_type
    return (f"{DTYPE_NAME[p.dtype]} GEMM {p.M}x{p.N}x{p.K}, A {'col' if p.a_col else 'row'}-major, "
            f"B {'col' if p.b_col else 'row'}-major, {acc} accumulate, {out} output"
            + (", C's contents as the initial value" if p.accum else "")
            + (", bias + ReLU epilogue" if p.bias else ""))


def roofline(dtype, flops, alg_bytes, ms, traffic):
    """The bound of a launch from its algorithmic intensity: below the ridge
    (MFMA peak / HBM peak) HBM bandwidth, above it the dtype's MFMA peak."""
    ridge = PEAK[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / alg_bytes < ridge:
        gbs = alg_bytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    value = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK[dtype],
            "unit": "TFLOP/s" if dtype != 3 else "TOP/s", "frac": round(value / PEAK[dtype], 4), "traffic": traffic}


def describe_conv(p):
    acc = "int32" if p.dtype == 3 else "f32"
    out = acc if p.c_type == "acc" else p.c_type
    return (f"{DTYPE_NAME[p.dtype]} Conv2d NHWC {p.N}x{p.H}x{p.W}x{p.C} * KRSC {p.K}x{p.R}x{p.S}x{p.C}, "
            f"pad {p.pad}, stride {p.stride}, dilation {p.dil} -> NPQK {p.N}x{p.P}x{p.Q}x{p.K} "
            f"(implicit GEMM {p.N * p.P * p.Q}x{p.K}x{p.R * p.S * p.C}), {acc} accumulate, {out} output"
            + (", bias + ReLU epilogue" if p.bias else ""))


class ConvJob:
    """A convolution workload resident on the device, one tcm_conv2d call per step."""

    def __init__(self, p, stream):
        import torch

        import synthetic as S
        import tensor_core_mixed_amd as T
        self.p, self.g = p, S.generate_conv(p)
        dev = lambda x: None if x is None else torch.from_numpy(
            np.ascontiguousarray(x.view(np.int16) if x.dtype == np.uint16 else x)).cuda()
        self.x, self.f, self.bias = dev(self.g["x"]), dev(self.g["f"]), dev(self.g["bias"])
        c_t = {"f16": torch.float16, "bf16": torch.bfloat16}.get(p.c_type, torch.int32 if p.dtype == 3 else torch.float32)
        self.y = torch.empty((p.N * p.P * p.Q, p.K), dtype=c_t, device="cuda")
        code = p.dtype | {"acc": 0, "f16": T.TCM_C_F16, "bf16": T.TCM_C_BF16}[p.c_type]
        epi = (T.TCM_EPI_BIAS if p.bias else 0) | (T.TCM_EPI_RELU if p.relu else 0)
        self.args = (p.N, p.H, p.W, p.C, p.K, p.R, p.S, p.pad[0], p.pad[1], p.stride[0], p.stride[1], p.dil[0],
                     p.dil[1], self.x.data_ptr(), self.f.data_ptr(), self.y.data_ptr(), code,
                     self.bias.data_ptr() if self.bias is not None else None, epi, stream)

    def call(self):
        import tensor_core_mixed_amd as T
        st = T.tcm_conv2d(*self.args)
        if st != 0:
            raise RuntimeError(T.tcm_status_string(st))

    def _oracle(self, mm, kk):
        import oracle
        p, g = self.p, self.g
        return oracle.get().conv2d_entries(g["x"], g["f"], p.dtype, mm, kk, pad=p.pad, stride=p.stride, dil=p.dil,
                                           bias=g["bias"], relu=p.relu)

    def sampled_check(self):
        """(CPU leg) The seeded sampled outputs of y against the oracle's values."""
        import torch

        import synthetic as S
        p, g = self.p, self.g
        mm, kk = S.sample_conv_entries(p)
        yc = self.y.float() if self.y.dtype in (torch.float16, torch.bfloat16) else self.y
        got = yc.cpu().numpy()[mm, kk]
        ref = self._oracle(mm, kk)
        if p.dtype == 3:
            return {"entries": int(got.size), "mismatches": int(np.sum(got != ref)), "ok": bool(np.all(got == ref))}
        denom = p.R * p.S * p.C * float(np.max(np.abs(_decode(g["x"], p.dtype)))) * \
            float(np.max(np.abs(_decode(g["f"], p.dtype))))
        denom += float(np.max(np.abs(g["bias"]))) if g["bias"] is not None else 0.0
        u = {"acc": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[p.c_type]
        err = max(float(np.max(np.abs(got.astype(np.float64) - ref) - u * np.abs(ref))), 0.0) / (denom or 1.0)
        tol = 1e-5 if p.dtype == 2 else 1e-3
        return {"entries": int(got.size), "normalised_error": err, "tolerance": tol, "ok": err <= tol}

    def _oracle_seconds(self, n):
        rng = np.random.default_rng(7)
        M = self.p.N * self.p.P * self.p.Q
        mm, kk = rng.integers(0, M, n), rng.integers(0, self.p.K, n)
        t = time.perf_counter()
        self._oracle(mm, kk)
        return time.perf_counter() - t

    def cpu_baseline(self, unit_scale, outputs=1 << 18, per_core_outputs=1 << 12):
        """The oracle's sampled-output entry point on `outputs` seeded random
        outputs with every OpenMP thread, then `per_core_outputs` with one."""
        import oracle
        o = oracle.get()
        p = self.p
        per_out = 2.0 * p.R * p.S * p.C
        threads = o.max_threads()
        dt = self._oracle_seconds(outputs)
        out = {"value": outputs * per_out / dt / unit_scale, "unit": "TFLOP/s" if p.dtype != 3 else "TOP/s",
               "cores": threads, "kind": "oracle", "seconds": round(dt, 2),
               "sample": f"{outputs} seeded random outputs of y (each a {p.R * p.S * p.C}-term sum; "
                         f"{outputs / (p.N * p.P * p.Q * p.K):.4f} of the convolution), binary64 accumulation"}
        o.set_threads(1)
        try:
            d1 = self._oracle_seconds(per_core_outputs)
        finally:
            o.set_threads(threads)
        out["per_core"] = {"value": per_core_outputs * per_out / d1 / unit_scale, "outputs": per_core_outputs,
                           "seconds": round(d1, 2)}
        return out


class GroupJob:
    """A group workload resident on the device: one tcm_gemm_grouped call per
    step, or (call_each) one tcm_gemm call per entry."""

    def __init__(self, ps, stream):
        import tensor_core_mixed_amd as T
        import synthetic as S
        self.ps, self.gs = ps, [S.generate(p) for p in ps]
        self.dev = [upload(g, p) for p, g in zip(ps, self.gs)]
        self.Cs = [make_c(p) for p in ps]
        self.ents = [(p.M, p.N, A.data_ptr(), p.LDA, B.data_ptr(), p.LDB, C.data_ptr(), p.LDC, None)
                     for p, (A, B, _), C in zip(ps, self.dev, self.Cs)]
        self.code = ps[0].dtype | (T.TCM_B_COLMAJOR if ps[0].b_col else 0)
        self.stream = stream
        self.singles = [make_call(p, A, B, bias, C, stream) for p, (A, B, bias), C in zip(ps, self.dev, self.Cs)]

    def call(self):
        import tensor_core_mixed_amd as T
        st = T.tcm_gemm_grouped(self.ents, self.ps[0].K, self.code, 0, self.stream)
        if st != 0:
            raise RuntimeError(T.tcm_status_string(st))

    def call_each(self):
        for c in self.singles:
            c()

    @property
    def flops(self):
        return sum(p.flops for p in self.ps)

    @property
    def alg_bytes(self):
        return sum(p.alg_bytes for p in self.ps)

    def sampled_check(self):
        """(CPU leg) Every non-empty entry's sampled entries against the oracle."""
        worst, n, ok = 0.0, 0, True
        for p, g, C in zip(self.ps, self.gs, self.Cs):
            if p.M == 0:
                continue
            r = _oracle_sampled_check(p, g, C)
            n += r["entries"]
            ok = ok and r["ok"]
            worst = max(worst, r.get("normalised_error", 0.0))
        return {"entries": n, "normalised_error": worst, "ok": ok}


def make_c(p):
    """C on the device in its storage type (M x ldc)."""
    import torch
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}.get(p.c_type, torch.int32 if p.dtype == 3 else torch.float32)
    lead = (p.batch,) if p.batch > 1 else ()
    return torch.empty(lead + (max(p.M, 1), p.LDC), dtype=dt, device="cuda")


def reset_c(p, g, C):
    """With accumulation, put the initial-value tensor back into C (no-op otherwise)."""
    import torch
    if p.accum:
        cin = g["C_in"]
        src = (torch.from_numpy(cin.view(np.int16).copy()).view(C.dtype) if cin.dtype == np.uint16
               else torch.from_numpy(cin.copy()))
        C.copy_(src.reshape(C.shape))


def upload(g, p):
    import torch
    def dev(x):
        if x is None:
            return None
        if x.dtype == np.uint16:
            x = x.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return dev(g["A"]), dev(g["B"]), dev(g["bias"])


def make_call(p, A, B, bias, C, stream):
    import tensor_core_mixed_amd as T
    code = p.dtype | (T.TCM_A_COLMAJOR if p.a_col else 0) | (T.TCM_B_COLMAJOR if p.b_col else 0)
    code |= {"acc": 0, "f16": T.TCM_C_F16, "bf16": T.TCM_C_BF16}[p.c_type]
    epi = (T.TCM_EPI_BIAS if p.bias else 0) | (T.TCM_EPI_RELU if p.relu else 0) | (T.TCM_EPI_ACCUM if p.accum else 0)
    bptr = bias.data_ptr() if bias is not None else None
    if p.batch > 1:  # entries packed back to back (B shared with stride 0 if so drawn)
        sa, sb, sc = A[0].numel(), 0 if p.b_shared else B[0].numel(), C[0].numel()
        args = (p.batch, p.M, p.N, p.K, A.data_ptr(), p.LDA, sa, B.data_ptr(), p.LDB, sb, C.data_ptr(), p.LDC, sc, code,
                bptr, p.N if bias is not None else 0, epi, stream)
        fn = T.tcm_gemm_batched
    else:
        args = (p.M, p.N, p.K, A.data_ptr(), p.LDA, B.data_ptr(), p.LDB, C.data_ptr(), p.LDC, code, bptr, epi, stream)
        fn = T.tcm_gemm

    def call():
        st = fn(*args)
        if st != 0:
            raise RuntimeError(T.tcm_status_string(st))
    return call


def time_steps(call, steps, warmup, stream_obj, min_warm_ms=0.0):
    """`warmup` untimed calls (continued until `min_warm_ms` of wall time has
    passed, if given), then `steps` calls between two events on the stream."""
    import torch
    t_warm = time.perf_counter()
    done = 0
    while done < warmup or (time.perf_counter() - t_warm) * 1e3 < min_warm_ms:
        call()
        done += 1
        if done % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream_obj)
    for _ in range(steps):
        call()
    e1.record(stream_obj)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def per_call_us(call, calls, stream_obj):
    """Each call bracketed by its own event pair (after the timed block): median and min in us."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for e0, e1 in ev:
        e0.record(stream_obj)
        call()
        e1.record(stream_obj)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    return {"median": round(t[len(t) // 2], 2), "min": round(t[0], 2), "calls": calls}


def cold_us(call, calls, stream_obj):
    """Median time of calls each preceded by a 512 MiB read (outside the event pair) that
    evicts the 256 MB MALL and the L2s: the HBM-bound shapes with nothing cached.  The
    buffer is written once before the loop; a write before every call would leave the MALL
    full of dirty lines, and the timed call would pay for their write-back (M = 1 at
    N = K = 4096: 19.4 us after a write, 13.3 us after a read)."""
    import torch
    scratch = torch.empty(512 * 2 ** 20 // 4, dtype=torch.float32, device="cuda")
    scratch.fill_(1.0)
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    t = []
    for i in range(calls):
        torch.sum(scratch, dim=0, out=sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream_obj)
        call()
        e1.record(stream_obj)
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    return round(sorted(t)[len(t) // 2], 2)


def _oracle_sampled_check(p, g, C):
    """(CPU leg) The sampled entries (4096 seeded + rows 0 and M-1) of C after one
    call from the initial state, against the oracle's values."""
    import torch

    import oracle
    import synthetic as S
    Cc = C.float() if C.dtype in (torch.float16, torch.bfloat16) else C
    Cc = Cc.cpu().numpy().reshape(max(p.batch, 1), -1, p.LDC)
    # a batch: the first and the last entry, each checked like a single product
    entries = [0] if p.batch == 1 else [0, p.batch - 1]
    got, ref = [], []
    for e in entries:
        pe, ge = (p, g) if p.batch == 1 else (p.entry(e), S.entry_inputs(p, g, e))
        ii, jj = S.sample_entries(pe)
        got.append(Cc[e][ii, jj])
        cin = {}
        if p.accum:
            cin = {"c_in": ge["C_in"].reshape(-1), "c_in_type": S.C_TYPE_CODE.get(p.c_type, S.F32), "ldcin": p.LDC}
        ref.append(oracle.get().gemm_entries(p.M, p.N, p.K, ge["A"], p.LDA, p.a_col, ge["B"], p.LDB, p.b_col, p.dtype,
                                             ii, jj, bias=ge["bias"], relu=p.relu, **cin))
    got, ref = np.concatenate(got), np.concatenate(ref)
    n_checked = int(got.size)
    if p.dtype == 3:
        return {"entries": n_checked, "mismatches": int(np.sum(got != ref)), "ok": bool(np.all(got == ref))}

    def amax(x, dt):
        return float(np.max(np.abs(_decode(x, dt))))
    denom = p.K * amax(g["A"], p.dtype) * amax(g["B"], p.dtype)
    denom += float(np.max(np.abs(g["bias"]))) if g["bias"] is not None else 0.0
    denom += amax(g["C_in"], S.C_TYPE_CODE.get(p.c_type, S.F32)) if p.accum else 0.0
    u = {"acc": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}[p.c_type]  # half an ulp of a 16-bit C
    excess = np.abs(got.astype(np.float64) - ref) - u * np.abs(ref)
    err = max(float(np.max(excess)), 0.0) / (denom if denom > 0 else 1.0)
    tol = 1e-5 if p.dtype == 2 else 1e-3
    return {"entries": n_checked, "normalised_error": err, "tolerance": tol, "ok": err <= tol}


def _decode(x, dt):
    if dt == 0:
        return x.view(np.float16).astype(np.float64)
    if dt == 1:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _oracle_rows(o, p, g, rows):
    if p.batch > 1:  # one entry of a batch stands for all of them
        import synthetic as S
        p, g = p.entry(0), S.entry_inputs(p, g, 0)
    A = g["A"]
    a_rows = A[:rows] if not p.a_col else A
    t = time.perf_counter()
    o.gemm(rows, p.N, p.K, a_rows, p.LDA, p.a_col, g["B"], p.LDB, p.b_col, p.dtype, bias=g["bias"], relu=p.relu)
    return time.perf_counter() - t


def cpu_baseline(p, g, unit_scale, rows=4096, per_core_rows=64):
    """The oracle (full-product entry point) on the first `rows` rows of C with
    every OpenMP thread, then on `per_core_rows` rows with one thread."""
    import oracle
    o = oracle.get()
    rows = min(rows, p.M)
    threads = o.max_threads()
    dt = _oracle_rows(o, p, g, rows)
    flops = 2.0 * rows * p.N * p.K
    out = {"value": flops / dt / unit_scale, "unit": "TFLOP/s" if p.dtype != 3 else "TOP/s", "cores": threads,
           "kind": "oracle", "seconds": round(dt, 2),
           "sample": f"rows 0..{rows - 1} of C ({rows}x{p.N} entries, K={p.K}; {rows / p.M:.4f} of the product), "
                     f"binary64 accumulation"}
    if per_core_rows:
        r1 = min(per_core_rows, p.M)
        o.set_threads(1)
        try:
            d1 = _oracle_rows(o, p, g, r1)
        finally:
            o.set_threads(threads)
        out["per_core"] = {"value": 2.0 * r1 * p.N * p.K / d1 / unit_scale, "rows": r1, "seconds": round(d1, 2)}
    return out


def load_traffic(p, plan):
    """Calibrated HBM bytes per launch of the dominant kernel from profiles/, or
    None when the kernel sources changed since the counters were taken or the
    plan no longer launches that kernel."""
    path = TRAFFIC_FILE.format(name=p.name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    family = GEMV_SOURCES if "kernel=gemv" in plan else KERNEL_SOURCES
    if t.get("source_hash") != kernel_source_hash(family) or t.get("dominant_kernel") not in plan_kernels(plan):
        return None
    return t.get("hbm_bytes_per_launch")


def run_bench_conv(args):
    import torch

    import synthetic as S
    import tensor_core_mixed_amd as T
    p = S.CONV_WORKLOADS[args.workload]
    if args.dist:
        from dataclasses import replace
        p = replace(p, dist=args.dist)
    torch.cuda.set_device(0)
    print(f"[bench] workload {p.name}: {describe_conv(p)}", file=sys.stderr, flush=True)
    stream_obj = torch.cuda.current_stream()
    job = ConvJob(p, stream_obj.cuda_stream)
    job.call()
    torch.cuda.synchronize()
    plan = T.tcm_last_plan()
    print(f"[bench] plan: {plan}", file=sys.stderr, flush=True)
    ms, wall_ms = time_steps(job.call, args.steps, args.warmup, stream_obj)
    calls = per_call_us(job.call, args.steps, stream_obj)
    value = p.flops / (ms * 1e-3) / 1e12
    print(f"[bench] {ms:.4f} ms/step, {value:.1f} T(FL)OP/s", file=sys.stderr, flush=True)
    roof = roofline(p.dtype, p.flops, p.alg_bytes, ms, load_traffic(p, plan))
    cpu, parity = None, None
    if not args.no_cpu:
        job.call()
        torch.cuda.synchronize()
        parity = job.sampled_check()
        print(f"[bench] sampled check {parity}", file=sys.stderr, flush=True)
        cpu = job.cpu_baseline(1e12)
    g = p.gemm()
    line = {
        "metric": "Conv2d + bias + ReLU (implicit GEMM) TFLOPS/TOPS on 1 MI355X and % of dtype MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s" if p.dtype != 3 else "TOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAME[p.dtype],
        "data": "synthetic",
        "config": {"workload": describe_conv(p), "gemm_M": g.M, "gemm_N": g.N, "gemm_K": g.K, "seed": p.seed,
                   "dist": p.dist, "plan": plan, "wall_ms_per_step": round(wall_ms, 5), "per_call_us": calls,
                   "hbm_frac": round(p.alg_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4), "parity": parity},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def run_bench_group(args):
    import torch

    import synthetic as S
    import tensor_core_mixed_amd as T
    ps = S.GROUP_WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    desc = (f"group of {len(ps)} f16 GEMMs sharing K={ps[0].K}, N={ps[0].N}, M = {[p.M for p in ps]}, "
            f"B row-major, f32 accumulate and output")
    print(f"[bench] workload {args.workload}: {desc}", file=sys.stderr, flush=True)
    stream_obj = torch.cuda.current_stream()
    job = GroupJob(ps, stream_obj.cuda_stream)
    job.call()
    torch.cuda.synchronize()
    plan = T.tcm_last_plan()
    print(f"[bench] plan: {plan}", file=sys.stderr, flush=True)
    ms, wall_ms = time_steps(job.call, args.steps, args.warmup, stream_obj)
    ms_each, _ = time_steps(job.call_each, args.steps, args.warmup, stream_obj)
    value = job.flops / (ms * 1e-3) / 1e12
    print(f"[bench] {ms:.4f} ms/step ({ms_each:.4f} one entry at a time), {value:.1f} TFLOP/s", file=sys.stderr,
          flush=True)
    parity = None
    if not args.no_cpu:
        job.call()
        torch.cuda.synchronize()
        parity = job.sampled_check()
    line = {
        "metric": "Grouped GEMM TFLOPS on 1 MI355X (one call for the whole group)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE_NAME[ps[0].dtype], "data": "synthetic",
        "config": {"workload": desc, "plan": plan, "wall_ms_per_step": round(wall_ms, 5),
                   "entries_one_by_one_ms": round(ms_each, 5), "parity": parity},
        "roofline": roofline(ps[0].dtype, job.flops, job.alg_bytes, ms,
                             load_traffic(types.SimpleNamespace(name=args.workload), plan)),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def run_bench(args):
    import torch

    import synthetic as S
    import tensor_core_mixed_amd as T
    if args.workload in S.CONV_WORKLOADS:
        return run_bench_conv(args)
    if args.workload in S.GROUP_WORKLOADS:
        return run_bench_group(args)
    p = S.workload(args.workload, **({"dist": args.dist} if args.dist else {}))
    torch.cuda.set_device(0)
    print(f"[bench] workload {p.name}: {describe(p)}", file=sys.stderr, flush=True)
    g = S.generate(p)
    A, B, bias = upload(g, p)
    C = make_c(p)
    stream_obj = torch.cuda.current_stream()
    call = make_call(p, A, B, bias, C, stream_obj.cuda_stream)
    reset_c(p, g, C)
    call()
    torch.cuda.synchronize()
    plan = T.tcm_last_plan()
    print(f"[bench] plan: {plan}", file=sys.stderr, flush=True)
    ms, wall_ms = time_steps(call, args.steps, args.warmup, stream_obj)
    calls = per_call_us(call, args.steps, stream_obj)
    flops = p.flops
    unit_scale = 1e12
    value = flops / (ms * 1e-3) / unit_scale
    print(f"[bench] {ms:.4f} ms/step, {value:.1f} T(FL)OP/s", file=sys.stderr, flush=True)
    roof = roofline(p.dtype, p.flops, p.alg_bytes, ms, load_traffic(p, plan))
    cpu, parity = None, None
    if not args.no_cpu:
        # CPU leg: one more call from the initial state, checked on sampled entries, then the oracle's rate
        reset_c(p, g, C)
        call()
        torch.cuda.synchronize()
        parity = _oracle_sampled_check(p, g, C)
        print(f"[bench] sampled check {parity}", file=sys.stderr, flush=True)
        cpu = cpu_baseline(p, g, unit_scale)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s" if p.dtype != 3 else "TOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAME[p.dtype],
        "data": "synthetic",
        "config": {"workload": describe(p), "M": p.M, "N": p.N, "K": p.K, "seed": p.seed, "dist": p.dist,
                   "plan": plan, "wall_ms_per_step": round(wall_ms, 5), "per_call_us": calls, "parity": parity},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.all:
        run_all(args)


def run_all(args):
    """Time every workload (DP, Stream-K and auto for the split-k shapes) -> stderr table."""
    import torch

    import synthetic as S
    import tensor_core_mixed_amd as T
    rows = []
    for name, p in S.WORKLOADS.items():
        g = S.generate(p)
        A, B, bias = upload(g, p)
        C = make_c(p)
        s = torch.cuda.current_stream()
        modes = [0, 1, 2] if name.startswith(("skinny", "sk_")) else [0]
        if name.startswith("skinny") and p.M <= 64:
            # the split-k GEMV forced, the tiled kernel's own plan, and the 4x4x4 GEMV kernel
            modes += [3, 4] + ([5] if p.M <= 16 else [])
        for mode in modes:
            T.tcm_set_option("force_mode", mode if mode <= 2 else 0)
            T.tcm_set_option("gemv", {3: 2, 4: 1, 5: 2}.get(mode, 0))
            T.tcm_set_option("gemv_wide", 1 if mode == 5 else 0)
            call = make_call(p, A, B, bias, C, s.cuda_stream)
            reset_c(p, g, C)
            call()
            torch.cuda.synchronize()
            plan = T.tcm_last_plan()
            ms, _ = time_steps(call, max(5, args.steps // 2), 10, s, min_warm_ms=200.0)
            pc = per_call_us(call, max(5, args.steps // 2), s)
            par = None
            if not args.no_cpu:  # CPU leg: sampled check of one call from the initial state
                reset_c(p, g, C)
                call()
                torch.cuda.synchronize()
                par = _oracle_sampled_check(p, g, C)
            v = p.flops / (ms * 1e-3) / 1e12
            row = {"workload": name, "mode": ["auto", "dp", "streamk", "gemv", "tiles", "gemv4x4x4"][mode], "ms": round(ms, 5),
                   "per_call_us": pc, "tflops": round(v, 2), "frac_peak": round(v / PEAK[p.dtype], 4),
                   "hbm_frac": round(p.alg_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                   "parity_ok": par["ok"] if par else None, "plan": plan}
            if name.startswith("skinny"):
                row["cold_median_us"] = cold_us(call, 20, s)
            if args.tune and mode == 0 and p.batch == 1:
                # the tuning table's choice for this signature, then the same timing
                code = p.dtype | (T.TCM_A_COLMAJOR if p.a_col else 0) | (T.TCM_B_COLMAJOR if p.b_col else 0)
                code |= {"acc": 0, "f16": T.TCM_C_F16, "bf16": T.TCM_C_BF16}[p.c_type]
                epi = (T.TCM_EPI_BIAS if p.bias else 0) | (T.TCM_EPI_RELU if p.relu else 0) | \
                      (T.TCM_EPI_ACCUM if p.accum else 0)
                st, best = T.tcm_tune(p.M, p.N, p.K, A.data_ptr(), p.LDA, B.data_ptr(), p.LDB, C.data_ptr(), p.LDC, code,
                                      bias.data_ptr() if bias is not None else None, epi, 10, s.cuda_stream)
                if st != 0:
                    raise RuntimeError(T.tcm_status_string(st))
                reset_c(p, g, C)
                call()
                torch.cuda.synchronize()
                tms, _ = time_steps(call, max(5, args.steps // 2), 10, s, min_warm_ms=200.0)
                row["tuned"] = {"ms": round(tms, 5), "plan": T.tcm_last_plan(), "model_over_tuned": round(ms / tms, 3)}
            rows.append(row)
        T.tcm_set_option("force_mode", 0)
        T.tcm_set_option("gemv", 0)
        T.tcm_set_option("gemv_wide", 0)
        mine = [r for r in rows if r["workload"] == name]
        by_mode = {r["mode"]: r for r in mine}
        if "dp" in by_mode and "streamk" in by_mode:
            lift = by_mode["dp"]["ms"] / by_mode["streamk"]["ms"]
            for r in mine:
                r["streamk_lift_dp_over_sk"] = round(lift, 3)
        if "gemv" in by_mode and "tiles" in by_mode:
            for r in mine:
                r["gemv_lift_tiles_over_gemv"] = round(by_mode["tiles"]["ms"] / by_mode["gemv"]["ms"], 3)
        if not args.no_cpu:
            import oracle
            r_cpu = min(p.M, max(1, int(2e10 // (2 * p.N * p.K))))
            dt = _oracle_rows(oracle.get(), p, g, r_cpu)
            for r in mine:
                r["cpu_oracle"] = {"tflops": round(2.0 * r_cpu * p.N * p.K / dt / 1e12, 5), "rows": r_cpu,
                                   "seconds": round(dt, 2), "threads": oracle.get().max_threads()}
        for r in mine:
            print("[all] " + json.dumps(r), file=sys.stderr, flush=True)
        del A, B, bias, C
        torch.cuda.empty_cache()
    for name, ps in S.GROUP_WORKLOADS.items():
        s = torch.cuda.current_stream()
        job = GroupJob(ps, s.cuda_stream)
        job.call()
        torch.cuda.synchronize()
        plan = T.tcm_last_plan()
        ms, _ = time_steps(job.call, max(5, args.steps // 2), 10, s, min_warm_ms=200.0)
        ms_each, _ = time_steps(job.call_each, max(5, args.steps // 2), 10, s, min_warm_ms=200.0)
        par = None
        if not args.no_cpu:
            job.call()
            torch.cuda.synchronize()
            par = job.sampled_check()
        v = job.flops / (ms * 1e-3) / 1e12
        row = {"workload": name, "mode": "auto", "ms": round(ms, 5), "tflops": round(v, 2),
               "frac_peak": round(v / PEAK[ps[0].dtype], 4),
               "hbm_frac": round(job.alg_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
               "entries_one_by_one_ms": round(ms_each, 5), "parity_ok": par["ok"] if par else None, "plan": plan}
        rows.append(row)
        print("[all] " + json.dumps(row), file=sys.stderr, flush=True)
        del job
        torch.cuda.empty_cache()
    for name, p in S.CONV_WORKLOADS.items():
        s = torch.cuda.current_stream()
        job = ConvJob(p, s.cuda_stream)
        job.call()
        torch.cuda.synchronize()
        plan = T.tcm_last_plan()
        ms, _ = time_steps(job.call, max(5, args.steps // 2), 10, s, min_warm_ms=200.0)
        pc = per_call_us(job.call, max(5, args.steps // 2), s)
        par = None
        if not args.no_cpu:
            job.call()
            torch.cuda.synchronize()
            par = job.sampled_check()
        v = p.flops / (ms * 1e-3) / 1e12
        row = {"workload": name, "mode": "auto", "ms": round(ms, 5), "per_call_us": pc, "tflops": round(v, 2),
               "frac_peak": round(v / PEAK[p.dtype], 4),
               "hbm_frac": round(p.alg_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
               "parity_ok": par["ok"] if par else None, "plan": plan}
        if not args.no_cpu:
            n = 1 << 16
            dt = job._oracle_seconds(n)
            row["cpu_oracle"] = {"tflops": round(2.0 * p.R * p.S * p.C * n / dt / 1e12, 5), "outputs": n,
                                 "seconds": round(dt, 2), "threads": oracle_threads()}
        rows.append(row)
        print("[all] " + json.dumps(row), file=sys.stderr, flush=True)
        del job
        torch.cuda.empty_cache()
    if args.report:
        with open(args.report, "w") as f:
            json.dump(rows, f, indent=1)


def render_report(src, dst):
    """A markdown table from the JSON rows `--all --report` writes."""
    rows = json.load(open(src))
    L = ["# bench.py --all: every workload, timed on one MI355X", "",
         "Made by `python -u bench.py --all --tune --no-cpu --report R.json` on the GPU, then "
         "`python bench.py --render-report R.json profiles/bench_all.md`.  Each case warms up for at least 200 ms; "
         "`block` is the average of back-to-back calls between two events, `per call` the median of calls timed one by "
         "one (it includes the launch gap).  For the split-k workloads every mode is timed: `auto` (the planner, with "
         "the shipped tuning table), `dp` (data-parallel tiles only) and `streamk`; `Stream-K lift` = dp / streamk.  "
         "Skinny products of at most 64 rows also run `gemv` (the split-k GEMV forced: the 16x16x32 kernel on row-major B) "
         "and `tiles` (the tiled kernel's own plan), and up to 16 rows `gemv4x4x4` (the GEMV's 4x4x4 kernel); "
         "`GEMV lift` = tiles / gemv.  `cold` "
         "(skinny products): the median call after a 512 MiB read that evicts the MALL (with clean lines).  `tuned`: the same call after "
         "`tcm_tune` searched it (block time).", "",
         "| workload | mode | block us | per call us | TFLOP/s (TOP/s) | of peak | of HBM | cold us | Stream-K lift | GEMV lift | tuned us | plan |",
         "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        pc = r.get("per_call_us", {}).get("median", "") if isinstance(r.get("per_call_us"), dict) else ""
        tuned = r.get("tuned", {}).get("ms")
        plan = " ".join(kv for kv in r["plan"].split() if kv.split("=")[0] in ("kernel", "config", "tile", "mode", "grid",
                                                                                  "fixup", "group", "tuned", "splits", "split",
                                                                                  "mfma"))
        L.append(f"| {r['workload']} | {r['mode']} | {r['ms'] * 1e3:.1f} | {pc} | {r['tflops']:.1f} | "
                 f"{100 * r['frac_peak']:.1f}% | {100 * r['hbm_frac']:.1f}% | {r.get('cold_median_us', '')} | "
                 f"{r.get('streamk_lift_dp_over_sk', '')} | {r.get('gemv_lift_tiles_over_gemv', '')} | "
                 f"{'' if tuned is None else f'{tuned * 1e3:.1f}'} | `{plan}` |")
    with open(dst, "w") as f:
        f.write("\n".join(L) + "\n")


def oracle_threads():
    import oracle
    return oracle.get().max_threads()


def run_sweep(args):
    """Every (tile config, mode) on the split-k workloads -> JSON rows (tuning data)."""
    import torch

    import synthetic as S
    import tensor_core_mixed_amd as T
    rows = []
    names = [n for n in S.WORKLOADS if n.startswith(("skinny", "sk_", "f16_512", "f32_2048", "i8_"))]
    for name in names:
        p = S.workload(name)
        g = S.generate(p)
        A, B, bias = upload(g, p)
        C = make_c(p)
        s = torch.cuda.current_stream()
        for cfg in range(T.tcm_config_count()):
            for mode in (1, 2):
                T.tcm_set_option("force_config", cfg)
                T.tcm_set_option("force_mode", mode)
                call = make_call(p, A, B, bias, C, s.cuda_stream)
                call()
                torch.cuda.synchronize()
                plan = T.tcm_last_plan()
                if f"config={cfg}" not in plan:
                    continue
                ms, _ = time_steps(call, 10, 10, s, min_warm_ms=200.0)
                rows.append({"workload": name, "config": cfg, "mode": mode, "us": round(ms * 1e3, 2), "plan": plan})
                print("[sweep] " + json.dumps(rows[-1]), file=sys.stderr, flush=True)
        T.tcm_set_option("force_config", -1)
        T.tcm_set_option("force_mode", 0)
        del A, B, bias, C
        torch.cuda.empty_cache()
    if args.report:
        with open(args.report, "w") as f:
            json.dump(rows, f, indent=1)


def calibrate_copy():
    """One device-to-device copy of exactly 512 MiB (read 512 MiB, write 512 MiB)."""
    import torch
    n = 512 * 2 ** 20 // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4}), flush=True)


def summarize_counters(d, name, calib=None):
    """profiles/traffic_<name>.json from rocprofv3 --pmc runs under d/{fetch,write} and the
    copy calibration under calib/{copy_fetch,copy_write} (calib defaults to d)."""
    import csv
    import glob

    calib = calib or d

    def per_kernel(root, sub, counter, kernel_pats):
        pats = (kernel_pats,) if isinstance(kernel_pats, str) else kernel_pats
        out = {}
        for f in glob.glob(os.path.join(root, sub, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter and any(k in r["Kernel_Name"] for k in pats):
                    out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    def per_dispatch_in(root, sub, counter, kernel_pat):
        files = glob.glob(os.path.join(root, sub, "**", "*counter_collection.csv"), recursive=True)
        vals = []
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter and kernel_pat in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
        return vals

    # per kernel (a Stream-K plan launches a data-parallel and a Stream-K kernel, and may sum its split
    # tiles in a second kernel; equal shares launch the shares' kernel and their sum): medians per dispatch
    import synthetic as S
    kpat = (("tile_conv_kernel", "conv_fixup_kernel") if name in S.CONV_WORKLOADS else
            ("tile_group_kernel", "group_fixup_kernel") if name in S.GROUP_WORKLOADS else
            ("tile_gemm_acol_kernel" if S.workload(name).a_col else "tile_gemm_kernel", "tile_fixup_kernel",
             "tile_split_kernel", "tile_split_fixup_kernel"))
    fetch = per_kernel(d, "fetch", "FETCH_SIZE", kpat)
    write = per_kernel(d, "write", "WRITE_SIZE", kpat)
    if not fetch:  # a product the split-k GEMV serves
        fetch = per_kernel(d, "fetch", "FETCH_SIZE", "tcm::gemv::")
        write = per_kernel(d, "write", "WRITE_SIZE", "tcm::gemv::")
    cf = per_dispatch_in(calib, "copy_fetch", "FETCH_SIZE", "copy")
    cw = per_dispatch_in(calib, "copy_write", "WRITE_SIZE", "copy")
    copy_kib = 512 * 1024
    f_fac = copy_kib / max(cf) if cf else 1.0
    w_fac = copy_kib / max(cw) if cw else 1.0
    kernels = {k: {"fetch_kib_per_dispatch": float(np.median(fetch[k])),
                   "write_kib_per_dispatch": float(np.median(write.get(k, [0.0]))),
                   "dispatches": len(fetch[k])} for k in fetch}
    dom = max(kernels, key=lambda k: kernels[k]["fetch_kib_per_dispatch"]) if kernels else None
    hbm = None
    if dom:
        kd = kernels[dom]
        hbm = (kd["fetch_kib_per_dispatch"] * f_fac + kd["write_kib_per_dispatch"] * w_fac) * 1024
    family = GEMV_SOURCES if dom and "tcm::gemv::" in dom else KERNEL_SOURCES
    out = {"workload": name, "source_hash": kernel_source_hash(family), "dominant_kernel": dom, "kernels": kernels,
           "copy_fetch_kib": max(cf) if cf else None, "copy_write_kib": max(cw) if cw else None,
           "fetch_scale": f_fac, "write_scale": w_fac, "hbm_bytes_per_launch": hbm}
    path = TRAFFIC_FILE.format(name=name)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed calls before the timed ones (the clock needs tens of ms of load to settle)")
    ap.add_argument("--workload", default="f16_8192")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--dist", default=None, choices=["uniform", "normal", "uniform12", "ones", "zeros"],
                    help="override the workload's value distribution (the matrix cores' clock depends on the data)")
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--report", default=None)
    ap.add_argument("--sweep", action="store_true", help="time every tile config and mode on the split-k workloads")
    ap.add_argument("--tune", action="store_true", help="with --all: also time each workload on its auto-tuned plan")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--render-report", nargs=2, metavar=("JSON", "MD"), default=None,
                    help="write the markdown table of a --all --report JSON file (host only)")
    ap.add_argument("--summarize-counters", default=None)
    ap.add_argument("--calibration", default=None, help="directory holding the copy-calibration counter runs")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, args.calibration)
        return
    if args.render_report:
        render_report(*args.render_report)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this engine runs on one GPU: every GPU box here has one, and the GEMM path "
                                   "has no collectives; run with --gpus 1"}), flush=True)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.sweep:
        run_sweep(args)
        return
    run_bench(args)


if __name__ == "__main__":
    main()
