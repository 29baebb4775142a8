"""Build the HIP library libtcm.so (gfx950 only) in-tree.

    python -m tensor_core_mixed_amd.build        # or: python tensor_core_mixed_amd/build.py

Every source under csrc/ is compiled with hipcc for gfx950 in parallel and
linked into tensor_core_mixed_amd/_build/libtcm.so.  Packed-FP32 VALU
instructions are disabled for all device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_build")
LIB = os.path.join(OUT, "libtcm.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]
# Per-source flags.  The GEMV kernels take their matrix-core accumulators in
# the architectural registers: with the accumulation registers the compiler
# copied the 64-row kernel's 128 accumulators out and back every step.
EXTRA_FLAGS = {"gemv_kernel.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(quiet=False, jobs=None):
    os.makedirs(OUT, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    if not quiet:
        print(f"[tcm] compiling {len(srcs)} sources for {ARCH} with {jobs} jobs", flush=True)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if not quiet:
        print(f"[tcm] built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(quiet="-q" in sys.argv)
