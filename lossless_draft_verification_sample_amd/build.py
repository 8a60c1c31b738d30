"""Build the HIP libraries of the package for gfx950, in-tree.

    python -m lossless_draft_verification_sample_amd.build [-v]

- libspecverify.so: the verifier behind include/spec_verify.h.
- libspecverify_bench.so: the same kernels and entry points, plus HIP event
  pairs around every launch and the two calls that read them
  (csrc/sv_bench_timing.h). Only bench.py loads it, for per-kernel times.
- libsvcalib.so: an HBM read-bandwidth calibration kernel (bench.py
  --read-ceiling); not on the verification path.

Every source is compiled to an object (in parallel) under _build/, then the
objects are linked; the shared objects land next to this file.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libspecverify.so"
BENCH_LIB_NAME = "libspecverify_bench.so"
KERNEL_SOURCES = ["row_stats.hip", "verify.hip", "overlap.hip", "greedy.hip", "commit.hip"]
API_SOURCE = "api.cpp"
# HBM read-bandwidth calibration (bench.py --read-ceiling); not on the path
CALIB_LIB_NAME = "libsvcalib.so"
CALIB_SOURCES = ["calib/read_ceiling.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    # IEEE float32 division: the repetition penalty divides logits
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    f"-I{os.path.join(ROOT, 'include')}",
]
NOISE = "packed-fp32-ops"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)


def _object(src, tag, extra, verbose):
    os.makedirs(OBJ_DIR, exist_ok=True)
    base = os.path.splitext(os.path.basename(src))[0]
    obj = os.path.join(OBJ_DIR, f"{base}{tag}.o")
    _run([hipcc(), *HIPCC_FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, src)], verbose)
    return obj


def _link(lib_name, objs, verbose, out_dir):
    out = os.path.join(out_dir, lib_name)
    tmp = out + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


def build(verbose=False, out_dir=PKG_DIR):
    """Compiles every source and links the three libraries; returns the path of
    libspecverify.so."""
    jobs = [(s, "", []) for s in KERNEL_SOURCES + CALIB_SOURCES]
    jobs += [(API_SOURCE, "", []), (API_SOURCE, "_bench", ["-DSV_BENCH_TIMING"])]
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda j: _object(*j, verbose), jobs))
    kern = objs[: len(KERNEL_SOURCES)]
    calib = objs[len(KERNEL_SOURCES): len(KERNEL_SOURCES) + len(CALIB_SOURCES)]
    api, api_bench = objs[-2], objs[-1]
    out = _link(LIB_NAME, kern + [api], verbose, out_dir)
    _link(BENCH_LIB_NAME, kern + [api_bench], verbose, out_dir)
    _link(CALIB_LIB_NAME, calib, verbose, out_dir)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
