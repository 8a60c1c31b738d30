"""Build libspecverify.so (the HIP library behind include/spec_verify.h) and
libsvcalib.so (an HBM read-bandwidth calibration kernel) for gfx950.

    python -m lossless_draft_verification_sample_amd.build

Compiles in-tree with hipcc; the shared object lands next to this file.
"""

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libspecverify.so"
SOURCES = ["row_stats.hip", "verify.hip", "overlap.hip", "greedy.hip", "commit.hip", "api.cpp"]
# HBM read-bandwidth calibration (bench.py --read-ceiling); not on the path
CALIB_LIB_NAME = "libsvcalib.so"
CALIB_SOURCES = ["calib/read_ceiling.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    # IEEE float32 division: the repetition penalty divides logits
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def build(verbose=False, out_dir=PKG_DIR):
    out = _compile(LIB_NAME, SOURCES, verbose, out_dir)
    _compile(CALIB_LIB_NAME, CALIB_SOURCES, verbose, out_dir)
    return out


def _compile(lib_name, sources, verbose, out_dir):
    out = os.path.join(out_dir, lib_name)
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in sources]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
