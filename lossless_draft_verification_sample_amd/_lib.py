"""ctypes declarations of the C interface in include/spec_verify.h.

Loading fails loudly when the HIP library has not been built; there is no
fallback implementation. load_bench() loads the benchmark build of the same
sources (libspecverify_bench.so), which adds per-kernel event timing
(csrc/sv_bench_timing.h); only bench.py uses it.
"""

import ctypes
import os

LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)
BENCH_LIB_NAME = "libspecverify_bench.so"
BENCH_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), BENCH_LIB_NAME)

SV_F32 = 0
SV_BF16 = 1

SV_OK = 0
SV_EINVAL = -1
SV_EDTYPE = -2
SV_EWORKSPACE = -3
SV_ESIZE = -4
SV_EHIP = -5
SV_ESCRATCH = -6
SV_NOALLOC_SCRATCH_BYTES = 8 << 20

SV_FLAG_TOKEN_RANGE = 1
SV_FLAG_Q_ZERO = 2
SV_FLAG_NONFINITE = 4
SV_FLAG_EMPTY = 8
SV_FLAG_RESIDUAL_ZERO = 16
SV_FLAG_BAD_PARAM = 32

SV_MAX_BANNED = 2048
SV_MAX_HISTORY = 1984

# kernel indices of sv_bench_profile_stop (csrc/sv_bench_timing.h)
SV_K_ROW_STATS = 0
SV_K_DRAW = 1
SV_K_GREEDY_ARGMAX = 2
SV_K_GREEDY_SCAN = 3
SV_K_OVERLAP = 4
SV_K_COMMIT = 5
SV_NUM_KERNELS = 6
KERNEL_NAMES = ["row_stats", "draw", "greedy_argmax", "greedy_scan", "overlap", "commit"]


class SvSampler(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_float)]


class SvRequests(ctypes.Structure):
    """sv_requests: device pointers (as integers) of per-request arrays."""
    _fields_ = [("gamma", ctypes.c_void_p), ("target", ctypes.c_void_p),
                ("draft", ctypes.c_void_p), ("banned_draft", ctypes.c_void_p),
                ("n_banned_draft", ctypes.c_int32), ("history", ctypes.c_void_p),
                ("n_history", ctypes.c_int32), ("penalty", ctypes.c_void_p),
                ("penalty_draft", ctypes.c_void_p)]


_c = ctypes
_vp = _c.c_void_p
_i32 = _c.c_int32
_u64 = _c.c_uint64

SIGNATURES = {
    "spec_verify_workspace_bytes": (_c.c_size_t, [_i32, _i32, _i32]),
    "spec_verify_sample": (_c.c_int, [
        _vp, _vp, _c.c_int, _vp, _vp, _i32, _i32, _i32, _i32, SvSampler, SvSampler,
        _c.POINTER(SvRequests), _u64, _u64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
        _c.c_size_t, _vp]),
    "spec_verify_sample_noalloc": (_c.c_int, [
        _vp, _vp, _c.c_int, _vp, _vp, _i32, _i32, _i32, _i32, SvSampler, SvSampler,
        _c.POINTER(SvRequests), _u64, _u64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "spec_verify_greedy": (_c.c_int, [_vp, _c.c_int, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                                      _vp, _vp, _vp]),
    "spec_verify_commit": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp,
                                      _vp]),
    "spec_verify_strerror": (_c.c_char_p, [_c.c_int]),
}
BENCH_SIGNATURES = {
    "sv_bench_profile_start": (_c.c_int, [_i32]),
    "sv_bench_profile_stop": (_c.c_int, [_vp, _vp]),
}

_LIB = None
_BENCH_LIB = None


def _open(path, name, sigs):
    if not os.path.exists(path):
        raise RuntimeError(
            f"{name} is not built ({path}); run "
            "`python -m lossless_draft_verification_sample_amd.build` or __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    for fname, (res, args) in sigs.items():
        fn = getattr(lib, fname)
        fn.restype = res
        fn.argtypes = args
    return lib


def load(path=LIB_PATH):
    """The loaded library with argument types set (cached)."""
    global _LIB
    if _LIB is None:
        _LIB = _open(path, LIB_NAME, SIGNATURES)
    return _LIB


def load_bench(path=BENCH_LIB_PATH):
    """The benchmark build (same entry points plus per-kernel event timing)."""
    global _BENCH_LIB
    if _BENCH_LIB is None:
        _BENCH_LIB = _open(path, BENCH_LIB_NAME, {**SIGNATURES, **BENCH_SIGNATURES})
    return _BENCH_LIB
