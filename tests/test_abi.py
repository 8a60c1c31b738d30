"""The C interface on the CPU: the library loads, exports every function the
header declares, sizes its workspace, and rejects bad arguments before any
launch (so these calls never need a GPU)."""

import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "spec_verify.h")


@pytest.fixture(scope="module")
def lib():
    from lossless_draft_verification_sample_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from lossless_draft_verification_sample_amd import build
        build.build()
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert {"spec_verify_sample", "spec_verify_greedy", "spec_verify_workspace_bytes",
            "spec_verify_strerror"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_names_match_header():
    import lossless_draft_verification_sample_amd as sv
    for n in _declared_functions():
        assert callable(getattr(sv, n)), n


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.spec_verify_strerror(code)
    assert b"unknown" in lib.spec_verify_strerror(42)


def test_workspace_bytes(lib):
    ws = lib.spec_verify_workspace_bytes
    a = ws(128, 8, 151936)
    assert a > 0 and a % 256 == 0
    assert ws(1, 4, 1000) > 0
    # room for the row statistics (32 B per row), the uniforms (8 B per slot),
    # the draw's sub-chunk sums (16 B per 2048 tokens per request) and lists
    # of up to 32 kept tokens per sub-chunk (a 4-byte length, 4-byte ids,
    # 8-byte weights), and the per-request arrival counters
    B, g, V = 128, 8, 151936
    nsub = -(-V // 2048)
    assert a >= (B * (2 * g + 1) * 32 + B * (g + 1) * 8 + B * nsub * 16
                 + B * nsub * (4 + 32 * 12) + B * 4)
    for bad in [(0, 4, 10), (1, 0, 10), (1, 64, 10), (1, 4, 0), (2**30, 63, 10)]:
        assert ws(*bad) == 0, bad


FAKE = 4096  # non-null, aligned; never dereferenced because validation fails first


def _sample(lib, **kw):
    from lossless_draft_verification_sample_amd._lib import SvSampler
    a = dict(target=FAKE, draft=FAKE, dtype=1, tokens=FAKE, banned=None, n_banned=0, B=2,
             gamma=3, V=100, ts=SvSampler(1.0, 0, 1.0), ds=SvSampler(1.0, 0, 1.0), seed=0,
             offset=0, requests=None, uniforms=None, out_tokens=FAKE, out_n=FAKE, out_flags=None,
             out_tl=None, out_dl=None, out_ov=None, out_hist=None, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return lib.spec_verify_sample(
        a["target"], a["draft"], a["dtype"], a["tokens"], a["banned"], a["n_banned"], a["B"],
        a["gamma"], a["V"], a["ts"], a["ds"], a["requests"], a["seed"], a["offset"], a["uniforms"],
        a["out_tokens"], a["out_n"], a["out_flags"], a["out_tl"], a["out_dl"], a["out_ov"],
        a["out_hist"], a["ws"], a["ws_bytes"], a["stream"])


def test_sample_argument_errors(lib):
    from lossless_draft_verification_sample_amd import _lib as L
    S = L.SvSampler
    # everything valid except the workspace: rejected before launching
    assert _sample(lib) == L.SV_EWORKSPACE
    need = lib.spec_verify_workspace_bytes(2, 3, 100)
    assert _sample(lib, ws=FAKE, ws_bytes=need - 1) == L.SV_EWORKSPACE
    assert _sample(lib, ws=FAKE + 8, ws_bytes=need) == L.SV_EWORKSPACE   # misaligned
    cases = {
        "target": dict(target=None), "draft": dict(draft=None), "tokens": dict(tokens=None),
        "out_tokens": dict(out_tokens=None), "out_n": dict(out_n=None),
        "B": dict(B=0), "gamma0": dict(gamma=0), "gamma64": dict(gamma=64), "V": dict(V=0),
        "n_banned<0": dict(n_banned=-1), "n_banned big": dict(n_banned=2049, banned=FAKE),
        "banned null": dict(n_banned=3), "T=0": dict(ts=S(0.0, 0, 1.0)),
        "T<0": dict(ds=S(-1.0, 0, 1.0)), "T nan": dict(ts=S(float("nan"), 0, 1.0)),
        "T inf": dict(ts=S(float("inf"), 0, 1.0)), "top_k<0": dict(ds=S(1.0, -1, 1.0)),
        "top_p=0": dict(ts=S(1.0, 0, 0.0)), "top_p>1": dict(ts=S(1.0, 0, 1.5)),
        "top_p nan": dict(ds=S(1.0, 0, float("nan"))), "misaligned": dict(target=FAKE + 1),
    }
    for name, kw in cases.items():
        assert _sample(lib, **kw) == L.SV_EINVAL, name
    assert _sample(lib, dtype=2) == L.SV_EDTYPE
    assert _sample(lib, dtype=0, target=FAKE + 2) == L.SV_EINVAL   # fp32 needs 4-byte alignment
    assert _sample(lib, B=2**30, gamma=63) == L.SV_ESIZE
    import ctypes
    bad_req = L.SvRequests(None, None, None, None, 3)          # n_banned_draft without a list
    assert _sample(lib, requests=ctypes.byref(bad_req)) == L.SV_EINVAL
    big = L.SvRequests(None, None, None, FAKE, 2049)
    assert _sample(lib, requests=ctypes.byref(big)) == L.SV_EINVAL


def test_history_bound(lib):
    """n_history above SV_MAX_HISTORY is rejected before any launch, and the
    bound keeps every row's penalized ids (history plus up to 63 earlier
    proposals) within half of the kernels' 4096-slot on-chip hash set."""
    import ctypes
    from lossless_draft_verification_sample_amd import _lib as L
    hdr = open(HEADER).read()
    hist_max = int(re.search(r"#define SV_MAX_HISTORY (\d+)", hdr).group(1))
    bans_max = int(re.search(r"#define SV_MAX_BANNED (\d+)", hdr).group(1))
    assert L.SV_MAX_HISTORY == hist_max and L.SV_MAX_BANNED == bans_max
    bans = open(os.path.join(ROOT, "lossless_draft_verification_sample_amd", "csrc",
                             "sv_bans.hpp")).read()
    slots = int(re.search(r"HT_SLOTS = (\d+)", bans).group(1))
    max_gamma = 63
    assert hist_max + max_gamma <= slots // 2
    assert bans_max <= slots // 2
    need = lib.spec_verify_workspace_bytes(2, 3, 100)
    ok = dict(ws=FAKE, ws_bytes=need)
    # the largest list passes validation (it then fails only on the fake device
    # pointers, which a CPU test cannot launch with, so check the rejection side)
    over = L.SvRequests(None, None, None, None, 0, FAKE, hist_max + 1, None, None)
    assert _sample(lib, requests=ctypes.byref(over), **ok) == L.SV_EINVAL
    neg = L.SvRequests(None, None, None, None, 0, FAKE, -1, None, None)
    assert _sample(lib, requests=ctypes.byref(neg), **ok) == L.SV_EINVAL
    nolist = L.SvRequests(None, None, None, None, 0, None, 5, None, None)
    assert _sample(lib, requests=ctypes.byref(nolist), **ok) == L.SV_EINVAL


def test_noalloc_rejects_sizes_beyond_the_scratch(lib):
    """spec_verify_sample_noalloc validates like spec_verify_sample and rejects
    sizes whose workspace exceeds its static scratch, before touching a device."""
    from lossless_draft_verification_sample_amd import _lib as L
    S = L.SvSampler(1.0, 0, 1.0)
    na = lib.spec_verify_sample_noalloc

    def call(B, gamma, V, target=FAKE):
        return na(target, FAKE, L.SV_BF16, FAKE, None, 0, B, gamma, V, S, S, None, 0, 0, None,
                  FAKE, FAKE, None, None, None, None, None, None)
    assert lib.spec_verify_workspace_bytes(8192, 8, 1 << 20) > L.SV_NOALLOC_SCRATCH_BYTES
    assert call(8192, 8, 1 << 20) == L.SV_ESCRATCH
    assert call(8192, 8, 1 << 20, target=None) == L.SV_EINVAL   # argument checks come first
    assert call(0, 8, 1000) == L.SV_EINVAL
    assert lib.spec_verify_workspace_bytes(128, 8, 151936) <= L.SV_NOALLOC_SCRATCH_BYTES
    assert b"scratch" in lib.spec_verify_strerror(L.SV_ESCRATCH)


def test_greedy_argument_errors(lib):
    from lossless_draft_verification_sample_amd import _lib as L
    g = lib.spec_verify_greedy
    assert g(None, 1, FAKE, None, 0, 2, 3, 10, FAKE, FAKE, None, None, None) == L.SV_EINVAL
    assert g(FAKE, 1, None, None, 0, 2, 3, 10, FAKE, FAKE, None, None, None) == L.SV_EINVAL
    assert g(FAKE, 1, FAKE, None, 0, 2, 3, 10, None, FAKE, None, None, None) == L.SV_EINVAL
    assert g(FAKE, 1, FAKE, None, 0, 2, 3, 10, FAKE, None, None, None, None) == L.SV_EINVAL
    assert g(FAKE, 5, FAKE, None, 0, 2, 3, 10, FAKE, FAKE, None, None, None) == L.SV_EDTYPE
    assert g(FAKE, 1, FAKE, None, 0, 0, 3, 10, FAKE, FAKE, None, None, None) == L.SV_EINVAL
    assert g(FAKE, 1, FAKE, None, 0, 2, 0, 10, FAKE, FAKE, None, None, None) == L.SV_EINVAL
    assert g(FAKE, 1, FAKE, None, 0, 2, 3, 0, FAKE, FAKE, None, None, None) == L.SV_EINVAL
    assert g(FAKE + 1, 1, FAKE, None, 0, 2, 3, 10, FAKE, FAKE, None, None, None) == L.SV_EINVAL
    assert g(FAKE, 1, FAKE, None, 0, 2**30, 3, 10, FAKE, FAKE, None, None, None) == L.SV_ESIZE
    assert g(FAKE, 1, FAKE, None, 3, 2, 3, 10, FAKE, FAKE, None, None, None) == L.SV_EINVAL
    assert g(FAKE, 1, FAKE, FAKE, 2049, 2, 3, 10, FAKE, FAKE, None, None, None) == L.SV_EINVAL


def test_commit_argument_errors(lib):
    from lossless_draft_verification_sample_amd import _lib as L
    c = lib.spec_verify_commit
    ok = dict(tok=FAKE, n=FAKE, kv=FAKE, slots=None, B=4, g=3, nk=FAKE, an=FAKE, nf=None, fs=None)

    def call(**kw):
        a = dict(ok, **kw)
        return c(a["tok"], a["n"], a["kv"], a["slots"], None, a["B"], a["g"], a["nk"], a["an"],
                 a["nf"], a["fs"], None)
    for name, kw in {"tokens": dict(tok=None), "num_accepted": dict(n=None), "kv_len": dict(kv=None),
                     "new_kv_len": dict(nk=None), "anchor": dict(an=None),
                     "free without slots": dict(fs=FAKE), "B": dict(B=0), "gamma0": dict(g=0),
                     "gamma64": dict(g=64)}.items():
        assert call(**kw) == L.SV_EINVAL, name
    assert call(B=2**30, g=63) == L.SV_ESIZE


def test_timing_lives_in_the_bench_build_only(lib):
    """The product library has no event timing; the benchmark build exports the
    same entry points plus the two timing calls, which reject misuse."""
    from lossless_draft_verification_sample_amd import _lib as L
    assert not hasattr(lib, "sv_bench_profile_start")
    assert not hasattr(lib, "sv_bench_profile_stop")
    bench = L.load_bench()
    for n in _declared_functions():
        assert hasattr(bench, n), n
    assert bench.sv_bench_profile_stop(None, None) == L.SV_EINVAL
    assert bench.sv_bench_profile_start(0) == L.SV_EINVAL


def test_product_does_not_import_oracle():
    pkg = os.path.join(ROOT, "lossless_draft_verification_sample_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f


def test_calibration_library_exports_and_rejects_bad_arguments():
    # the read-bandwidth calibration kernel lives in its own library; argument
    # checks run before any launch
    from lossless_draft_verification_sample_amd import build
    path = os.path.join(build.PKG_DIR, build.CALIB_LIB_NAME)
    if not os.path.exists(path):
        build.build()
    cal = ctypes.CDLL(path)
    cal.sv_calib_read_blocks.restype = ctypes.c_int64
    cal.sv_calib_read_blocks.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    cal.sv_calib_read.restype = ctypes.c_int
    cal.sv_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert cal.sv_calib_read_blocks(1 << 20, 0, 0, 2048) == 2048
    assert cal.sv_calib_read_blocks(1000 * 16, 1, 48, 0) == (1000 * 16 + 47) // 48
    assert cal.sv_calib_read_blocks(100, 0, 0, 64) == -1          # not a multiple of 16
    assert cal.sv_calib_read_blocks(1 << 20, 1, 24, 0) == -1      # chunk not a multiple of 16
    assert cal.sv_calib_read_blocks(1 << 20, 2, 16, 0) == -1      # unknown mode
    assert cal.sv_calib_read(None, 1 << 20, 0, 0, 64, None, None) == -1
    assert cal.sv_calib_read(16, 1 << 20, 0, 0, 64, None, None) == -1   # no output
    assert cal.sv_calib_read(8, 1 << 20, 0, 0, 64, 16, None) == -1      # misaligned
