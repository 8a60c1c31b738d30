"""Lossless speculative-sampling verifier for AMD MI355X (gfx950).

Thin Python binding over the C interface of include/spec_verify.h. The
functions below only marshal arguments (device pointers of torch tensors, the
current HIP stream) and allocate outputs; every step of verification runs in
the HIP kernels of libspecverify.so. PyTorch supplies device memory and
streams. If the library is missing, every call raises.
"""

from collections import namedtuple

from . import _lib
from ._lib import (  # noqa: F401
    SV_BF16,
    SV_EDTYPE,
    SV_EHIP,
    SV_ESCRATCH,
    SV_EINVAL,
    SV_ESIZE,
    SV_EWORKSPACE,
    SV_F32,
    SV_FLAG_BAD_PARAM,
    SV_FLAG_EMPTY,
    SV_FLAG_NONFINITE,
    SV_FLAG_Q_ZERO,
    SV_FLAG_RESIDUAL_ZERO,
    SV_FLAG_TOKEN_RANGE,
    SV_MAX_BANNED,
    SV_MAX_HISTORY,
    SV_NOALLOC_SCRATCH_BYTES,
    SV_OK,
    SvRequests,
    SvSampler,
)

SampleOut = namedtuple("SampleOut",
                       "tokens num_accepted flags target_lse draft_lse overlap accept_hist",
                       defaults=(None, None))
GreedyOut = namedtuple("GreedyOut", "tokens num_accepted flags accept_hist", defaults=(None,))
CommitOut = namedtuple("CommitOut", "new_kv_len anchor n_free free_slots")
# Per-request settings of a mixed batch (see sv_requests in include/spec_verify.h):
# gamma [B] int32, target / draft [B, 12] uint8 sv_sampler records (sampler_array),
# banned_draft [B, m] int32, history [B, H] int32, penalty / penalty_draft [B]
# float32 repetition penalties; None keeps the call-wide value (no penalty).
Requests = namedtuple("Requests",
                      "gamma target draft banned_draft history penalty penalty_draft",
                      defaults=(None,) * 7)


class SpecVerifyError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {spec_verify_strerror(status)} (status {status})")
        self.status = status


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _checked(t, name, dtype, shape):
    """Device pointer of an optional output whose shape the library assumes."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return _dev_ptr(t, name, dtype)


def _sampler(s):
    if isinstance(s, SvSampler):
        return s
    if isinstance(s, dict):
        return SvSampler(float(s.get("temperature", 1.0)), int(s.get("top_k", 0)),
                         float(s.get("top_p", 1.0)))
    t, k, p = s
    return SvSampler(float(t), int(k), float(p))


def sampler_array(samplers, device):
    """[B] sv_sampler records (float temperature, int32 top_k, float top_p) on
    `device`, as a [B, 12] uint8 tensor, from (temperature, top_k, top_p)
    tuples, dicts or SvSampler."""
    import numpy as np
    torch = _torch()
    rec = np.zeros(len(samplers), dtype=[("t", "<f4"), ("k", "<i4"), ("p", "<f4")])
    for j, smp in enumerate(samplers):
        c = _sampler(smp)
        rec[j] = (c.temperature, c.top_k, c.top_p)
    return torch.from_numpy(rec.view(np.uint8).reshape(len(samplers), 12).copy()).to(device)


def _requests(req, B):
    """ctypes sv_requests for a Requests tuple (or None)."""
    import ctypes
    if req is None:
        return None
    torch = _torch()
    for name, t in (("target", req.target), ("draft", req.draft)):
        if t is not None and (tuple(t.shape) != (B, 12) or t.dtype != torch.uint8):
            raise ValueError(f"requests.{name} must be a [B, 12] uint8 tensor (sampler_array)")
    if req.gamma is not None and tuple(req.gamma.shape) != (B,):
        raise ValueError("requests.gamma must be [B]")
    nbd = 0
    if req.banned_draft is not None:
        nbd = int(req.banned_draft.shape[1])
        if tuple(req.banned_draft.shape) != (B, nbd):
            raise ValueError("requests.banned_draft must be [B, n]")
    nh = 0
    if req.history is not None:
        nh = int(req.history.shape[1])
        if tuple(req.history.shape) != (B, nh):
            raise ValueError("requests.history must be [B, H]")
        if nh > SV_MAX_HISTORY:
            raise ValueError(f"requests.history holds {nh} > SV_MAX_HISTORY = {SV_MAX_HISTORY} "
                             "tokens per request")
    r = SvRequests(_dev_ptr(req.gamma, "requests.gamma", torch.int32),
                   _dev_ptr(req.target, "requests.target"), _dev_ptr(req.draft, "requests.draft"),
                   _dev_ptr(req.banned_draft, "requests.banned_draft", torch.int32), nbd,
                   _dev_ptr(req.history, "requests.history", torch.int32), nh,
                   _checked(req.penalty, "requests.penalty", torch.float32, (B,)),
                   _checked(req.penalty_draft, "requests.penalty_draft", torch.float32, (B,)))
    return ctypes.byref(r), r


def _stream(stream):
    """(hipStream_t handle, torch stream) of the call. None means torch's
    current stream; a raw handle is wrapped as an external stream. Outputs and
    the workspace the binding allocates are allocated on that stream, so the
    caching allocator keeps them until the call's kernels have run."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    elif not isinstance(stream, torch.cuda.Stream):
        stream = (torch.cuda.default_stream() if int(stream) == 0
                  else torch.cuda.ExternalStream(int(stream)))
    return stream.cuda_stream, stream


def spec_verify_strerror(status):
    return _lib.load().spec_verify_strerror(int(status)).decode()


def spec_verify_workspace_bytes(B, gamma, V):
    return int(_lib.load().spec_verify_workspace_bytes(int(B), int(gamma), int(V)))


def spec_verify_sample_noalloc(target_logits, draft_logits, draft_tokens,
                               target_sampler=(1.0, 0, 1.0), draft_sampler=(1.0, 0, 1.0),
                               banned_ids=None, seed=0, offset=0, uniforms=None, want_lse=True,
                               want_overlap=False, want_hist=False, requests=None, out=None,
                               stream=None, lib=None):
    """spec_verify_sample on the library's static per-GPU scratch instead of a
    workspace (see include/spec_verify.h). Pass `out` to avoid every
    allocation in this binding as well."""
    return spec_verify_sample(target_logits, draft_logits, draft_tokens, target_sampler,
                              draft_sampler, banned_ids, seed, offset, uniforms, want_lse,
                              want_overlap, want_hist, requests, None, out, stream, lib,
                              _noalloc=True)


def spec_verify_sample(target_logits, draft_logits, draft_tokens, target_sampler=(1.0, 0, 1.0),
                       draft_sampler=(1.0, 0, 1.0), banned_ids=None, seed=0, offset=0,
                       uniforms=None, want_lse=True, want_overlap=False, want_hist=False,
                       requests=None, workspace=None, out=None, stream=None, lib=None,
                       _noalloc=False):
    """Speculative-sampling verification of a batch (see include/spec_verify.h).

    target_logits [B, gamma+1, V] and draft_logits [B, gamma, V] (bf16 or fp32),
    draft_tokens [B, gamma] int32, banned_ids [B, n] int32 or None,
    uniforms [B, gamma+1] float64 or None (then Philox(seed, offset)).
    Samplers are (temperature, top_k, top_p) tuples, dicts or SvSampler.
    want_overlap adds the per-position overlaps [B, gamma] (float64; one more
    read of the rows), want_hist the accepted-prefix histogram [gamma+1]
    (int32 storage of the library's uint32 counts). requests: a Requests tuple
    of per-request settings (mixed batch) or None. stream: a torch stream, a
    raw hipStream_t handle or None (torch's current stream). lib: the loaded
    library to call (default libspecverify.so; bench.py passes the timing
    build).
    Returns SampleOut(tokens, num_accepted, flags, target_lse, draft_lse,
    overlap, accept_hist).
    """
    torch = _torch()
    lib = lib or _lib.load()
    B, G1, V = target_logits.shape
    gamma = G1 - 1
    if tuple(draft_logits.shape) != (B, gamma, V):
        raise ValueError("draft_logits must be [B, gamma, V]")
    if draft_logits.dtype != target_logits.dtype:
        raise TypeError("target and draft logits must share a dtype")
    if tuple(draft_tokens.shape) != (B, gamma):
        raise ValueError("draft_tokens must be [B, gamma]")
    dt = _dtype_code(target_logits)
    n_banned = 0 if banned_ids is None else int(banned_ids.shape[1])
    if banned_ids is not None and tuple(banned_ids.shape) != (B, n_banned):
        raise ValueError("banned_ids must be [B, n_banned]")
    if uniforms is not None and tuple(uniforms.shape) != (B, G1):
        raise ValueError("uniforms must be [B, gamma+1]")
    dev = target_logits.device
    handle, strm = _stream(stream)
    with torch.cuda.stream(strm):
        if out is None:
            out = SampleOut(
                torch.empty((B, G1), dtype=torch.int32, device=dev),
                torch.empty((B,), dtype=torch.int32, device=dev),
                torch.empty((B,), dtype=torch.int32, device=dev),
                torch.empty((B, G1), dtype=torch.float32, device=dev) if want_lse else None,
                torch.empty((B, gamma), dtype=torch.float32, device=dev) if want_lse else None,
                torch.empty((B, gamma), dtype=torch.float64, device=dev) if want_overlap else None,
                torch.empty((G1,), dtype=torch.int32, device=dev) if want_hist else None,
            )
        if workspace is None and not _noalloc:
            need = lib.spec_verify_workspace_bytes(B, gamma, V)
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    req = _requests(requests, B)
    fn = lib.spec_verify_sample_noalloc if _noalloc else lib.spec_verify_sample
    ws_args = () if _noalloc else (_dev_ptr(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size())
    rc = fn(
        _dev_ptr(target_logits, "target_logits"), _dev_ptr(draft_logits, "draft_logits"), dt,
        _dev_ptr(draft_tokens, "draft_tokens", torch.int32),
        _dev_ptr(banned_ids, "banned_ids", torch.int32), n_banned, B, gamma, V,
        _sampler(target_sampler), _sampler(draft_sampler), None if req is None else req[0],
        int(seed), int(offset),
        _dev_ptr(uniforms, "uniforms", torch.float64),
        _dev_ptr(out.tokens, "out_tokens", torch.int32),
        _dev_ptr(out.num_accepted, "out_num_accepted", torch.int32),
        _dev_ptr(out.flags, "out_flags", torch.int32),
        _dev_ptr(out.target_lse, "out_target_lse", torch.float32),
        _dev_ptr(out.draft_lse, "out_draft_lse", torch.float32),
        _checked(out.overlap, "out_overlap", torch.float64, (B, gamma)),
        _checked(out.accept_hist, "out_accept_hist", torch.int32, (G1,)), *ws_args, handle)
    if rc != SV_OK:
        raise SpecVerifyError(rc, fn.__name__)
    return out


def spec_verify_greedy(target_logits, draft_tokens, banned_ids=None, want_hist=False, out=None,
                       stream=None, lib=None):
    """Greedy verification (see include/spec_verify.h); banned_ids [B, n] int32
    or None; stream and lib as for spec_verify_sample.
    Returns GreedyOut(tokens, num_accepted, flags, accept_hist)."""
    torch = _torch()
    lib = lib or _lib.load()
    B, G1, V = target_logits.shape
    gamma = G1 - 1
    if tuple(draft_tokens.shape) != (B, gamma):
        raise ValueError("draft_tokens must be [B, gamma]")
    n_banned = 0 if banned_ids is None else int(banned_ids.shape[1])
    if banned_ids is not None and tuple(banned_ids.shape) != (B, n_banned):
        raise ValueError("banned_ids must be [B, n_banned]")
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    handle, strm = _stream(stream)
    if out is None:
        with torch.cuda.stream(strm):
            out = GreedyOut(torch.empty((B, G1), dtype=torch.int32, device=dev),
                            torch.empty((B,), dtype=torch.int32, device=dev),
                            torch.empty((B,), dtype=torch.int32, device=dev),
                            torch.empty((G1,), dtype=torch.int32, device=dev) if want_hist else None)
    rc = lib.spec_verify_greedy(
        _dev_ptr(target_logits, "target_logits"), dt,
        _dev_ptr(draft_tokens, "draft_tokens", torch.int32),
        _dev_ptr(banned_ids, "banned_ids", torch.int32), n_banned, B, gamma, V,
        _dev_ptr(out.tokens, "out_tokens", torch.int32),
        _dev_ptr(out.num_accepted, "out_num_accepted", torch.int32),
        _dev_ptr(out.flags, "out_flags", torch.int32),
        _checked(out.accept_hist, "out_accept_hist", torch.int32, (G1,)), handle)
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_greedy")
    return out


def spec_verify_commit(tokens, num_accepted, kv_len, slots=None, gamma_b=None, out=None,
                       stream=None, lib=None):
    """Chain KV-commit metadata of a verification round (see include/spec_verify.h).

    tokens [B, gamma+1] and num_accepted [B] from spec_verify_sample or
    spec_verify_greedy, kv_len [B] int32, slots [B, gamma+1] int32 or None,
    gamma_b [B] int32 proposals per request or None.
    Returns CommitOut(new_kv_len, anchor, n_free, free_slots); free_slots is
    None when slots is None. stream and lib as for spec_verify_sample.
    """
    torch = _torch()
    lib = lib or _lib.load()
    B, G1 = tokens.shape
    gamma = G1 - 1
    if tuple(num_accepted.shape) != (B,) or tuple(kv_len.shape) != (B,):
        raise ValueError("num_accepted and kv_len must be [B]")
    if slots is not None and tuple(slots.shape) != (B, G1):
        raise ValueError("slots must be [B, gamma+1]")
    dev = tokens.device
    handle, strm = _stream(stream)
    if out is None:
        with torch.cuda.stream(strm):
            out = CommitOut(torch.empty((B,), dtype=torch.int32, device=dev),
                            torch.empty((B,), dtype=torch.int32, device=dev),
                            torch.empty((B,), dtype=torch.int32, device=dev),
                            torch.empty((B, gamma), dtype=torch.int32, device=dev)
                            if slots is not None else None)
    rc = lib.spec_verify_commit(
        _dev_ptr(tokens, "tokens", torch.int32), _dev_ptr(num_accepted, "num_accepted", torch.int32),
        _dev_ptr(kv_len, "kv_len", torch.int32), _dev_ptr(slots, "slots", torch.int32),
        _checked(gamma_b, "gamma_b", torch.int32, (B,)), B, gamma,
        _checked(out.new_kv_len, "new_kv_len", torch.int32, (B,)),
        _checked(out.anchor, "anchor", torch.int32, (B,)),
        _checked(out.n_free, "n_free", torch.int32, (B,)),
        _checked(out.free_slots, "free_slots", torch.int32, (B, gamma)), handle)
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_commit")
    return out


def bench_profile_start(max_launches_per_kernel):
    """Starts per-kernel event timing in the benchmark build (_lib.load_bench());
    only calls made with lib=_lib.load_bench() are timed."""
    rc = _lib.load_bench().sv_bench_profile_start(int(max_launches_per_kernel))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "sv_bench_profile_start")


def bench_profile_stop():
    """Returns {kernel name: (total_ms, launches)} since bench_profile_start."""
    import ctypes
    ms = (ctypes.c_double * _lib.SV_NUM_KERNELS)()
    n = (ctypes.c_int32 * _lib.SV_NUM_KERNELS)()
    rc = _lib.load_bench().sv_bench_profile_stop(ctypes.cast(ms, ctypes.c_void_p),
                                                 ctypes.cast(n, ctypes.c_void_p))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "sv_bench_profile_stop")
    return {name: (ms[k], n[k]) for k, name in enumerate(_lib.KERNEL_NAMES)}
