"""spec_verify_sample_noalloc (the entry point without a workspace argument,
whose workspace is the library's static per-GPU scratch array) against
spec_verify_sample with a caller workspace: identical outputs on two calls in a
row, the second one smaller, both called through the C interface with
preallocated outputs."""

import ctypes

import numpy as np
import pytest

from tests import parity_util as pu

pytestmark = pytest.mark.gpu


def _call(lib, noalloc, t, d, xs, bans, samp, seed, offset, outs, ws, stream):
    from lossless_draft_verification_sample_amd import _lib as L
    B, G1, V = t.shape
    gamma = G1 - 1
    s = L.SvSampler(*samp)
    args = [t.data_ptr(), d.data_ptr(), L.SV_BF16, xs.data_ptr(),
            None if bans is None else bans.data_ptr(), 0 if bans is None else bans.shape[1],
            B, gamma, V, s, s, None, seed, offset, None,
            outs["tokens"].data_ptr(), outs["n"].data_ptr(), outs["flags"].data_ptr(),
            outs["tlse"].data_ptr(), outs["dlse"].data_ptr(), outs["ov"].data_ptr(),
            outs["hist"].data_ptr()]
    if noalloc:
        return lib.spec_verify_sample_noalloc(*args, stream)
    return lib.spec_verify_sample(*args, ws.data_ptr(), ws.numel(), stream)


def _outs(torch, B, gamma, dev):
    return {"tokens": torch.full((B, gamma + 1), 7, dtype=torch.int32, device=dev),
            "n": torch.full((B,), 7, dtype=torch.int32, device=dev),
            "flags": torch.full((B,), 7, dtype=torch.int32, device=dev),
            "tlse": torch.zeros((B, gamma + 1), dtype=torch.float32, device=dev),
            "dlse": torch.zeros((B, gamma), dtype=torch.float32, device=dev),
            "ov": torch.zeros((B, gamma), dtype=torch.float64, device=dev),
            "hist": torch.full((gamma + 1,), 7, dtype=torch.int32, device=dev)}


def test_noalloc_matches_workspace_call_twice():
    import torch
    from lossless_draft_verification_sample_amd import _lib as L
    lib = L.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    cases = [dict(name="c5", B=24, seed=123),               # c5 shape, fewer requests
             dict(name="c5", B=3, gamma=4, V=5003, seed=124)]  # smaller second call
    samplers = [(0.8, 0, 0.9), (0.7, 40, 1.0)]
    for case, samp, (seed, offset) in zip(cases, samplers, [(3, 11), (5, 2)]):
        over = dict(case)
        wl = pu.make(over.pop("name"), **over)
        cfg = wl.cfg
        print(f"[noalloc] B={cfg.B} gamma={cfg.gamma} V={cfg.V} sampler={samp}", flush=True)
        t = pu.logits_tensor(wl.target, wl.target_bits, "bf16", dev)
        d = pu.logits_tensor(wl.draft, wl.draft_bits, "bf16", dev)
        xs = torch.from_numpy(pu.oracle_proposals(wl, samp)).to(dev)
        bans = torch.from_numpy(wl.banned).to(dev)
        need = lib.spec_verify_workspace_bytes(cfg.B, cfg.gamma, cfg.V)
        assert 0 < need <= L.SV_NOALLOC_SCRATCH_BYTES
        ws = torch.empty((need,), dtype=torch.uint8, device=dev)
        ref = _outs(torch, cfg.B, cfg.gamma, dev)
        got = _outs(torch, cfg.B, cfg.gamma, dev)
        assert _call(lib, False, t, d, xs, bans, samp, seed, offset, ref, ws, stream) == L.SV_OK
        assert _call(lib, True, t, d, xs, bans, samp, seed, offset, got, None, stream) == L.SV_OK
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), k
        n = got["n"].cpu().numpy()
        assert np.all((n >= 0) & (n <= cfg.gamma))
        assert int(got["hist"].sum()) == cfg.B


def test_noalloc_rejects_sizes_beyond_the_scratch():
    import torch
    from lossless_draft_verification_sample_amd import _lib as L
    lib = L.load()
    # B * nsub * 16 bytes of draw sums alone exceed 8 MiB here: rejected on the
    # host before anything touches the device
    fake = 4096
    s = L.SvSampler(1.0, 0, 1.0)
    rc = lib.spec_verify_sample_noalloc(fake, fake, L.SV_BF16, fake, None, 0, 8192, 8, 1 << 20,
                                        s, s, None, 0, 0, None, fake, fake, None, None, None,
                                        None, None, torch.cuda.current_stream().cuda_stream)
    assert rc == L.SV_ESCRATCH
    assert "scratch" in lib.spec_verify_strerror(rc).decode()


def test_noalloc_beyond_the_draw_lists():
    # B = 700, V = 64000: everything but the draw's kept-token lists fits the
    # scratch array, the lists do not, so the no-alloc call runs without them
    # (its selections reread their sub-chunks) while the workspace call uses
    # them; the outputs must agree. A smaller call follows, with lists again.
    import torch
    from lossless_draft_verification_sample_amd import _lib as L
    lib = L.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    gen = torch.Generator(device=dev)
    for k, (B, gamma, V) in enumerate([(700, 2, 64000), (40, 3, 64000)]):
        print(f"[noalloc] B={B} gamma={gamma} V={V} random bf16 logits", flush=True)
        gen.manual_seed(321 + k)
        t = (torch.randn((B, gamma + 1, V), generator=gen, device=dev) * 3).to(torch.bfloat16)
        d = (torch.randn((B, gamma, V), generator=gen, device=dev) * 3).to(torch.bfloat16)
        xs = torch.randint(0, V, (B, gamma), generator=gen, device=dev, dtype=torch.int32)
        bans = torch.randint(-2, V, (B, 16), generator=gen, device=dev, dtype=torch.int32)
        need = lib.spec_verify_workspace_bytes(B, gamma, V)
        assert (need > L.SV_NOALLOC_SCRATCH_BYTES) == (k == 0)
        ws = torch.empty((need,), dtype=torch.uint8, device=dev)
        samp = (0.8, 0, 0.9)
        ref = _outs(torch, B, gamma, dev)
        got = _outs(torch, B, gamma, dev)
        assert _call(lib, False, t, d, xs, bans, samp, 9, k, ref, ws, stream) == L.SV_OK
        assert _call(lib, True, t, d, xs, bans, samp, 9, k, got, None, stream) == L.SV_OK
        torch.cuda.synchronize()
        for key in ref:
            assert torch.equal(got[key], ref[key]), (B, key)
        n = got["n"].cpu().numpy()
        assert np.all((n >= 0) & (n <= gamma)) and np.any(n < gamma)
