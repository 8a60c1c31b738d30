"""Final-draw cases at the edges of the draw kernel's read modes.

At a rejection whose target row is truncated, each wave of the draw kernel
queues the kept tokens of its sub-chunks (2048 tokens each) in LDS and gathers
the draft logits only there; a sub-chunk keeping more tokens than the queue
holds (256 per wave) is evaluated in place; an untruncated target row streams
the draft row alongside. These tests put requests on both sides of those lines
in one batch, cut the vocabulary at sub-chunk edges, and start from a workspace
full of arbitrary bytes (the kernels must clear what they rely on). Same bar as
the other parity tests: tokens, accepted counts and flags bit-exact outside
the 1e-10 decision band, lse within 1e-5.
"""

import numpy as np
import pytest

from lossless_draft_verification_sample_amd import synth
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import lossless_draft_verification_sample_amd._lib as L
    L.load()


def _set_logits(wl, target, draft):
    if wl.cfg.dtype == "bf16":
        wl.target_bits = synth.f32_to_bf16_bits(target)
        wl.draft_bits = synth.f32_to_bf16_bits(draft)
        wl.target = synth.bf16_bits_to_f32(wl.target_bits)
        wl.draft = synth.bf16_bits_to_f32(wl.draft_bits)
    else:
        wl.target = target.astype(np.float32)
        wl.draft = draft.astype(np.float32)


def _check(wl, samp, where, seed=11, offset=4):
    cfg = wl.cfg
    xs = pu.oracle_proposals(wl, samp)
    got = pu.run_gpu_sample(wl, xs, tsamp=samp, dsamp=samp, seed=seed, offset=offset)
    u = pu.philox_uniforms(seed, offset, cfg.B, cfg.gamma)
    ref = pu.run_oracle_sample(wl, xs, u, range(cfg.B), tsamp=samp, dsamp=samp)
    assert pu.compare_sample(got, ref, range(cfg.B), where=where) <= 1, where
    return got, ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_batch_of_sparse_and_dense_draw_rows(dtype):
    # requests 0-3 keep about a thousand tokens under top-p 0.9 (queued
    # gathers); the rows of requests 4-7 are nearly flat, so top-p keeps most
    # of the vocabulary and every sub-chunk overflows the queue
    wl = pu.make("c5" if dtype == "bf16" else "c5f32", B=8, gamma=4, V=60013, seed=501)
    t, d = wl.target.copy(), wl.draft.copy()
    t[4:] *= np.float32(0.03)
    d[4:] *= np.float32(0.03)
    _set_logits(wl, t, d)
    for off in (0, 1, 2):
        _check(wl, (0.8, 0, 0.9), f"{dtype} offset {off}", offset=off)


@pytest.mark.parametrize("k", [1500, 4096, 9000])
def test_top_k_around_the_queue_capacity(k):
    # fp32 rows have no ties, so top-k keeps exactly k tokens, about
    # k * 2048 / 30011 per sub-chunk: below, near and above the 256 a wave
    # queues
    wl = pu.make("c5f32", B=3, gamma=3, V=30011, seed=502)
    _check(wl, (1.0, k, 1.0), f"top-k {k}")


@pytest.mark.parametrize("V", [2048, 4096, 4099])
def test_vocabulary_at_sub_chunk_edges(V):
    # whole sub-chunks, and one token into the next
    wl = pu.make("c5", B=6, gamma=5, V=V, seed=503)
    _check(wl, (1.0, 0, 1.0), f"V {V} untruncated")
    _check(wl, (0.9, 40, 0.95), f"V {V} truncated")


def test_workspace_with_arbitrary_contents():
    import torch
    import lossless_draft_verification_sample_amd as sv
    wl = pu.make("c5", B=16, gamma=4, V=20011, seed=505)
    cfg = wl.cfg
    samp = pu.sampler_of(cfg)
    xs = pu.oracle_proposals(wl, samp)
    dev = pu.torch_dev()
    t = pu.logits_tensor(wl.target, wl.target_bits, cfg.dtype, dev)
    d = pu.logits_tensor(wl.draft, wl.draft_bits, cfg.dtype, dev)
    toks = torch.from_numpy(xs).to(dev)
    bans = torch.from_numpy(wl.banned).to(dev)
    n = sv.spec_verify_workspace_bytes(cfg.B, cfg.gamma, cfg.V)
    g = torch.Generator().manual_seed(7)
    for fill in ("random", "ones", "random"):
        if fill == "random":
            junk = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g)
        else:
            junk = torch.full((n,), 0xFF, dtype=torch.uint8)
        ws = junk.to(dev)
        for off in (3, 4):
            out = sv.spec_verify_sample(t, d, toks, samp, samp, banned_ids=bans, seed=9,
                                        offset=off, workspace=ws, want_hist=True)
            torch.cuda.synchronize()
            got = {"tokens": out.tokens.cpu().numpy(), "num_accepted": out.num_accepted.cpu().numpy(),
                   "flags": out.flags.cpu().numpy().astype(np.uint32),
                   "target_lse": out.target_lse.cpu().numpy().astype(np.float64),
                   "draft_lse": out.draft_lse.cpu().numpy().astype(np.float64)}
            u = pu.philox_uniforms(9, off, cfg.B, cfg.gamma)
            ref = pu.run_oracle_sample(wl, xs, u, range(cfg.B))
            assert pu.compare_sample(got, ref, range(cfg.B), where=f"{fill} {off}") <= 1
            hist = out.accept_hist.cpu().numpy().astype(np.int64)
            assert np.array_equal(hist, np.bincount(got["num_accepted"], minlength=cfg.gamma + 1))
