"""HIP-graph capture of the verifier calls.

The library launches its kernels on the caller's stream and allocates, clears
or synchronizes nothing, so a call can be captured once and replayed. Each
replay must reproduce the eager call bit for bit (same inputs, same seed).
Between replays the test runs eager work of its own, synchronizes, and
overwrites the outputs, so that every replay is seen to write them again.
"""

import numpy as np
import pytest

import parity_util as pu

pytestmark = pytest.mark.gpu


def _graph_replays(call, outs, n=4):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    junk = torch.ones(1 << 20, device="cuda")
    got = []
    for k in range(n):
        for t in outs:
            t.fill_(-7)
        junk.mul_(1.0001)                        # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got.append([t.cpu().numpy().copy() for t in outs])
    return got


def test_sample_call_replays_in_a_graph():
    import torch
    import lossless_draft_verification_sample_amd as sv
    wl = pu.make("c5", B=4, V=20011)
    xs = pu.oracle_proposals(wl)
    cfg = wl.cfg
    dev = torch.device("cuda:0")
    t = pu.logits_tensor(wl.target, wl.target_bits, cfg.dtype, dev)
    d = pu.logits_tensor(wl.draft, wl.draft_bits, cfg.dtype, dev)
    toks = torch.from_numpy(xs).to(dev)
    bans = torch.from_numpy(wl.banned).to(dev)
    samp = pu.sampler_of(cfg)
    ws = torch.empty(sv.spec_verify_workspace_bytes(cfg.B, cfg.gamma, cfg.V),
                     dtype=torch.uint8, device=dev)

    def new_out():
        return sv.SampleOut(torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=dev),
                            torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                            torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                            torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.float32, device=dev),
                            torch.empty((cfg.B, cfg.gamma), dtype=torch.float32, device=dev),
                            None, torch.empty((cfg.gamma + 1,), dtype=torch.int32, device=dev))

    ref = new_out()
    sv.spec_verify_sample(t, d, toks, samp, samp, banned_ids=bans, seed=5, offset=3,
                          workspace=ws, out=ref)
    torch.cuda.synchronize()
    out = new_out()

    def call():
        sv.spec_verify_sample(t, d, toks, samp, samp, banned_ids=bans, seed=5, offset=3,
                              workspace=ws, out=out)

    fields = [out.tokens, out.num_accepted, out.flags, out.target_lse, out.draft_lse,
              out.accept_hist]
    expect = [x.cpu().numpy() for x in (ref.tokens, ref.num_accepted, ref.flags, ref.target_lse,
                                        ref.draft_lse, ref.accept_hist)]
    for k, replay in enumerate(_graph_replays(call, fields)):
        for a, b in zip(replay, expect):
            assert np.array_equal(a, b), f"replay {k}"


def test_greedy_call_replays_in_a_graph():
    import torch
    import lossless_draft_verification_sample_amd as sv
    wl = pu.make("c4", B=8, V=30011)
    cfg = wl.cfg
    dev = torch.device("cuda:0")
    t = pu.logits_tensor(wl.target, wl.target_bits, cfg.dtype, dev)
    am = np.argmax(wl.target[:, : cfg.gamma], axis=2)
    xs = np.where(wl.match_coin < 0.7, am, wl.random_tokens).astype(np.int32)
    toks = torch.from_numpy(xs).to(dev)

    def new_out():
        return sv.GreedyOut(torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=dev),
                            torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                            torch.empty((cfg.B,), dtype=torch.int32, device=dev),
                            torch.empty((cfg.gamma + 1,), dtype=torch.int32, device=dev))

    ref = new_out()
    sv.spec_verify_greedy(t, toks, out=ref)
    torch.cuda.synchronize()
    out = new_out()

    def call():
        sv.spec_verify_greedy(t, toks, out=out)

    fields = [out.tokens, out.num_accepted, out.flags, out.accept_hist]
    expect = [x.cpu().numpy() for x in (ref.tokens, ref.num_accepted, ref.flags, ref.accept_hist)]
    for k, replay in enumerate(_graph_replays(call, fields)):
        for a, b in zip(replay, expect):
            assert np.array_equal(a, b), f"replay {k}"
