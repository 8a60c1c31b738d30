"""Whole-batch parity at full size: every request of the c2, c3a, c3b, c5 and
c5f32 (c5 with float32 logits) workloads, at several Philox offsets, against
the float64 oracle.

"Speculative Decoding - Turn guesses into parallel work", section
"Implementation roadmap and tests", asks for more than a few matching outputs.
Here the HIP path verifies the whole batch with device Philox uniforms at
(seed, offset) for each offset; the oracle verifies the same batch with the
same uniforms (its requests split over host processes, tests/oracle_pool.py).
Tokens, accepted counts and flags must be identical for every request whose
decisions all lie more than 1e-10 from their edge, and every row's
log-normaliser must agree within 1e-5. Requests excluded by the 1e-10 band
must stay below 1e-4 of the decisions taken; the count of requests with a
decision within the wider 1e-6 band is printed for reference.
"""

import time

import numpy as np
import pytest

from tests import parity_util as pu
from tests.oracle_pool import OraclePool

pytestmark = pytest.mark.gpu

OFFSETS = {"c2": (0, 1, 2, 3, 4, 5, 6, 7), "c3a": (0, 1, 2), "c3b": (0, 1, 2), "c5": (0, 1, 2),
           "c5f32": (0, 1)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import lossless_draft_verification_sample_amd._lib as L
    L.load()


@pytest.mark.parametrize("name", sorted(OFFSETS))
def test_full_batch_every_request(name):
    import torch
    import lossless_draft_verification_sample_amd as sv
    t0 = time.perf_counter()
    wl = pu.make(name)
    cfg = wl.cfg
    xs = pu.stored_proposals(name)
    dev = torch.device("cuda:0")
    t = pu.logits_tensor(wl.target, wl.target_bits, cfg.dtype, dev)
    d = pu.logits_tensor(wl.draft, wl.draft_bits, cfg.dtype, dev)
    toks = torch.from_numpy(xs).to(dev)
    bans = None if wl.banned is None else torch.from_numpy(wl.banned).to(dev)
    samp = pu.sampler_of(cfg)
    tot = dict(requests=0, decisions=0, excluded=0, within_1e6=0)
    with OraclePool(wl.target, wl.draft, xs, wl.banned, samp, samp) as pool:
        for off in OFFSETS[name]:
            out = sv.spec_verify_sample(t, d, toks, samp, samp, banned_ids=bans,
                                        seed=cfg.philox_seed, offset=off)
            u = pu.philox_uniforms(cfg.philox_seed, off, cfg.B, cfg.gamma)
            rt, rn, rf, rm, rtl, rdl = pool.verify(u)
            torch.cuda.synchronize()
            gt = out.tokens.cpu().numpy()
            gn = out.num_accepted.cpu().numpy()
            gf = out.flags.cpu().numpy().astype(np.uint32)
            keep = rm > pu.EXACT_BAND
            same = (gt == rt).all(axis=1) & (gn == rn) & (gf == rf.astype(np.uint32))
            bad = np.flatnonzero(~same & keep)
            assert bad.size == 0, (name, off, bad[:8].tolist(), gt[bad[:2]], rt[bad[:2]])
            for key, g, r in (("target_lse", out.target_lse, rtl), ("draft_lse", out.draft_lse, rdl)):
                g = g.cpu().numpy().astype(np.float64)
                fin = np.isfinite(r)
                assert np.array_equal(np.isfinite(g), fin), (name, off, key)
                err = np.abs(g[fin] - r[fin]) / np.maximum(1.0, np.abs(r[fin]))
                assert err.max() <= 1e-5, (name, off, key, float(err.max()))
            tot["requests"] += cfg.B
            # acceptance tests taken, plus one final draw per request
            tot["decisions"] += int(np.minimum(rn + 1, cfg.gamma).sum() + cfg.B)
            tot["excluded"] += int((~keep).sum())
            tot["within_1e6"] += int((rm <= pu.STATED_BAND).sum())
    # nearly every decision is compared bit-exactly
    assert tot["excluded"] <= max(1, tot["decisions"] // 10000), tot
    print(f"[full-batch] {name}: {tot} in {time.perf_counter() - t0:.1f} s", flush=True)
