"""The pooled oracle of the full-batch parity tests equals one oracle call
over the same batch (CPU only)."""

import numpy as np

import oracle
from lossless_draft_verification_sample_amd import synth
from tests.oracle_pool import OraclePool


def test_pool_equals_single_call():
    cfg = synth.config("c5", B=5, V=3001)
    wl = synth.make_workload(cfg)
    xs = np.random.default_rng(3).integers(0, cfg.V, (cfg.B, cfg.gamma)).astype(np.int32)
    samp = (cfg.temperature, cfg.top_k, cfg.top_p)
    s = oracle.Sampler(*samp)
    with OraclePool(wl.target, wl.draft, xs, wl.banned, samp, samp, workers=2) as pool:
        for off in (0, 1):
            u = np.array(oracle.uniforms(cfg.philox_seed, off, cfg.B, cfg.gamma))
            got = pool.verify(u)
            ref = oracle.verify_sample(wl.target.astype(np.float64), wl.draft.astype(np.float64),
                                       xs, u, s, s, wl.banned)
            for g, r in zip(got, (ref.tokens, ref.num_accepted, ref.flags, ref.margin,
                                  ref.target_lse, ref.draft_lse)):
                assert np.array_equal(g, r)
