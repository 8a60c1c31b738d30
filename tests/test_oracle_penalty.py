"""Pins of the oracle's repetition penalty (oracle.repetition_penalty,
oracle.round_to_bf16, and the penalty inside row_distribution / verify_batch).

The pages require the penalty to be part of p and q but fix no formula; the
oracle takes the multiplicative penalty of Keskar et al. 2019 in its
sign-aware form. What is pinned: bf16 rounding against torch's independent
conversion, the penalty's algebra, the emitted-token law under penalties, and
that row i penalizes the proposals that precede position i."""

import math

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import _chisq_pvalue


def test_round_to_bf16_matches_torch():
    import torch
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    bits[:2000] = (bits[:2000] & 0xFFFF0000) | 0x8000        # exact ties
    bits[2000:2100] = (bits[2000:2100] & 0xFFFF0000) | 0x7FFF
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([oracle.round_to_bf16(v) for v in vals], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_penalty_algebra():
    rng = np.random.default_rng(2)
    for _ in range(3000):
        z = float(np.float32(rng.normal(0, 6)))
        theta = float(np.float32(1.0 + rng.exponential(0.5)))
        for dtype in ("f32", "bf16"):
            zz = oracle.round_to_bf16(z) if dtype == "bf16" else z
            v = oracle.repetition_penalty(zz, theta, dtype)
            assert v <= zz                                   # never raises a logit
            assert (v > 0) == (zz > 0) or v == 0.0           # keeps the sign
            if dtype == "bf16":
                assert oracle.round_to_bf16(v) == v          # a bf16 value
            if zz > 0:
                assert abs(v * theta - zz) <= abs(zz) * (2**-7 if dtype == "bf16" else 2**-22)
            else:
                assert abs(v / theta - zz) <= abs(zz) * (2**-7 if dtype == "bf16" else 2**-22)
        assert oracle.repetition_penalty(z, 1.0, "f32") == z
    assert oracle.repetition_penalty(0.0, 2.0, "f32") == 0.0


def test_penalized_row_distribution():
    rng = np.random.default_rng(3)
    V = 30
    z = rng.normal(0, 2, V)
    s = oracle.Sampler(0.7)
    pen = [3, 3, 7, 40, -1]                     # a duplicate, an out-of-range id
    theta = 1.8
    d = oracle.row_distribution(z, s, (), pen, theta, "f32")
    zz = z.copy()
    for t in (3, 7):
        zz[t] = oracle.repetition_penalty(z[t], theta, "f32")
    # probability ratios follow the penalized logits
    T = float(np.float32(s.temperature))        # samplers carry float32 settings
    for x in range(V):
        assert math.isclose(d.p[x] / d.p[0], math.exp((zz[x] - zz[0]) / T), rel_tol=1e-12)
    # banned wins over penalized
    d2 = oracle.row_distribution(z, s, (3,), pen, theta, "f32")
    assert d2.p[3] == 0.0


def test_emitted_token_follows_the_penalized_law():
    rng = np.random.default_rng(4)
    V = 6
    zt = rng.normal(0, 1.5, V)
    zd = zt + rng.normal(0, 0.7, V)
    hist = np.array([[1, 4, -1]])
    theta_t, theta_d = 1.7, 1.3
    ts = oracle.Sampler(0.9)
    p = oracle.row_distribution(zt, ts, (), [1, 4], theta_t, "f32").p
    q = oracle.row_distribution(zd, ts, (), [1, 4], theta_d, "f32").p
    counts = np.zeros(V)
    target = np.stack([zt, zt])[None]
    draft = zd[None, None]
    for _ in range(8000):
        x = oracle.sample_categorical(q, 1.0 - rng.random())[0]
        r = oracle.verify_batch(target, draft, np.array([[x]]), 1.0 - rng.random((1, 2)), [ts], [ts],
                                history=hist, penalties=[theta_t], penalties_draft=[theta_d])
        counts[r.tokens[0, 0]] += 1
    assert _chisq_pvalue(counts, p) > 1e-4
    p_raw = oracle.row_distribution(zt, ts).p
    assert _chisq_pvalue(counts, p_raw) < 1e-4              # the test tells the two apart


@pytest.mark.parametrize("with_penalty", [True, False])
def test_row_one_penalizes_the_first_proposal(with_penalty):
    # both proposals are token 0; row 1 must penalize token 0 because x_0 = 0
    # precedes position 1. The acceptance rate at position 1 then equals
    # min(1, p1(0) / q1(0)) with penalized rows.
    V = 4
    z0 = np.array([2.0, 0.0, 0.0, 0.0])
    z1 = np.array([2.13, 2.53, -0.43, 2.36])    # acceptance 0.37 penalized, 0.59 not
    d0 = np.array([2.0, 0.0, 0.0, 0.0])
    d1 = np.array([1.65, -1.1, 0.37, 1.55])
    target = np.stack([z0, z1, z1])[None]
    draft = np.stack([d0, d1])[None]
    s = oracle.Sampler(1.0)
    theta = 3.0
    rng = np.random.default_rng(5)
    n = 12000
    reached = accepted = 0
    for _ in range(n):
        u = 1.0 - rng.random((1, 3))
        r = oracle.verify_batch(target, draft, np.array([[0, 0]]), u, [s], [s],
                                history=np.array([[-1]]), penalties=[theta], penalties_draft=[theta])
        if r.num_accepted[0] >= 1:
            reached += 1
            accepted += r.num_accepted[0] >= 2
    p1 = oracle.row_distribution(z1, s, (), [0] if with_penalty else [], theta).p
    q1 = oracle.row_distribution(d1, s, (), [0] if with_penalty else [], theta).p
    a = min(1.0, p1[0] / q1[0])
    assert 0.2 < a < 0.8 and reached > n // 2
    se = math.sqrt(a * (1 - a) / reached)
    consistent = abs(accepted / reached - a) < 5 * se
    assert consistent == with_penalty
