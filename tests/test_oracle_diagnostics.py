"""Pins of the oracle's per-position diagnostics (oracle/diagnostics.py) to what
the pages and the mathematics fix: the worked examples' overlaps, the identity
with total variation, the acceptance rate of the walk itself, the closed form
of the expected block length and the sampled law of accepted lengths."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import diagnostics as od
from tests.conftest import GOLDEN
from tests.test_oracle_pins import _chisq_pvalue, _overlap_pair, _simulate


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_overlap_of_the_worked_examples():
    g = _golden("three_token_example.json")
    p, q = g["reconstructed"]["p"], g["reconstructed"]["q"]
    assert abs(od.overlap(p, q) - (1.0 - g["printed"]["rejection_probability"])) < 1e-12
    g8 = _golden("alpha08_example.json")
    for a in np.linspace(0.0, 0.8, 9):
        b = (1.0 - a) / 2.0
        pp, qq = np.array([a, b, b]), np.array([a + 0.2, b - 0.1, b - 0.1])
        assert abs(od.overlap(pp, qq) - g8["printed"]["alpha"]) < 1e-12


def test_overlap_is_one_minus_total_variation():
    rng = np.random.default_rng(11)
    for V in (2, 5, 40, 1000):
        for _ in range(20):
            p = rng.dirichlet(np.ones(V) * 0.3)
            q = rng.dirichlet(np.ones(V) * 0.3)
            tv = 0.5 * np.abs(p - q).sum()
            assert abs(od.overlap(p, q) - (1.0 - tv)) < 1e-12
            assert abs(od.overlap(p, q) - od.overlap(q, p)) < 1e-15
    p = rng.dirichlet(np.ones(10))
    assert abs(od.overlap(p, p) - 1.0) < 1e-12
    a = np.zeros(10)
    a[:5] = rng.dirichlet(np.ones(5))
    c = np.zeros(10)
    c[5:] = rng.dirichlet(np.ones(5))
    assert od.overlap(a, c) == 0.0


def test_overlap_is_the_acceptance_rate_of_the_walk():
    # one position: x ~ q, accepted by the oracle's own rule
    rng = np.random.default_rng(12)
    p = rng.dirichlet(np.ones(6))
    q = rng.dirichlet(np.ones(6))
    n = 20000
    _, nacc = _simulate([p, p], [q], n, seed=13)
    a = od.overlap(p, q)
    se = math.sqrt(a * (1 - a) / n)
    assert abs((nacc == 1).mean() - a) < 5 * se


def _transformed_fixture():
    """Two requests, gamma 4, V 12, with distinct rows, bans and different
    target and draft samplers."""
    rng = np.random.default_rng(14)
    B, gamma, V = 2, 4, 12
    target = rng.normal(0.0, 1.5, (B, gamma + 1, V))
    draft = target[:, :gamma] + rng.normal(0.0, 0.8, (B, gamma, V))
    banned = np.array([[3, -1, 7], [0, 11, -1]], dtype=np.int32)
    ts = oracle.Sampler(0.8, 0, 0.9)
    ds = oracle.Sampler(1.2, 6, 1.0)
    return target, draft, banned, ts, ds


def _rows(target, draft, banned, ts, ds, b):
    bans = [t for t in banned[b].tolist() if t >= 0]
    g = draft.shape[1]
    p = [oracle.row_distribution(target[b, i], ts, bans).p for i in range(g + 1)]
    q = [oracle.row_distribution(draft[b, i], ds, bans).p for i in range(g)]
    return p, q


def test_position_overlaps_are_conditional_acceptance():
    target, draft, banned, ts, ds = _transformed_fixture()
    alpha, margin = od.position_overlaps(target, draft, ts, ds, banned)
    assert alpha.shape == (2, 4) and np.all((alpha >= 0) & (alpha <= 1 + 1e-12))
    n = 12000
    est = {}
    for b in range(2):
        p, q = _rows(target, draft, banned, ts, ds, b)
        _, nacc = _simulate(p, q, n, seed=15 + b)
        for i in range(4):
            reached = nacc >= i
            r = int(reached.sum())
            if r >= 500:
                est[b, i] = ((nacc[reached] > i).mean(), r)

    def consistent(a):
        return all(abs(e - a[b, i]) < 5 * math.sqrt(max(a[b, i] * (1 - a[b, i]), 1e-4) / r)
                   for (b, i), (e, r) in est.items())

    assert len(est) >= 6
    assert consistent(alpha)
    # the same test has the power to tell the right rows apart: overlaps with the
    # samplers swapped, the bans dropped or the target rows shifted by one fail it
    swapped, _ = od.position_overlaps(target, draft, ds, ts, banned)
    unbanned, _ = od.position_overlaps(target, draft, ts, ds, None)
    shifted, _ = od.position_overlaps(np.concatenate([target[:, 1:], target[:, :1]], axis=1),
                                      draft, ts, ds, banned)
    for wrong in (swapped, unbanned, shifted):
        assert not consistent(wrong)


def test_histogram_and_conditional_acceptance_against_a_loop():
    rng = np.random.default_rng(16)
    gamma = 6
    nacc = rng.integers(0, gamma + 1, 500)
    h = od.accepted_prefix_histogram(nacc, gamma)
    assert h.sum() == 500
    for k in range(gamma + 1):
        assert h[k] == sum(1 for v in nacc if v == k)
    reached, accepted = od.conditional_acceptance(h)
    for i in range(gamma):
        assert reached[i] == sum(1 for v in nacc if v >= i)
        assert accepted[i] == sum(1 for v in nacc if v > i)


def test_prefix_length_law_closed_form():
    g = _golden("expected_tokens_per_step.json")["scenario_alpha_0.3_gamma_8"]
    law = od.prefix_length_law([g["alpha"]] * g["gamma"])
    assert abs(law.sum() - 1.0) < 1e-15
    expected_block = float(np.dot(np.arange(1, g["gamma"] + 2), law))
    assert abs(expected_block - g["closed_form"]) < 1e-8
    for a in (0.05, 0.6, 0.95):
        for gamma in (1, 4, 9):
            law = od.prefix_length_law([a] * gamma)
            e = float(np.dot(np.arange(1, gamma + 2), law))
            assert abs(e - (1 - a ** (gamma + 1)) / (1 - a)) < 1e-12


def _law_off_by_one(alphas):
    # planted mistake: P(n = k) uses c_k for the stopping position's survival
    gamma = len(alphas)
    law = np.zeros(gamma + 1)
    surv = 1.0
    for k in range(gamma):
        surv *= alphas[k]
        law[k] = surv * (1.0 - alphas[k])
    law[gamma] = 1.0 - law[:gamma].sum()
    return law


@pytest.mark.parametrize("law_fn,should_pass", [(od.prefix_length_law, True),
                                                (_law_off_by_one, False)])
def test_prefix_length_law_sampled(law_fn, should_pass):
    rng = np.random.default_rng(17)
    alphas = [0.9, 0.55, 0.75, 0.4, 0.8]
    pairs = [_overlap_pair(a, rng=rng) for a in alphas]
    for (pp, qq), a in zip(pairs, alphas):
        assert abs(od.overlap(pp, qq) - a) < 1e-12
    n = 15000
    _, nacc = _simulate([pp for pp, _ in pairs] + [pairs[0][0]], [qq for _, qq in pairs], n,
                        seed=18)
    h = od.accepted_prefix_histogram(nacc, len(alphas))
    pv = _chisq_pvalue(h, law_fn(alphas))
    assert (pv > 1e-4) == should_pass, pv
    if should_pass:
        reached, accepted = od.conditional_acceptance(h)
        for i, a in enumerate(alphas):
            se = math.sqrt(a * (1 - a) / reached[i])
            assert abs(accepted[i] / reached[i] - a) < 5 * se
