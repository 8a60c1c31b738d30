"""Pins of the float64 oracle to things other than itself.

Each test checks the oracle against what the pages print (fixtures under
tests/golden with their citation), a closed form, an independent library
implementation, or brute force on tiny inputs. test_mutants_are_caught plants
plausible mistakes in the oracle (on the CPU) and checks that a pin fails.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import verifier as ov
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _logits_of(p):
    """Logits whose T=1 softmax is p (zero-probability tokens become -inf)."""
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p)


def _draw(q, u):
    x, _, _ = oracle.sample_categorical(q, u)
    return x


def _simulate(p_rows, q_rows, n_trials, seed):
    """Run the oracle's per-request walk n_trials times with fresh proposals
    drawn from q and fresh uniforms. Returns tokens [n, gamma+1] and n_acc."""
    rng = np.random.default_rng(seed)
    gamma = len(q_rows)
    toks = np.empty((n_trials, gamma + 1), dtype=np.int64)
    nacc = np.empty(n_trials, dtype=np.int64)
    for t in range(n_trials):
        prop_u = 1.0 - rng.random(gamma)
        xs = [_draw(q_rows[i], prop_u[i]) for i in range(gamma)]
        u = 1.0 - rng.random(gamma + 1)
        out, n, _, _, _ = oracle.verify_block(p_rows, q_rows, xs, u)
        toks[t] = out
        nacc[t] = n
    return toks, nacc


def _chisq_pvalue(counts, probs):
    counts = np.asarray(counts, dtype=np.float64)
    probs = np.asarray(probs, dtype=np.float64)
    support = probs > 0
    assert counts[~support].sum() == 0, "a zero-probability token was emitted"
    exp = probs[support] / probs[support].sum() * counts[support].sum()
    return stats.chisquare(counts[support], exp).pvalue


# ---------------------------------------------------------------- Philox

def _numpy_philox_block(counter, key):
    """NumPy's Philox bit generator increments its 256-bit counter before each
    block, so seeding it with counter - 1 yields the block of `counter`."""
    c = sum(int(v) << (64 * i) for i, v in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = [(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)]
    bg = np.random.Philox(counter=np.array(words, dtype=np.uint64),
                          key=np.array([int(k) for k in key], dtype=np.uint64))
    return [int(v) for v in bg.random_raw(4)]


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 2, 3, 4), (5, 6)),
    ((0, 7, 0, 0), (0, 0)),
    ((2**64 - 1, 2**64 - 1, 2**64 - 1, 2**64 - 1), (2**64 - 1, 2**64 - 1)),
    ((8, 127, 12345, 0), (0xDEADBEEFCAFEF00D, 0)),
])
def test_philox_matches_numpy(counter, key):
    assert list(oracle.philox4x64_10(counter, key)) == _numpy_philox_block(counter, key)


def test_philox_uniform_layout_matches_numpy():
    rng = np.random.default_rng(7)
    for _ in range(50):
        seed = int(rng.integers(0, 2**63))
        offset = int(rng.integers(0, 2**40))
        b = int(rng.integers(0, 4096))
        j = int(rng.integers(0, 17))
        r = _numpy_philox_block((j, b, offset, 0), (seed, 0))[0]
        assert oracle.uniform(seed, offset, b, j) == ((r >> 11) + 1) / 2.0**53


def test_uniform_range_edges():
    assert oracle.word_to_uniform(0) == 2.0**-53
    assert oracle.word_to_uniform(2**64 - 1) == 1.0
    us = np.array(oracle.uniforms(0, 0, 64, 8))
    assert us.shape == (64, 9) and np.all(us > 0) and np.all(us <= 1)


# ---------------------------------------------------------------- worked examples

def test_three_token_example_analytic():
    g = _golden("three_token_example.json")
    p = np.array(g["reconstructed"]["p"])
    q = np.array(g["reconstructed"]["q"])
    pr = g["printed"]
    # the oracle's transform returns p and q from their logits
    dp = oracle.row_distribution(_logits_of(p), oracle.Sampler())
    dq = oracle.row_distribution(_logits_of(q), oracle.Sampler())
    np.testing.assert_allclose(dp.p, p, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dq.p, q, rtol=0, atol=1e-15)
    law, alpha, residual = oracle.first_token_law(dp.p, dq.p)
    assert abs((1 - alpha) - pr["rejection_probability"]) < 1e-12
    np.testing.assert_allclose(oracle.residual_weights(dp.p, dq.p),
                               pr["positive_part_p_minus_q"], atol=1e-12)
    np.testing.assert_allclose(residual, pr["replacement_probabilities"], atol=1e-12)
    assert abs(np.minimum(p, q)[1] - pr["final_B_accept_part"]) < 1e-12
    assert abs(law[1] - pr["final_B"]) < 1e-12
    assert abs(law[2] - pr["final_C"]) < 1e-12
    np.testing.assert_allclose(law, p, atol=1e-12)


def test_three_token_example_sampled():
    g = _golden("three_token_example.json")
    p = np.array(g["reconstructed"]["p"])
    q = np.array(g["reconstructed"]["q"])
    n = 30000
    toks, nacc = _simulate([p, p], [q], n, seed=11)
    rejected = nacc == 0
    # rejection frequency 0.40 within 5 standard errors
    se = math.sqrt(0.4 * 0.6 / n)
    assert abs(rejected.mean() - 0.40) < 5 * se
    # replacement law among rejections: 0.75 / 0.25 / 0
    rep = np.bincount(toks[rejected, 0], minlength=3)
    assert rep[2] == 0
    assert _chisq_pvalue(rep, [0.75, 0.25, 0.0]) > 1e-4
    # the emitted first token follows p
    assert _chisq_pvalue(np.bincount(toks[:, 0], minlength=3), p) > 1e-4


def _alpha08_member(a):
    """(cat, dog, bear) with p = (a, b, b), q = (a + 0.2, b - 0.1, b - 0.1)."""
    b = (1.0 - a) / 2.0
    return np.array([a, b, b]), np.array([a + 0.2, b - 0.1, b - 0.1])


def test_alpha08_family_invariants():
    g = _golden("alpha08_example.json")["printed"]
    canon_p, canon_q = _alpha08_member(0.6)
    np.testing.assert_allclose(canon_p, [0.6, 0.2, 0.2])
    np.testing.assert_allclose(canon_q, [0.8, 0.1, 0.1])
    for a in np.linspace(0.0, 0.8, 9):
        p, q = _alpha08_member(a)
        law, alpha, residual = oracle.first_token_law(p, q)
        assert abs(alpha - g["alpha"]) < 1e-12
        assert abs((1 - alpha) - g["rejection_probability"]) < 1e-12
        np.testing.assert_allclose(residual, [0.0, g["residual"]["dog"], g["residual"]["bear"]],
                                   atol=1e-12)
        np.testing.assert_allclose(law, p, atol=1e-12)


def test_alpha08_sampled_and_negative_control(monkeypatch):
    p, q = _alpha08_member(0.6)
    n = 20000
    toks, nacc = _simulate([p, p], [q], n, seed=5)
    assert _chisq_pvalue(np.bincount(toks[:, 0], minlength=3), p) > 1e-4
    # planted mistake: after a rejection draw from p itself (the double count
    # the page warns about); the same test must now fail
    monkeypatch.setattr(ov, "residual_weights", lambda pp, qq: np.asarray(pp, dtype=np.float64))
    toks_bad, _ = _simulate([p, p], [q], n, seed=5)
    assert _chisq_pvalue(np.bincount(toks_bad[:, 0], minlength=3), p) < 1e-6


# ---------------------------------------------------------------- closed forms

def _overlap_pair(alpha, V=8, rng=None):
    """p = alpha * q + (1 - alpha) * r with r on a support disjoint from q's,
    so sum(min(p, q)) = alpha exactly."""
    rng = rng or np.random.default_rng(0)
    q = np.zeros(V)
    r = np.zeros(V)
    q[: V // 2] = rng.dirichlet(np.ones(V // 2))
    r[V // 2:] = rng.dirichlet(np.ones(V - V // 2))
    return alpha * q + (1 - alpha) * r, q


@pytest.mark.parametrize("alpha", [0.3, 0.6, 0.8, 0.95])
@pytest.mark.parametrize("gamma", [1, 4, 8])
def test_expected_tokens_closed_form(alpha, gamma):
    rng = np.random.default_rng(int(alpha * 100) + gamma)
    pairs = [_overlap_pair(alpha, rng=rng) for _ in range(gamma)]
    p_rows = [pp for pp, _ in pairs] + [pairs[0][0]]
    q_rows = [qq for _, qq in pairs]
    for pp, qq in pairs:
        assert abs(oracle.first_token_law(pp, qq)[1] - alpha) < 1e-12
    n = 12000
    _, nacc = _simulate(p_rows, q_rows, n, seed=gamma * 1000 + int(alpha * 100))
    emitted = nacc + 1
    expected = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    se = emitted.std(ddof=1) / math.sqrt(n)
    assert abs(emitted.mean() - expected) < 5 * se + 1e-9


def test_fundamentals_scenario_gamma8_alpha03():
    g = _golden("expected_tokens_per_step.json")["scenario_alpha_0.3_gamma_8"]
    expected = (1 - 0.3 ** 9) / 0.7
    assert abs(expected - g["closed_form"]) < 1e-12
    assert 1.0 < expected < 2.0                # "keeps one or two"
    rng = np.random.default_rng(3)
    pairs = [_overlap_pair(0.3, rng=rng) for _ in range(8)]
    _, nacc = _simulate([pp for pp, _ in pairs] + [pairs[0][0]], [qq for _, qq in pairs],
                        12000, seed=99)
    emitted = nacc + 1
    assert abs(emitted.mean() - expected) < 5 * emitted.std(ddof=1) / math.sqrt(12000)


def test_survival_form_position_varying():
    rng = np.random.default_rng(21)
    alphas = [0.9, 0.7, 0.5, 0.85, 0.6]
    pairs = [_overlap_pair(a, rng=rng) for a in alphas]
    p_rows = [pp for pp, _ in pairs] + [pairs[0][0]]
    q_rows = [qq for _, qq in pairs]
    n = 15000
    _, nacc = _simulate(p_rows, q_rows, n, seed=77)
    expected = 1.0 + sum(np.prod(alphas[:j]) for j in range(1, len(alphas) + 1))
    emitted = nacc + 1
    assert abs(emitted.mean() - expected) < 5 * emitted.std(ddof=1) / math.sqrt(n)
    # per-position conditional acceptance c_i
    for i, a in enumerate(alphas):
        reached = nacc >= i
        acc = nacc[reached] > i
        se = math.sqrt(a * (1 - a) / reached.sum())
        assert abs(acc.mean() - a) < 5 * se


# ---------------------------------------------------------------- chi-square on tiny vocabularies

@pytest.mark.parametrize("V", [2, 3, 8, 16])
def test_emitted_tokens_follow_p(V):
    rng = np.random.default_rng(V)
    gamma = 3
    p_rows, q_rows = [], []
    for i in range(gamma + 1):
        pp = rng.dirichlet(np.ones(V))
        if V > 2:
            pp[rng.integers(V)] = 0.0          # a token the target never emits
            pp /= pp.sum()
        p_rows.append(pp)
    for i in range(gamma):
        qq = rng.dirichlet(np.ones(V))
        zero = int(np.argmax(p_rows[i]))       # q(x) = 0 where p(x) is largest
        qq[zero] = 0.0
        qq /= qq.sum()
        q_rows.append(qq)
    n = 20000
    toks, nacc = _simulate(p_rows, q_rows, n, seed=1000 + V)
    for i in range(gamma + 1):
        reached = nacc >= i
        counts = np.bincount(toks[reached, i], minlength=V)
        assert _chisq_pvalue(counts, p_rows[i]) > 1e-4, f"position {i}"
        if i < gamma:
            # q(x) = 0 but p(x) > 0: still emitted, only through the residual
            assert counts[int(np.argmax(p_rows[i]))] > 0


# ---------------------------------------------------------------- transforms by brute force

def _brute_kept(z, banned, T, k, P):
    """Threshold search straight from the definitions, over present values:
    top-k keeps z >= the largest t with #{z >= t} >= k; top-p keeps z >= the
    largest t whose upper set {z >= t} carries tempered mass >= P."""
    V = len(z)
    K = [i for i in range(V) if math.isfinite(z[i]) and i not in banned]
    if k > 0 and k < len(K):
        cand = sorted({z[i] for i in K}, reverse=True)
        t = next(t for t in cand if sum(1 for i in K if z[i] >= t) >= k)
        K = [i for i in K if z[i] >= t]
    if P < 1.0 and K:
        m = max(z[i] / T for i in K)
        Zk = math.fsum(math.exp(z[i] / T - m) for i in K)
        cand = sorted({z[i] for i in K}, reverse=True)
        t = next((t for t in cand
                  if math.fsum(math.exp(z[i] / T - m) for i in K if z[i] >= t) / Zk >= P),
                 cand[-1])
        K = [i for i in K if z[i] >= t]
    return sorted(K)


def test_transforms_match_brute_force():
    rng = np.random.default_rng(123)
    for trial in range(300):
        V = int(rng.integers(1, 40))
        levels = rng.normal(0, 2, size=int(rng.integers(1, 8)))
        z = rng.choice(levels, size=V)             # many exact ties
        z = np.where(rng.random(V) < 0.1, -np.inf, z)
        banned = set(rng.choice(V, int(rng.integers(0, max(1, V // 4) + 1))).tolist())
        T = float(np.float32(rng.uniform(0.3, 2.0)))
        k = int(rng.integers(0, V + 2))
        P = float(np.float32(rng.choice([1.0, rng.uniform(0.05, 0.999)])))
        d = oracle.row_distribution(z, oracle.Sampler(T, k, P), banned)
        want = _brute_kept(list(z), banned, T, k, P)
        assert sorted(np.flatnonzero(d.kept).tolist()) == want, (trial, z, banned, T, k, P)
        if want:
            m = max(z[i] / T for i in want)
            lse = m + math.log(math.fsum(math.exp(z[i] / T - m) for i in want))
            assert abs(d.lse - lse) < 1e-12
            np.testing.assert_allclose(d.p[want], np.exp(z[want] / T - lse), rtol=1e-12)
            assert abs(math.fsum(d.p) - 1.0) < 1e-12
        else:
            assert d.empty and d.lse == -math.inf


def test_top_k_one_equals_argmax_and_sampling_equals_greedy():
    rng = np.random.default_rng(9)
    B, gamma, V = 40, 4, 50
    target = rng.normal(0, 2, (B, gamma + 1, V))       # continuous: no ties
    draft = target[:, :gamma] + rng.normal(0, 1.5, (B, gamma, V))
    s1 = oracle.Sampler(0.8, 1, 1.0)
    xs = np.argmax(draft, axis=2)
    u = 1.0 - rng.random((B, gamma + 1))
    res = oracle.verify_sample(target, draft, xs, u, s1, s1)
    g = oracle.verify_greedy(target, xs)
    np.testing.assert_array_equal(res.tokens, g.tokens)
    np.testing.assert_array_equal(res.num_accepted, g.num_accepted)
    for b in range(B):
        d = oracle.row_distribution(target[b, 0], s1)
        assert np.flatnonzero(d.kept).tolist() == [int(np.argmax(target[b, 0]))]


def test_p_equals_q_never_rejects():
    rng = np.random.default_rng(4)
    B, gamma, V = 30, 6, 64
    target = rng.normal(0, 3, (B, gamma + 1, V))
    draft = target[:, :gamma].copy()
    s = oracle.Sampler(0.9, 20, 0.95)
    xs = np.zeros((B, gamma), dtype=np.int64)
    for b in range(B):
        for i in range(gamma):
            xs[b, i] = _draw(oracle.row_distribution(draft[b, i], s).p, 1.0 - rng.random())
    res = oracle.verify_sample(target, draft, xs, 1.0 - rng.random((B, gamma + 1)), s, s)
    assert np.all(res.num_accepted == gamma)
    assert np.all(res.tokens >= 0)


def test_banned_tokens_never_emitted():
    rng = np.random.default_rng(8)
    B, gamma, V = 200, 3, 12
    target = rng.normal(0, 1, (B, gamma + 1, V))
    draft = rng.normal(0, 1, (B, gamma, V))
    banned = np.stack([rng.choice(V, 4, replace=False) for _ in range(B)])
    s = oracle.Sampler(1.0)
    xs = rng.integers(0, V, (B, gamma))                  # includes banned proposals
    res = oracle.verify_sample(target, draft, xs, 1.0 - rng.random((B, gamma + 1)), s, s, banned)
    for b in range(B):
        emitted = res.tokens[b, : res.num_accepted[b] + 1]
        assert not set(emitted.tolist()) & set(banned[b].tolist())
        if set(xs[b, : res.num_accepted[b] + 1].tolist()) & set(banned[b].tolist()):
            assert res.flags[b] & oracle.FLAG_Q_ZERO


def test_greedy_brute_force_ties_and_signed_zero():
    rng = np.random.default_rng(31)
    for trial in range(200):
        B, gamma, V = 3, int(rng.integers(1, 6)), int(rng.integers(1, 30))
        target = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 2.0, -np.inf]),
                            size=(B, gamma + 1, V))
        xs = rng.integers(-1, V + 1, (B, gamma))
        g = oracle.verify_greedy(target, xs)
        for b in range(B):
            am = [max(range(V), key=lambda i: (target[b, r, i], -i)) for r in range(gamma + 1)]
            n = gamma
            for i in range(gamma):
                if xs[b, i] != am[i]:
                    n = i
                    break
            assert g.num_accepted[b] == n
            assert g.tokens[b, :n].tolist() == xs[b, :n].tolist()
            assert g.tokens[b, n] == am[n]
            assert np.all(g.tokens[b, n + 1:] == -1)
            assert bool(g.flags[b] & 1) == bool(np.any((xs[b] < 0) | (xs[b] >= V)))


def test_greedy_out_of_range_proposal_never_matches():
    """A proposal outside [0, V) is not a token: greedy verification rejects it
    even where the row has no admissible id (its argmax is then -1, and the
    -1 of a padding proposal must not count as a match). Checked for
    verify_greedy and for the greedy requests of verify_batch."""
    V, gamma = 6, 2
    nan_row = np.full(V, np.nan)
    target = np.zeros((2, gamma + 1, V))
    target[0, 0] = nan_row                       # request 0: row 0 has no admissible id
    target[1, 0] = nan_row
    target[1, 0, 3] = 1.0                        # request 1: only id 3 is a number
    banned = np.array([[-1, -1], [3, -1]])       # ... but 3 is banned: no admissible id
    xs = np.array([[-1, 2], [-1, 0]], dtype=np.int32)
    g = oracle.verify_greedy(target, xs, banned)
    for b in range(2):
        assert g.argmax[b, 0] == -1
        assert g.num_accepted[b] == 0
        assert g.tokens[b].tolist() == [-1, -1, -1]
        assert g.flags[b] & oracle.FLAG_TOKEN_RANGE and g.flags[b] & oracle.FLAG_EMPTY
    assert g.flags[0] & oracle.FLAG_NONFINITE
    greedy = [oracle.Sampler(0.0, 0, 1.0)] * 2
    mb = oracle.verify_batch(target, np.zeros((2, gamma, V)), xs, np.full((2, gamma + 1), 0.5),
                             greedy, greedy, banned)
    assert mb.num_accepted.tolist() == [0, 0]
    assert mb.tokens.tolist() == g.tokens.tolist()
    assert mb.flags.tolist() == g.flags.tolist()


def test_flags_and_edge_cases():
    V, gamma = 10, 2
    z = np.zeros((1, gamma + 1, V))
    d = np.zeros((1, gamma, V))
    s = oracle.Sampler()
    u = np.full((1, gamma + 1), 0.5)
    # out-of-range proposal: rejected at position 0, flag 1
    r = oracle.verify_sample(z, d, np.array([[V, 0]]), u, s, s)
    assert r.num_accepted[0] == 0 and r.flags[0] & oracle.FLAG_TOKEN_RANGE
    # NaN in a row read: flag 4
    z2 = z.copy()
    z2[0, 1, 3] = np.nan
    assert oracle.verify_sample(z2, d, np.array([[0, 0]]), u, s, s).flags[0] & oracle.FLAG_NONFINITE
    # every token banned: empty support, flag 8, no token can be drawn
    r = oracle.verify_sample(z, d, np.array([[0, 0]]), u, s, s, banned=np.arange(V)[None])
    assert r.flags[0] & oracle.FLAG_EMPTY and r.tokens[0, 0] == -1
    # draft row fully masked: proposal has q = 0 -> flag 2, residual equals p
    d3 = d.copy()
    d3[0, 0, :] = -np.inf
    r = oracle.verify_sample(z, d3, np.array([[4, 0]]), u, s, s)
    assert r.flags[0] & oracle.FLAG_Q_ZERO and r.num_accepted[0] == 0
    assert r.tokens[0, 0] == 4       # uniform p, u = 0.5 -> smallest x with (x+1)/10 >= 0.5


def test_residual_zero_fallback_flag():
    q = np.array([0.5, 0.5])
    # p(0) = 0 rejects proposal 0; residual (0, 0.5) draws token 1
    toks, n, f, _, _ = oracle.verify_block([np.array([0.0, 1.0]), q], [q], [0], [0.9, 0.3])
    assert n == 0 and toks[0] == 1 and f == 0
    # a target row with no mass: residual is 0 (flag 16), p is empty too (flag 8)
    toks, n, f, _, _ = oracle.verify_block([np.array([0.0, 0.0]), q], [q], [0], [0.9, 0.3])
    assert f & oracle.FLAG_RESIDUAL_ZERO and f & oracle.FLAG_EMPTY and toks[0] == -1


# ---------------------------------------------------------------- power of the pins

def _pin_suite_passes():
    """Fast subset of the pins above; False as soon as one fails."""
    g = _golden("three_token_example.json")
    p = np.array(g["reconstructed"]["p"])
    q = np.array(g["reconstructed"]["q"])
    toks, nacc = _simulate([p, p], [q], 8000, seed=1)
    if _chisq_pvalue_safe(np.bincount(toks[:, 0], minlength=3), p) < 1e-4:
        return False
    rng = np.random.default_rng(2)
    pairs = [_overlap_pair(0.6, rng=rng) for _ in range(4)]
    _, nacc = _simulate([pp for pp, _ in pairs] + [pairs[0][0]], [qq for _, qq in pairs],
                        8000, seed=3)
    expected = (1 - 0.6 ** 5) / 0.4
    emitted = nacc + 1
    if abs(emitted.mean() - expected) > 5 * emitted.std(ddof=1) / math.sqrt(8000):
        return False
    return True


def _chisq_pvalue_safe(counts, probs):
    try:
        return _chisq_pvalue(counts, probs)
    except AssertionError:
        return 0.0


MUTANTS = {
    "residual_is_p": ("residual_weights", lambda p, q: np.asarray(p, dtype=np.float64)),
    "residual_sign_flipped": ("residual_weights",
                              lambda p, q: np.maximum(np.asarray(q) - np.asarray(p), 0.0)),
    "residual_dropped_clamp": ("residual_weights",
                               lambda p, q: np.abs(np.asarray(p) - np.asarray(q))),
    "accept_inverted": ("accept", lambda u, px, qx: u * qx >= px),
    "accept_transposed": ("accept", lambda u, px, qx: u * px <= qx),
    "accept_always": ("accept", lambda u, px, qx: True),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    assert _pin_suite_passes()
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ov, attr, fn)
    assert not _pin_suite_passes(), f"mutant {name} survived the pins"
