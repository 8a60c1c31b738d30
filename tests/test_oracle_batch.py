"""Pins of the oracle's mixed-batch verification (oracle.verify_batch) and of
greedy verification with bans (oracle.greedy_argmax, oracle.verify_greedy).

A mixed batch composes pinned parts: each request must equal the same request
verified alone, a request with g_b proposals must equal a batch of draft
length g_b, and a greedy request must equal greedy verification. Draft-only
bans are checked against what the pages fix for any proposal distribution:
the emitted token still follows p."""

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import _chisq_pvalue


def test_greedy_argmax_brute_force():
    rng = np.random.default_rng(1)
    for _ in range(300):
        V = int(rng.integers(1, 12))
        z = rng.integers(-3, 3, V).astype(np.float64)      # many exact ties
        z[rng.random(V) < 0.15] = -np.inf
        z[rng.random(V) < 0.1] = np.nan
        bans = rng.integers(-2, V + 2, int(rng.integers(0, 4))).tolist()
        best, arg = None, -1
        for x in range(V):
            if x in bans or np.isnan(z[x]):
                continue
            if best is None or z[x] > best:
                best, arg = z[x], x
        assert oracle.greedy_argmax(z, bans) == arg, (z, bans)
    assert oracle.greedy_argmax(np.array([1.0, 2.0]), [0, 1]) == -1
    assert oracle.greedy_argmax(np.array([-np.inf, -np.inf]), [0]) == 1


def _workload(B, gamma, V, seed):
    rng = np.random.default_rng(seed)
    target = rng.normal(0, 2, (B, gamma + 1, V))
    draft = target[:, :gamma] + rng.normal(0, 0.7, (B, gamma, V))
    return rng, target, draft


def _proposals(rng, draft, samplers, bans):
    B, gamma, V = draft.shape
    xs = np.zeros((B, gamma), dtype=np.int64)
    for b in range(B):
        s = samplers[b]
        if oracle.verifier._f32(s.temperature) == 0.0:
            s = oracle.Sampler()
        for i in range(gamma):
            q = oracle.row_distribution(draft[b, i], s, bans[b]).p
            xs[b, i] = oracle.sample_categorical(q, 1.0 - rng.random())[0]
    return xs


def test_uniform_metadata_equals_verify_sample():
    B, gamma, V = 5, 3, 40
    rng, target, draft = _workload(B, gamma, V, 2)
    s = oracle.Sampler(0.8, 10, 0.9)
    banned = rng.integers(0, V, (B, 3))
    xs = _proposals(rng, draft, [s] * B, [b.tolist() for b in banned])
    u = 1.0 - rng.random((B, gamma + 1))
    a = oracle.verify_sample(target, draft, xs, u, s, s, banned)
    c = oracle.verify_batch(target, draft, xs, u, [s] * B, [s] * B, banned)
    for f in ("tokens", "num_accepted", "flags", "target_lse", "draft_lse", "margin"):
        assert np.array_equal(getattr(a, f), getattr(c, f)), f


def test_each_request_equals_itself_alone():
    B, gamma, V = 8, 4, 30
    rng, target, draft = _workload(B, gamma, V, 3)
    ts = [oracle.Sampler(0.7, 0, 0.9), oracle.Sampler(0.0), oracle.Sampler(1.3, 5, 1.0),
          oracle.Sampler(1.0), oracle.Sampler(0.0), oracle.Sampler(0.9, 0, 0.8),
          oracle.Sampler(1.0, 3, 0.95), oracle.Sampler(0.5)]
    ds = [oracle.Sampler(1.0), oracle.Sampler(1.0), oracle.Sampler(1.0, 8, 1.0),
          oracle.Sampler(0.6, 0, 0.9), oracle.Sampler(2.0), oracle.Sampler(0.9, 0, 0.8),
          oracle.Sampler(1.1), oracle.Sampler(0.5)]
    gammas = np.array([4, 2, 0, 3, 4, 1, 4, 2])
    banned = rng.integers(-1, V, (B, 4))
    banned_draft = rng.integers(-1, V, (B, 2))
    xs = _proposals(rng, draft, ds, [[t for t in row.tolist() if t >= 0] for row in banned_draft])
    u = 1.0 - rng.random((B, gamma + 1))
    r = oracle.verify_batch(target, draft, xs, u, ts, ds, banned, banned_draft, gammas)
    for b in range(B):
        g = int(gammas[b])
        assert np.all(r.tokens[b, g + 1:] == -1)
        if oracle.verifier._f32(ts[b].temperature) == 0.0:
            a = oracle.verify_greedy(target[b:b + 1, :g + 1], xs[b:b + 1, :g], banned[b:b + 1])
            assert np.array_equal(r.tokens[b, :g + 1], a.tokens[0])
            assert r.num_accepted[b] == a.num_accepted[0] and r.flags[b] == a.flags[0]
            assert np.all(np.isnan(r.target_lse[b]))
            continue
        # the request alone, with draft length g and its own uniforms
        ua = np.concatenate([u[b, :g], u[b, gamma:]])[None]
        tb = [t for t in banned[b].tolist() if t >= 0]
        db = [t for t in banned_draft[b].tolist() if t >= 0]
        pt = [oracle.row_distribution(target[b, i], ts[b], tb) for i in range(g + 1)]
        qd = [oracle.row_distribution(draft[b, i], ds[b], db) for i in range(g)]
        out, n, fb, _, _ = oracle.verify_block([d.p for d in pt], [d.p for d in qd],
                                               xs[b, :g].tolist(), ua[0])
        assert np.array_equal(r.tokens[b, :g + 1], out) and r.num_accepted[b] == n
        assert np.allclose(r.target_lse[b, :g + 1], [d.lse for d in pt])
        assert np.all(np.isnan(r.target_lse[b, g + 1:])) and np.all(np.isnan(r.draft_lse[b, g:]))
    assert r.num_accepted[2] == 0          # g_b = 0: the bonus draw only


def test_bad_parameters_are_flagged():
    B, gamma, V = 4, 2, 10
    rng, target, draft = _workload(B, gamma, V, 4)
    ok = oracle.Sampler(1.0)
    ts = [oracle.Sampler(-1.0), ok, oracle.Sampler(1.0, -2, 1.0), ok]
    ds = [ok, oracle.Sampler(0.0), ok, ok]
    gammas = np.array([2, 2, 2, 3])
    xs = np.zeros((B, gamma), dtype=np.int64)
    u = np.full((B, gamma + 1), 0.5)
    r = oracle.verify_batch(target, draft, xs, u, ts, ds, gammas=gammas)
    assert np.all(r.flags == oracle.FLAG_BAD_PARAM)
    assert np.all(r.tokens == -1) and np.all(r.num_accepted == 0)


@pytest.mark.parametrize("V", [3, 6])
def test_draft_only_bans_keep_the_output_law(V):
    # proposals drawn from a q with a draft-only ban; the emitted first token
    # must still follow p (the method is exact for any proposal distribution)
    rng = np.random.default_rng(10 + V)
    z_t = rng.normal(0, 1, V)
    z_d = z_t + rng.normal(0, 0.8, V)
    ts = oracle.Sampler(1.0)
    p = oracle.row_distribution(z_t, ts).p
    q = oracle.row_distribution(z_d, ts, [0]).p
    assert q[0] == 0.0 and p[0] > 0.0
    target = np.stack([z_t, z_t])[None]
    draft = z_d[None, None]
    counts = np.zeros(V)
    n = 8000
    for t in range(n):
        x = oracle.sample_categorical(q, 1.0 - rng.random())[0]
        u = 1.0 - rng.random((1, 2))
        r = oracle.verify_batch(target, draft, np.array([[x]]), u, [ts], [ts],
                                banned=None, banned_draft=np.array([[0]]))
        counts[r.tokens[0, 0]] += 1
    assert counts[0] > 0                       # reached only through the residual
    assert _chisq_pvalue(counts, p) > 1e-4


def test_zero_proposals_is_sampling_from_p0():
    rng = np.random.default_rng(11)
    V = 5
    z = rng.normal(0, 1, V)
    p = oracle.row_distribution(z, oracle.Sampler(0.8)).p
    target = np.stack([z, z])[None]
    draft = z[None, None]
    counts = np.zeros(V)
    for t in range(6000):
        u = 1.0 - rng.random((1, 2))
        r = oracle.verify_batch(target, draft, np.array([[0]]), u, [oracle.Sampler(0.8)],
                                [oracle.Sampler(0.8)], gammas=[0])
        assert r.num_accepted[0] == 0
        counts[r.tokens[0, 0]] += 1
    assert _chisq_pvalue(counts, p) > 1e-4
