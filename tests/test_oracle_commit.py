"""Pins of the chain KV-commit oracle (oracle/commit.py): the running example
of "Drafters and Speculative Decoding", section "Committing state after
rejection", and invariants that hold for every round."""

import json
import os

import numpy as np

from oracle.commit import commit_chain
from tests.conftest import GOLDEN


def test_running_example():
    with open(os.path.join(GOLDEN, "commit_example.json")) as f:
        g = json.load(f)
    r, pr = g["reading"], g["printed"]
    voc = r["vocab"]
    # the fixture encodes the printed example
    assert r["tokens"][:2] == [voc[w] for w in pr["accepted_prefix"]]
    assert r["tokens"][2] == voc[pr["correction"]]
    assert r["num_accepted"] == len(pr["accepted_prefix"])
    assert r["gamma"] == len(pr["proposed_block"])
    new_kv, anchor, n_free, free = commit_chain([r["tokens"]], [r["num_accepted"]], [r["kv_len"]],
                                                [r["slots"]])
    e = r["expected"]
    assert new_kv[0] == e["new_kv_len"] == len(pr["retained_rows_through"])
    assert anchor[0] == e["anchor"] == voc[pr["pending_anchor"]]
    assert n_free[0] == e["n_free"] == len(pr["discarded"])
    assert free[0].tolist() == e["free_slots"]
    # the freed slots are those of the discarded proposals' positions
    pos_of = {w: i for i, w in enumerate(["saw"] + pr["proposed_block"])}
    assert [r["slots"][pos_of[w]] for w in pr["discarded"]] == e["free_slots"][:2]
    assert new_kv[0] + 1 == e["logical_len"] == len(pr["existing_prefix"]) + 3


def test_invariants_random_rounds():
    rng = np.random.default_rng(5)
    for gamma in (1, 3, 8):
        B = 200
        n = rng.integers(0, gamma + 1, B)
        toks = np.full((B, gamma + 1), -1)
        for b in range(B):
            toks[b, : n[b] + 1] = rng.integers(0, 1000, n[b] + 1)
        kv = rng.integers(0, 5000, B)
        slots = rng.permutation(B * (gamma + 1)).reshape(B, gamma + 1)
        new_kv, anchor, n_free, free = commit_chain(toks, n, kv, slots)
        assert np.all(new_kv - kv == n + 1)
        assert np.all(anchor == toks[np.arange(B), n])
        assert np.all(n_free == gamma - n)
        for b in range(B):
            kept = slots[b, : n[b] + 1].tolist()
            freed = [s for s in free[b].tolist() if s >= 0]
            assert len(freed) == n_free[b]
            assert sorted(kept + freed) == sorted(slots[b].tolist())   # a partition
            assert np.all(free[b, n_free[b]:] == -1)
        full = n == gamma
        assert np.all(n_free[full] == 0)
    _, _, _, none = commit_chain(toks, n, kv, None)
    assert none is None


def test_ragged_lengths():
    # a request with g_b proposals wrote rows for positions K .. K+g_b only
    toks = np.array([[5, 6, -1, -1], [7, -1, -1, -1], [1, 2, 3, 4]])
    n = np.array([1, 0, 3])
    kv = np.array([10, 20, 30])
    slots = np.array([[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]])
    gammas = np.array([2, 0, 3])
    new_kv, anchor, n_free, free = commit_chain(toks, n, kv, slots, gammas)
    assert new_kv.tolist() == [12, 21, 34] and anchor.tolist() == [6, 7, 4]
    assert n_free.tolist() == [1, 0, 0]
    assert free.tolist() == [[2, -1, -1], [-1, -1, -1], [-1, -1, -1]]
    # an accepted count beyond the request's own length is not a verifier output
    new_kv, anchor, n_free, _ = commit_chain(toks, np.array([3, 0, 3]), kv, slots, gammas)
    assert new_kv[0] == 10 and anchor[0] == -1 and n_free[0] == 0
