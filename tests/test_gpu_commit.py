"""Parity of spec_verify_commit with the oracle's chain KV-commit metadata
(oracle/commit.py). Integer work: bit-exact."""

import json
import os

import numpy as np
import pytest

import oracle
from tests import parity_util as pu
from tests.conftest import GOLDEN

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import lossless_draft_verification_sample_amd._lib as L
    L.load()


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(pu.torch_dev())


def _run(tokens, n, kv, slots):
    import torch
    import lossless_draft_verification_sample_amd as sv
    out = sv.spec_verify_commit(_dev(tokens), _dev(n), _dev(kv), None if slots is None else _dev(slots))
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy().astype(np.int64) for t in out]


def _check(tokens, n, kv, slots, where=""):
    got = _run(tokens, n, kv, slots)
    ref = oracle.commit_chain(tokens, n, kv, slots)
    for name, g, r in zip(("new_kv_len", "anchor", "n_free", "free_slots"), got, ref):
        if r is None:
            assert g is None, (where, name)
        else:
            assert np.array_equal(g, r), (where, name, g, r)


def test_running_example():
    with open(os.path.join(GOLDEN, "commit_example.json")) as f:
        r = json.load(f)["reading"]
    got = _run(np.array([r["tokens"]]), np.array([r["num_accepted"]]), np.array([r["kv_len"]]),
               np.array([r["slots"]]))
    e = r["expected"]
    assert got[0][0] == e["new_kv_len"] and got[1][0] == e["anchor"] and got[2][0] == e["n_free"]
    assert got[3][0].tolist() == e["free_slots"]


@pytest.mark.parametrize("B,gamma", [(1, 1), (7, 4), (300, 8), (5000, 63)])
def test_random_rounds(B, gamma):
    rng = np.random.default_rng(B + gamma)
    n = rng.integers(0, gamma + 1, B)
    n[0] = 0
    n[-1] = gamma
    toks = np.full((B, gamma + 1), -1)
    for b in range(B):
        toks[b, : n[b] + 1] = rng.integers(0, 150000, n[b] + 1)
    kv = rng.integers(0, 1 << 20, B)
    slots = rng.permutation(B * (gamma + 1)).reshape(B, gamma + 1)
    _check(toks, n, kv, slots, where=f"B={B} gamma={gamma}")
    _check(toks, n, kv, None, where=f"B={B} gamma={gamma} no slots")


def test_after_a_verification_call():
    # the verifier's own outputs, then the commit on the same stream
    wl = pu.make("c5", B=16, V=20011, seed=91)
    xs = pu.oracle_proposals(wl)
    got = pu.run_gpu_sample(wl, xs)
    cfg = wl.cfg
    kv = np.arange(cfg.B) * 100
    slots = np.arange(cfg.B * (cfg.gamma + 1)).reshape(cfg.B, cfg.gamma + 1) + 7
    _check(got["tokens"], got["num_accepted"], kv, slots, where="after sample")


def test_out_of_range_accept_count_leaves_request_unchanged():
    toks = np.array([[5, 6, 7], [8, 9, -1]])
    n = np.array([3, -1])
    kv = np.array([10, 20])
    slots = np.array([[1, 2, 3], [4, 5, 6]])
    nk, an, nf, fs = _run(toks, n, kv, slots)
    assert nk.tolist() == [10, 20] and an.tolist() == [-1, -1] and nf.tolist() == [0, 0]
    assert np.all(fs == -1)
