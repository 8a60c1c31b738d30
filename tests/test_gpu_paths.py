"""Parity of code paths and limits of the HIP verifier beyond the benchmark
recipes: unaligned rows and many draw parts, vocabularies past the old LDS
bitmap size and past the radix selection's 2^24 elements, the largest draft
length, full ban lists, the zero-residual
fallback and explicit uniforms at the ends of (0, 1]. Same bar as
test_gpu_parity: bit-exact outside the 1e-10 decision band, lse within 1e-5."""

import numpy as np
import pytest

import oracle
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import lossless_draft_verification_sample_amd._lib as L
    L.load()


def _check(wl, xs, samp, banned=None, seed=0, offset=0, uniforms=None, where=""):
    cfg = wl.cfg
    u = pu.philox_uniforms(seed, offset, cfg.B, cfg.gamma) if uniforms is None else uniforms
    got = pu.run_gpu_sample(wl, xs, tsamp=samp, dsamp=samp, banned=banned, seed=seed, offset=offset,
                            uniforms=uniforms)
    ref = pu.run_oracle_sample(wl, xs, u, range(cfg.B), tsamp=samp, dsamp=samp, banned=banned)
    nb = pu.compare_sample(got, ref, range(cfg.B), where=where)
    assert nb <= 1, where
    return got, ref


@pytest.mark.parametrize("samp", [(0.8, 0, 0.9), (1.0, 0, 1.0), (0.7, 200, 1.0)])
def test_unaligned_rows_many_draw_parts(samp):
    # odd V: rows are not 16-byte aligned, so every load takes the scalar path;
    # V spans 49 sub-chunks, drawn by many parts per request
    V, B, gamma = 100003, 3, 4
    wl = pu.make("c5", B=B, gamma=gamma, V=V, seed=71)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    _check(wl, xs, samp, seed=5, offset=1, where=f"odd V {samp}")


def test_vocabulary_beyond_bitmap_size_fp32_bans():
    # fp32 rows take the generic path; a radix cut takes the 700 banned ids
    # (duplicates included) out of its exact sums
    V, B, gamma = 300007, 1, 2
    wl = pu.make("c3a", B=B, gamma=gamma, V=V, dtype="f32", boost="none", seed=72)
    rng = np.random.default_rng(72)
    banned = rng.integers(0, V, (B, 700)).astype(np.int32)
    banned[0, :50] = banned[0, 50:100]                  # duplicates
    wl.banned = banned
    samp = (0.9, 0, 0.95)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    _check(wl, xs, samp, banned=banned, where="V=300007 fp32")


@pytest.mark.parametrize("dtype,samp", [("f32", (0.8, 0, 0.9)), ("f32", (1.0, 50, 1.0)),
                                        ("bf16", (0.9, 0, 0.95))])
def test_vocabulary_beyond_the_radix_limit(dtype, samp):
    # 2^24 + 3 tokens: the generic path's cuts come from a bisection over the
    # order-preserving keys (the radix selection's fixed-point sums stop at
    # 2^24 elements); bf16 rows get there through one logit of -700, outside
    # the counted window. One request, one proposal; 67 MB per fp32 row.
    from lossless_draft_verification_sample_amd import synth
    V = (1 << 24) + 3
    wl = pu.make("c5f32" if dtype == "f32" else "c5", B=1, gamma=1, V=V, seed=79)
    if dtype == "bf16":
        t, d = wl.target.copy(), wl.draft.copy()
        t[:, :, 12345] = -700.0
        d[:, :, 12346] = -700.0
        wl.target_bits = synth.f32_to_bf16_bits(t)
        wl.draft_bits = synth.f32_to_bf16_bits(d)
        wl.target = synth.bf16_bits_to_f32(wl.target_bits)
        wl.draft = synth.bf16_bits_to_f32(wl.draft_bits)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    _check(wl, xs, samp, seed=3, offset=1, where=f"V=2^24+3 {dtype} {samp}")


def test_largest_gamma():
    wl = pu.make("c3a", B=2, gamma=63, V=1500, boost="none", target_sd=1.0, draft_sd=0.05,
                 seed=73)
    samp = (1.0, 0, 1.0)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    got, ref = _check(wl, xs, samp, where="gamma=63")
    assert got["num_accepted"].max() > 5            # long accepted prefixes occur


def test_full_ban_lists():
    V, B, gamma = 5000, 4, 3
    wl = pu.make("c5", B=B, gamma=gamma, V=V, seed=74)
    rng = np.random.default_rng(74)
    banned = rng.integers(-3, V + 3, (B, 2048)).astype(np.int32)   # padding, duplicates
    wl.banned = banned
    samp = (0.8, 0, 0.9)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    got, _ = _check(wl, xs, samp, banned=banned, where="2048 bans")
    for b in range(B):
        n = got["num_accepted"][b]
        assert got["tokens"][b, n] not in set(banned[b].tolist())


def test_zero_residual_falls_back_to_p():
    # p == q everywhere, and an out-of-range proposal forces a rejection there:
    # the residual max(0, p - q) has no mass, so the token is drawn from p
    V, B, gamma = 3000, 6, 3
    wl = pu.make("c3a", B=B, gamma=gamma, V=V, boost="none", seed=75)
    wl.draft = wl.target[:, :gamma].copy()
    wl.draft_bits = wl.target_bits[:, :gamma].copy()
    samp = (0.9, 0, 0.95)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    xs[:, 1] = V + 1
    got, ref = _check(wl, xs, samp, where="zero residual")
    assert np.all(got["num_accepted"] <= 1)
    assert np.all(got["flags"] & oracle.FLAG_RESIDUAL_ZERO)
    assert np.all(got["flags"] & oracle.FLAG_TOKEN_RANGE)


@pytest.mark.parametrize("name, samp", [("c5", (1.0, 0, 1.0)), ("c5", (0.8, 0, 0.9)),
                                         ("c5f32", (1.0, 0, 1.0))])
def test_zero_residual_at_full_vocabulary(name, samp):
    # p == q on every row of c5's vocabulary, c5's bans on both rows, and a
    # rejection forced at position 1: the draw's stream sums only the
    # residual, so the selecting workgroup makes the p sums of all 75
    # sub-chunks itself before it draws from p
    wl = pu.make(name, B=3, gamma=3, seed=78)
    g = wl.cfg.gamma
    wl.draft = wl.target[:, :g].copy()
    if wl.target_bits is not None:
        wl.draft_bits = wl.target_bits[:, :g].copy()
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    xs[:, 1] = wl.cfg.V + 1
    got, _ = _check(wl, xs, samp, banned=wl.banned, where=f"zero residual {name} {samp}")
    assert np.all(got["flags"] & oracle.FLAG_RESIDUAL_ZERO)
    assert np.all(got["num_accepted"] <= 1)


def test_explicit_uniforms_at_the_ends():
    V, B, gamma = 2000, 8, 3
    wl = pu.make("c3a", B=B, gamma=gamma, V=V, boost="none", seed=76)
    samp = (1.0, 0, 1.0)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    u = np.full((B, gamma + 1), 0.37)
    u[0::2, :gamma] = 1.0               # accept iff q <= p
    u[1::2, :gamma] = 2.0 ** -53        # the smallest uniform: accept whenever p > 0
    u[2, gamma] = 1.0                   # the draw's target is the whole mass: the last token
    u[3, gamma] = 2.0 ** -53            # the first token with weight
    cfg = wl.cfg
    got = pu.run_gpu_sample(wl, xs, tsamp=samp, dsamp=samp, uniforms=u)
    ref = pu.run_oracle_sample(wl, xs, u, range(B), tsamp=samp, dsamp=samp)
    nb = pu.compare_sample(got, ref, range(B), where="u at the ends")
    assert nb <= 2                      # requests 2 and 3 sit on a CDF edge by construction
    assert np.all(got["num_accepted"][1::2] == gamma)
    n2, n3 = got["num_accepted"][2], got["num_accepted"][3]
    w2 = np.flatnonzero(oracle.row_distribution(wl.target[2, n2].astype(np.float64),
                                                oracle.Sampler(*samp)).p > 0) if n2 == gamma else None
    if w2 is not None:
        assert got["tokens"][2, n2] == w2[-1]
    assert 0 <= got["tokens"][3, n3] < V


def test_many_requests_small_rows():
    # B far above the resident workgroup count, tiny V (one sub-chunk)
    wl = pu.make("c2", B=600, gamma=2, V=300, seed=77)
    samp = (0.7, 50, 1.0)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    _check(wl, xs, samp, seed=3, where="B=600")


@pytest.mark.parametrize("k", [5000, 30000])
def test_dense_truncated_targets_at_a_rejection(k):
    # a truncated target keeping ~12% (k = 5000) or ~75% (k = 30000) of V: the
    # draw's per-wave queue of kept tokens is drained mid-stream, or a
    # sub-chunk keeps more tokens than the queue holds and is evaluated in place
    V, B, gamma = 40000, 6, 3
    wl = pu.make("c3a", B=B, gamma=gamma, V=V, boost="none", target_sd=1.0, draft_sd=1.0,
                 seed=78 + k % 7)
    samp = (1.0, k, 1.0)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    got, ref = _check(wl, xs, samp, seed=9, where=f"top-k {k}")
    assert np.any(got["num_accepted"] < gamma)      # rejections take the queued path


@pytest.mark.parametrize("K", [1, 31, 32, 33, 64])
def test_residual_draw_from_one_crowded_sub_chunk(K):
    # target rows keep their top K tokens, all in the second sub-chunk of 2048
    # tokens and at distinct values; the draft rows are low there, so the
    # proposals are rejected at once and every kept token carries residual
    # weight p. The selecting workgroup draws from that sub-chunk's list of K
    # weighted tokens (in lane order; a list holds 32 at most, longer ones are
    # read again from the rows). Sixteen requests draw at sixteen uniforms.
    from lossless_draft_verification_sample_amd import synth
    V, B, gamma = 3 * 2048 + 100, 16, 2
    wl = pu.make("c3a", B=B, gamma=gamma, V=V, boost="none", target_sd=1.0, draft_sd=1.0,
                 seed=80 + K)
    rng = np.random.default_rng(80 + K)
    t, d = wl.target.copy(), wl.draft.copy()
    for b in range(B):
        for i in range(gamma + 1):
            pos = 2048 + rng.choice(2048, K, replace=False)
            t[b, i, pos] = 20.0 + 0.125 * rng.choice(96, K, replace=False)
            if i < gamma:
                d[b, i, pos] = -10.0
    wl.target_bits = synth.f32_to_bf16_bits(t)
    wl.draft_bits = synth.f32_to_bf16_bits(d)
    wl.target = synth.bf16_bits_to_f32(wl.target_bits)
    wl.draft = synth.bf16_bits_to_f32(wl.draft_bits)
    samp = (1.0, K, 1.0)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    got, _ = _check(wl, xs, samp, seed=11, offset=2, where=f"crowded sub-chunk K={K}")
    assert np.all(got["num_accepted"] == 0)
    picked = got["tokens"][:, 0]
    assert np.all((picked >= 2048) & (picked < 4096))
    if K > 1:
        assert len(set(picked.tolist())) > 1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_truncating_sampler_that_keeps_everything(dtype):
    # top-k above V: the sampler truncates nothing, yet the batch is drawn by
    # the kernel for truncating samplers, whose rejections take the queued
    # mode; every sub-chunk then overflows the queue and is evaluated in place
    V, B, gamma = 5000, 6, 3
    wl = pu.make("c3a", B=B, gamma=gamma, V=V, dtype=dtype, boost="none", target_sd=1.0,
                 draft_sd=1.0, seed=81)
    samp = (0.9, V + 5, 1.0)
    xs = pu.oracle_proposals(wl, draft_sampler=samp)
    got, _ = _check(wl, xs, samp, seed=4, where=f"top-k above V {dtype}")
    assert np.any(got["num_accepted"] < gamma)
