"""The generic path's top-k and top-p cuts (radix selection over the
order-preserving keys, one pass per 8-bit digit) against the oracle, at the
full c5 vocabulary: fp32 rows (32-bit keys, four digits) and bf16 rows that
leave the counted window (16-bit keys, two digits); every sampler shape
(top-p alone, top-k alone, both, top-k = 1), exact ties at the cut, and rows
whose kept values are all negative. Same bar as the other parity tests:
tokens, accepted counts and flags bit-exact outside the 1e-10 decision band,
lse within 1e-5."""

import numpy as np
import pytest

import oracle
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

SAMPLERS = [(0.8, 0, 0.9), (0.7, 50, 1.0), (1.0, 40, 0.95), (1.3, 1, 1.0), (0.5, 0, 0.5),
            (1.0, 3000, 0.999)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import lossless_draft_verification_sample_amd._lib as L
    L.load()


def _check(wl, samp, where, seed=3, offset=9):
    cfg = wl.cfg
    xs = pu.oracle_proposals(wl, samp)
    got = pu.run_gpu_sample(wl, xs, tsamp=samp, dsamp=samp, seed=seed, offset=offset)
    u = pu.philox_uniforms(seed, offset, cfg.B, cfg.gamma)
    ref = pu.run_oracle_sample(wl, xs, u, range(cfg.B), tsamp=samp, dsamp=samp)
    nb = pu.compare_sample(got, ref, range(cfg.B), where=where)
    assert nb <= 1, where


@pytest.mark.parametrize("samp", SAMPLERS)
def test_fp32_full_vocabulary(samp):
    wl = pu.make("c5f32", B=3, gamma=3, seed=400)
    _check(wl, samp, f"fp32 {samp}")


@pytest.mark.parametrize("samp", [(1.0, 1000, 1.0), (1.0, 0, 0.7), (1.0, 700, 0.9)])
def test_fp32_ties_at_the_cut(samp):
    # 40 distinct values, each shared by thousands of tokens: the cuts fall
    # inside runs of equal keys
    wl = pu.make("c5f32", B=2, gamma=2, seed=401)
    rng = np.random.default_rng(5)
    levels = np.sort(rng.normal(0, 2, 40)).astype(np.float32)
    wl.target = levels[rng.integers(0, 40, wl.target.shape)]
    wl.draft = levels[rng.integers(0, 40, wl.draft.shape)]
    _check(wl, samp, f"fp32 ties {samp}")


@pytest.mark.parametrize("samp", [(0.8, 0, 0.9), (1.0, 25, 1.0)])
def test_fp32_all_negative_rows(samp):
    wl = pu.make("c5f32", B=2, gamma=2, seed=402)
    wl.target = (wl.target - np.float32(80.0)).astype(np.float32)
    wl.draft = (wl.draft - np.float32(80.0)).astype(np.float32)
    _check(wl, samp, f"fp32 negative {samp}")


@pytest.mark.parametrize("samp", SAMPLERS)
def test_bf16_rows_on_the_generic_path(samp):
    # one logit of 700 in every row leaves the counted window (|z| < 512)
    from lossless_draft_verification_sample_amd import synth
    wl = pu.make("c5", B=3, gamma=3, seed=403)
    t, d = wl.target.copy(), wl.draft.copy()
    t[:, :, 777] = -700.0
    d[:, :, 778] = -700.0
    wl.target_bits = synth.f32_to_bf16_bits(t)
    wl.draft_bits = synth.f32_to_bf16_bits(d)
    wl.target = synth.bf16_bits_to_f32(wl.target_bits)
    wl.draft = synth.bf16_bits_to_f32(wl.draft_bits)
    _check(wl, samp, f"bf16 generic {samp}")


@pytest.mark.parametrize("samp", [(0.8, 0, 0.9), (1.0, 30, 1.0), (1.0, 200, 0.8)])
def test_fp32_bans_holding_the_maximum(samp):
    # every row's two largest logits are banned (the generic path then
    # recomputes the admissible maximum), next to duplicate and out-of-range
    # ids and a banned NaN; the counts and masses of the banned values are
    # taken out of the radix sums exactly
    wl = pu.make("c5f32", B=3, gamma=3, V=40009, seed=404)
    rng = np.random.default_rng(9)
    t, d = wl.target.copy(), wl.draft.copy()
    # the same two tokens top every row of a request, so that one ban list
    # covers them; in the last request a NaN sits at a third banned token
    for b in range(wl.cfg.B):
        top2 = rng.choice(wl.cfg.V, 2, replace=False)
        t[b, :, top2[0]] = 30.0
        t[b, :, top2[1]] = 29.5
        d[b, :, top2[0]] = 28.0
        d[b, :, top2[1]] = 27.5
        nan_id = (int(top2[0]) + 17) % wl.cfg.V
        if b == 2:   # a flagged request: only its flags are compared
            t[b, 0, nan_id] = np.nan
        bans = wl.banned[b].copy()
        bans[:6] = [top2[0], top2[1], top2[0], -1, wl.cfg.V + 3, nan_id]
        wl.banned[b] = bans
    wl.target, wl.draft = t.astype(np.float32), d.astype(np.float32)
    _check(wl, samp, f"fp32 banned maximum {samp}")


@pytest.mark.parametrize("m", [300, 516, 517, 2000])
@pytest.mark.parametrize("pmode", ["top-k", "top-k then top-p"])
def test_fp32_cut_inside_a_prefix_cluster(m, pmode):
    # m distinct values that share their first 16 key bits (all in
    # [8, 8.0625)) above a background that stays below 6, and ten values
    # above them: the top-k cut falls inside the cluster, so the last digit
    # level sees exactly m candidates, the most the third pass can list for
    # it being 516 (larger clusters take a fourth pass over the row)
    wl = pu.make("c5f32", B=2, gamma=2, V=30011, seed=405)
    rng = np.random.default_rng(11 + m)
    V = wl.cfg.V
    t = np.clip(rng.normal(0, 1, wl.target.shape), -6, 5.9).astype(np.float32)
    d = np.clip(rng.normal(0, 1, wl.draft.shape), -6, 5.9).astype(np.float32)
    base = np.float32(8.0).view(np.uint32)
    for arr in (t, d):
        for b in range(arr.shape[0]):
            for i in range(arr.shape[1]):
                pos = rng.choice(V, m + 10, replace=False)
                bits = base + rng.choice(1 << 16, m, replace=False).astype(np.uint32)
                arr[b, i, pos[:m]] = bits.view(np.float32)
                arr[b, i, pos[m:]] = 12.0 + np.arange(10, dtype=np.float32)
    wl.target, wl.draft = t, d
    k = 10 + m // 2
    samp = (1.0, k, 1.0) if pmode == "top-k" else (1.0, k, 0.97)
    _check(wl, samp, f"fp32 prefix cluster m={m} {samp}")
