"""Parity of mixed batches (per-request draft lengths, samplers with greedy
requests among sampled ones, draft-only ban lists, settings out of range)
with oracle.verify_batch. Same bar as test_gpu_parity: tokens, accept counts
and flags bit-exact outside the 1e-10 decision band, lse within 1e-5, NaN
exactly where a request does not use a row."""

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


def _dev(a, dtype=np.int32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).to(pu.torch_dev())


def _mixed_setup(wl, seed, n_greedy=3, bad=True, draft_bans=True):
    cfg = wl.cfg
    B, g, V = cfg.B, cfg.gamma, cfg.V
    rng = np.random.default_rng(seed)
    choices = [(0.8, 0, 0.9), (1.0, 0, 1.0), (0.7, 50, 1.0), (1.3, 0, 0.95), (0.9, 20, 0.8),
               (0.5, 0, 1.0)]
    ts = [choices[int(rng.integers(len(choices)))] for _ in range(B)]
    ds = [choices[int(rng.integers(len(choices)))] for _ in range(B)]
    greedy = rng.choice(B, n_greedy, replace=False)
    for b in greedy:
        ts[b] = (0.0, 0, 1.0)
    gammas = rng.integers(0, g + 1, B).astype(np.int32)
    gammas[0] = g
    gammas[1] = 0
    if bad:
        ts[2] = (1.0, 0, 1.5)          # top_p out of range
        gammas[3] = g + 2              # more proposals than the batch holds
    banned = rng.integers(-1, V, (B, 24)).astype(np.int32)
    banned_draft = rng.integers(-1, V, (B, 9)).astype(np.int32) if draft_bans else None
    # proposals: sampled requests draw from their transformed q; greedy ones
    # mostly copy the target argmax
    xs = np.zeros((B, g), dtype=np.int32)
    for b in range(B):
        db = [t for t in (banned_draft if draft_bans else banned)[b].tolist() if t >= 0]
        tb = [t for t in banned[b].tolist() if t >= 0]
        for i in range(g):
            if ts[b][0] == 0.0:
                am = oracle.greedy_argmax(wl.target[b, i].astype(np.float64), tb)
                xs[b, i] = am if rng.random() < 0.75 else int(rng.integers(V))
            elif oracle.sampler_valid(oracle.Sampler(*ds[b]), False):
                q = oracle.row_distribution(wl.draft[b, i].astype(np.float64),
                                            oracle.Sampler(*ds[b]), db).p
                xs[b, i] = oracle.sample_categorical(q, 1.0 - rng.random())[0]
    return ts, ds, gammas, banned, banned_draft, xs


def _run(wl, xs, ts, ds, gammas, banned, banned_draft, seed=4, offset=2, diagnostics=False,
         requests_override=None):
    import torch
    import lossless_draft_verification_sample_amd as sv
    cfg = wl.cfg
    dev = pu.torch_dev()
    t = pu.logits_tensor(wl.target, wl.target_bits, cfg.dtype, dev)
    d = pu.logits_tensor(wl.draft, wl.draft_bits, cfg.dtype, dev)
    req = requests_override or sv.Requests(
        gamma=None if gammas is None else _dev(gammas),
        target=sv.sampler_array(ts, dev), draft=sv.sampler_array(ds, dev),
        banned_draft=None if banned_draft is None else _dev(banned_draft))
    out = sv.spec_verify_sample(t, d, _dev(xs), (1.0, 0, 1.0), (1.0, 0, 1.0),
                                banned_ids=None if banned is None else _dev(banned),
                                seed=seed, offset=offset, requests=req,
                                want_overlap=diagnostics, want_hist=diagnostics)
    torch.cuda.synchronize()
    res = {k: getattr(out, k).cpu().numpy() for k in ("tokens", "num_accepted")}
    res["flags"] = out.flags.cpu().numpy().astype(np.uint32)
    res["target_lse"] = out.target_lse.cpu().numpy().astype(np.float64)
    res["draft_lse"] = out.draft_lse.cpu().numpy().astype(np.float64)
    if diagnostics:
        res["overlap"] = out.overlap.cpu().numpy()
        res["accept_hist"] = out.accept_hist.cpu().numpy().astype(np.int64)
    return res


def _oracle(wl, xs, ts, ds, gammas, banned, banned_draft, seed=4, offset=2):
    cfg = wl.cfg
    u = pu.philox_uniforms(seed, offset, cfg.B, cfg.gamma)
    return oracle.verify_batch(wl.target.astype(np.float64), wl.draft.astype(np.float64), xs, u,
                               [oracle.Sampler(*s) for s in ts], [oracle.Sampler(*s) for s in ds],
                               banned, banned_draft, gammas)


def _compare(got, ref, where):
    bnd = ref.margin <= pu.EXACT_BAND
    for b in range(len(ref.tokens)):
        assert got["flags"][b] == ref.flags[b], (where, b, got["flags"][b], ref.flags[b])
        if not bnd[b]:
            assert np.array_equal(got["tokens"][b], ref.tokens[b]), (where, b, got["tokens"][b],
                                                                     ref.tokens[b])
            assert got["num_accepted"][b] == ref.num_accepted[b], (where, b)
        for name, r in (("target_lse", ref.target_lse[b]), ("draft_lse", ref.draft_lse[b])):
            g = got[name][b]
            assert np.array_equal(np.isnan(g), np.isnan(r)), (where, b, name, g, r)
            fin = np.isfinite(r)
            assert np.array_equal(np.isfinite(g), fin), (where, b, name)
            assert np.all(np.abs(g[fin] - r[fin]) <= 1e-5 * np.maximum(1.0, np.abs(r[fin]))), where
    assert int(bnd.sum()) <= 1, where


@pytest.mark.parametrize("dtype,V", [("bf16", 20011), ("bf16", 40000), ("f32", 9001)])
def test_mixed_batch_matches_oracle(dtype, V):
    wl = pu.make("c5", B=12, gamma=5, V=V, dtype=dtype, seed=90 + V % 13)
    ts, ds, gammas, banned, banned_draft, xs = _mixed_setup(wl, seed=V)
    got = _run(wl, xs, ts, ds, gammas, banned, banned_draft)
    ref = _oracle(wl, xs, ts, ds, gammas, banned, banned_draft)
    _compare(got, ref, f"{dtype} V={V}")
    assert got["flags"][2] == oracle.FLAG_BAD_PARAM and got["flags"][3] == oracle.FLAG_BAD_PARAM
    assert got["num_accepted"][1] == 0


def test_shared_bans_and_no_ragged_lengths():
    wl = pu.make("c2", B=10, V=8000, seed=92)
    ts, ds, _, banned, _, xs = _mixed_setup(wl, seed=5, bad=False, draft_bans=False)
    got = _run(wl, xs, ts, ds, None, banned, None)
    ref = _oracle(wl, xs, ts, ds, None, banned, None)
    _compare(got, ref, "shared bans")


def test_uniform_requests_reproduce_the_plain_call():
    import lossless_draft_verification_sample_amd as sv
    wl = pu.make("c5", B=8, V=30011, seed=93)
    cfg = wl.cfg
    s = pu.sampler_of(cfg)
    xs = pu.oracle_proposals(wl)
    plain = pu.run_gpu_sample(wl, xs, seed=4, offset=2)
    dev = pu.torch_dev()
    req = sv.Requests(gamma=_dev(np.full(cfg.B, cfg.gamma)), target=sv.sampler_array([s] * cfg.B, dev),
                      draft=sv.sampler_array([s] * cfg.B, dev))
    import torch
    out = sv.spec_verify_sample(pu.logits_tensor(wl.target, wl.target_bits, cfg.dtype, dev),
                                pu.logits_tensor(wl.draft, wl.draft_bits, cfg.dtype, dev), _dev(xs),
                                s, s, banned_ids=_dev(wl.banned), seed=4, offset=2, requests=req)
    torch.cuda.synchronize()
    assert np.array_equal(out.tokens.cpu().numpy(), plain["tokens"])
    assert np.array_equal(out.num_accepted.cpu().numpy(), plain["num_accepted"])
    assert np.array_equal(out.flags.cpu().numpy().astype(np.uint32), plain["flags"])
    assert np.array_equal(out.target_lse.cpu().numpy(), plain["target_lse"].astype(np.float32))


def test_mixed_overlap_and_histogram():
    wl = pu.make("c5", B=10, gamma=4, V=12011, seed=94)
    ts, ds, gammas, banned, banned_draft, xs = _mixed_setup(wl, seed=6)
    got = _run(wl, xs, ts, ds, gammas, banned, banned_draft, diagnostics=True)
    ref = _oracle(wl, xs, ts, ds, gammas, banned, banned_draft)
    assert np.array_equal(got["accept_hist"], np.bincount(got["num_accepted"], minlength=5))
    for b in range(wl.cfg.B):
        sampled = not (ref.flags[b] & oracle.FLAG_BAD_PARAM) and ts[b][0] != 0.0
        for i in range(wl.cfg.gamma):
            a = got["overlap"][b, i]
            if not sampled or i >= gammas[b]:
                assert np.isnan(a), (b, i, a)
                continue
            tb = [t for t in banned[b].tolist() if t >= 0]
            db = [t for t in banned_draft[b].tolist() if t >= 0]
            pd = oracle.row_distribution(wl.target[b, i].astype(np.float64), oracle.Sampler(*ts[b]), tb)
            qd = oracle.row_distribution(wl.draft[b, i].astype(np.float64), oracle.Sampler(*ds[b]), db)
            if min(pd.topp_margin, qd.topp_margin) <= pu.EXACT_BAND:
                continue
            assert abs(a - oracle.overlap(pd.p, qd.p)) <= 1e-9, (b, i)


def test_mixed_commit():
    import torch
    import lossless_draft_verification_sample_amd as sv
    wl = pu.make("c5", B=12, gamma=5, V=8009, seed=95)
    ts, ds, gammas, banned, banned_draft, xs = _mixed_setup(wl, seed=7)
    got = _run(wl, xs, ts, ds, gammas, banned, banned_draft)
    B, G1 = got["tokens"].shape
    kv = np.arange(B) * 10
    slots = np.arange(B * G1).reshape(B, G1) + 100
    out = sv.spec_verify_commit(_dev(got["tokens"]), _dev(got["num_accepted"]), _dev(kv), _dev(slots),
                                gamma_b=_dev(gammas))
    torch.cuda.synchronize()
    ref = oracle.commit_chain(got["tokens"], got["num_accepted"], kv, slots, gammas)
    for g, r in zip(out, ref):
        assert np.array_equal(g.cpu().numpy().astype(np.int64), r)


def _penalty_setup(wl, seed, H=40):
    """History rich in each request's high-logit tokens, per-request factors
    (1 = off for some), one request with an invalid factor."""
    cfg = wl.cfg
    rng = np.random.default_rng(seed)
    hist = np.full((cfg.B, H), -1, dtype=np.int32)
    for b in range(cfg.B):
        top = np.argsort(-wl.target[b, 0])[:H // 2]
        hist[b, :H // 2] = top
        hist[b, H // 2:H - 4] = rng.integers(0, cfg.V, H // 2 - 4)
    pen_t = rng.choice(np.array([1.0, 1.3, 2.0], np.float32), cfg.B)
    pen_d = rng.choice(np.array([1.0, 1.2, 1.8], np.float32), cfg.B)
    pen_t[4] = 0.5                                   # out of range: not verified
    return hist, pen_t, pen_d


def _run_pen(wl, xs, ts, ds, gammas, banned, banned_draft, hist, pen_t, pen_d, diagnostics=False):
    import torch
    import lossless_draft_verification_sample_amd as sv
    dev = pu.torch_dev()
    req = sv.Requests(gamma=None if gammas is None else _dev(gammas),
                      target=sv.sampler_array(ts, dev), draft=sv.sampler_array(ds, dev),
                      banned_draft=None if banned_draft is None else _dev(banned_draft),
                      history=_dev(hist),
                      penalty=torch.from_numpy(pen_t).to(dev),
                      penalty_draft=torch.from_numpy(pen_d).to(dev))
    return _run(wl, xs, ts, ds, gammas, banned, banned_draft, diagnostics=diagnostics,
                requests_override=req)


@pytest.mark.parametrize("dtype,V", [("bf16", 20011), ("f32", 7001)])
def test_repetition_penalty_matches_oracle(dtype, V):
    wl = pu.make("c5", B=12, gamma=5, V=V, dtype=dtype, seed=96 + V % 11)
    ts, ds, gammas, banned, banned_draft, xs = _mixed_setup(wl, seed=V + 1)
    hist, pen_t, pen_d = _penalty_setup(wl, seed=V + 2)
    got = _run_pen(wl, xs, ts, ds, gammas, banned, banned_draft, hist, pen_t, pen_d)
    cfg = wl.cfg
    u = pu.philox_uniforms(4, 2, cfg.B, cfg.gamma)
    ref = oracle.verify_batch(wl.target.astype(np.float64), wl.draft.astype(np.float64), xs, u,
                              [oracle.Sampler(*s) for s in ts], [oracle.Sampler(*s) for s in ds],
                              banned, banned_draft, gammas, hist, pen_t, pen_d, dtype)
    _compare(got, ref, f"penalty {dtype}")
    assert got["flags"][4] & oracle.FLAG_BAD_PARAM
    # the test has power: without penalties the outputs differ
    ref0 = oracle.verify_batch(wl.target.astype(np.float64), wl.draft.astype(np.float64), xs, u,
                               [oracle.Sampler(*s) for s in ts], [oracle.Sampler(*s) for s in ds],
                               banned, banned_draft, gammas, None, None, None, dtype)
    fin = np.isfinite(ref.target_lse) & np.isfinite(ref0.target_lse)
    assert (not np.array_equal(ref.tokens, ref0.tokens)) or np.abs(
        ref.target_lse[fin] - ref0.target_lse[fin]).max() > 1e-3


def test_penalty_outside_the_counted_window():
    # a penalized logit of -300 becomes -600: beyond the bf16 count window, so
    # the row takes the generic path
    wl = pu.make("c5", B=3, gamma=2, V=5003, seed=97)
    from lossless_draft_verification_sample_amd import synth
    t = wl.target.copy()
    t[:, :, 17] = -300.0
    wl.target = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(t))
    wl.target_bits = synth.f32_to_bf16_bits(wl.target)
    ts = [(1.0, 0, 1.0)] * 3
    ds = [(1.0, 0, 1.0)] * 3
    xs = pu.oracle_proposals(wl, draft_sampler=(1.0, 0, 1.0))
    hist = np.array([[17, 3], [17, -1], [-1, -1]], dtype=np.int32)
    pen = np.array([2.0, 2.0, 2.0], np.float32)
    got = _run_pen(wl, xs, ts, ds, None, None, None, hist, pen, pen)
    u = pu.philox_uniforms(4, 2, 3, 2)
    ref = oracle.verify_batch(wl.target.astype(np.float64), wl.draft.astype(np.float64), xs, u,
                              [oracle.Sampler(*s) for s in ts], [oracle.Sampler(*s) for s in ds],
                              None, None, None, hist, pen, pen, "bf16")
    _compare(got, ref, "penalty window")


def test_overlap_with_penalties():
    wl = pu.make("c5", B=8, gamma=4, V=9001, seed=98)
    ts, ds, gammas, banned, banned_draft, xs = _mixed_setup(wl, seed=8, bad=False)
    hist, pen_t, pen_d = _penalty_setup(wl, seed=9)
    pen_t[4] = 1.5
    got = _run_pen(wl, xs, ts, ds, gammas, banned, banned_draft, hist, pen_t, pen_d,
                   diagnostics=True)
    for b in range(wl.cfg.B):
        if ts[b][0] == 0.0:
            assert np.all(np.isnan(got["overlap"][b]))
            continue
        tb = [t for t in banned[b].tolist() if t >= 0]
        db = [t for t in banned_draft[b].tolist() if t >= 0]
        hb = [t for t in hist[b].tolist() if t >= 0]
        for i in range(int(gammas[b])):
            pen_set = hb + xs[b, :i].tolist()
            pd = oracle.row_distribution(wl.target[b, i].astype(np.float64), oracle.Sampler(*ts[b]), tb,
                                         pen_set, float(pen_t[b]), "bf16")
            qd = oracle.row_distribution(wl.draft[b, i].astype(np.float64), oracle.Sampler(*ds[b]), db,
                                         pen_set, float(pen_d[b]), "bf16")
            if min(pd.topp_margin, qd.topp_margin) <= pu.EXACT_BAND:
                continue
            assert abs(got["overlap"][b, i] - oracle.overlap(pd.p, qd.p)) <= 1e-9, (b, i)


@pytest.mark.parametrize("dtype,V", [("bf16", 20011), ("f32", 7001)])
def test_penalty_at_the_history_limit(dtype, V):
    """The longest history the interface accepts (SV_MAX_HISTORY ids, all
    distinct) plus 63 distinct proposals: every row's penalized set is as large
    as it can be (2047 ids at the bonus row). A sampled request with top-p, a
    greedy request and a sampled request with top-k; the draft rows of the
    sampled ones are penalized too."""
    import lossless_draft_verification_sample_amd as sv
    g = 63
    H = sv.SV_MAX_HISTORY
    wl = pu.make("c5", B=3, gamma=g, V=V, dtype=dtype, seed=99 + V % 7)
    rng = np.random.default_rng(V)
    ids = rng.permutation(V).astype(np.int32)
    xs = np.stack([ids[b * g:(b + 1) * g] for b in range(3)])
    rest = ids[3 * g:]
    hist = np.stack([rng.choice(rest, H, replace=False) for _ in range(3)]).astype(np.int32)
    # request 0 mostly proposes its penalized target's argmax, so that its walk
    # runs deep into the block
    for i in range(g):
        pen_set = hist[0].tolist() + xs[0, :i].tolist()
        am = oracle.greedy_argmax(wl.target[0, i].astype(np.float64), (), pen_set, 1.3, dtype)
        if am not in xs[0, :i].tolist() and am not in hist[0].tolist():
            xs[0, i] = am
    ts = [(0.8, 0, 0.9), (0.0, 0, 1.0), (1.0, 40, 1.0)]
    ds = [(0.8, 0, 0.9), (1.0, 0, 1.0), (1.0, 40, 1.0)]
    pen_t = np.array([1.3, 1.5, 1.2], np.float32)
    pen_d = np.array([1.1, 1.0, 1.4], np.float32)
    banned = rng.integers(-1, V, (3, 16)).astype(np.int32)
    got = _run_pen(wl, xs, ts, ds, None, banned, None, hist, pen_t, pen_d)
    u = pu.philox_uniforms(4, 2, 3, g)
    ref = oracle.verify_batch(wl.target.astype(np.float64), wl.draft.astype(np.float64), xs, u,
                              [oracle.Sampler(*s) for s in ts], [oracle.Sampler(*s) for s in ds],
                              banned, None, None, hist, pen_t, pen_d, dtype)
    _compare(got, ref, f"history limit {dtype}")
    assert not np.any(got["flags"] & oracle.FLAG_BAD_PARAM)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_residual_with_penalties(dtype):
    # p == q on every row (same logits, samplers, bans and penalties on both
    # sides) and a rejection forced at position 1: the residual has no mass,
    # so the selecting workgroup makes the penalized p sums of all 35
    # sub-chunks (three batches of at most 16, the last one ragged) and draws
    # from p
    V, B, g = 70001, 6, 3
    wl = pu.make("c5", B=B, gamma=g, V=V, dtype=dtype, seed=131)
    wl.draft = wl.target[:, :g].copy()
    if wl.target_bits is not None:
        wl.draft_bits = wl.target_bits[:, :g].copy()
    rng = np.random.default_rng(132)
    choices = [(0.8, 0, 0.9), (1.0, 0, 1.0), (0.7, 50, 1.0), (1.3, 0, 0.95), (0.9, 300, 0.8),
               (1.1, 0, 1.0)]
    ts = [choices[b % len(choices)] for b in range(B)]
    gammas = np.full(B, g, np.int32)
    banned = rng.integers(-1, V, (B, 24)).astype(np.int32)
    hist, pen_t, _ = _penalty_setup(wl, seed=133)
    pen_t = np.array([1.3, 2.0, 1.0, 1.5, 1.2, 1.8], np.float32)
    xs = np.zeros((B, g), dtype=np.int32)
    for b in range(B):
        tb = [t for t in banned[b].tolist() if t >= 0]
        for i in range(g):
            pen = [t for t in np.concatenate([hist[b], xs[b, :i]]).tolist() if 0 <= t < V]
            q = oracle.row_distribution(wl.draft[b, i].astype(np.float64), oracle.Sampler(*ts[b]),
                                        tb, pen, float(pen_t[b]), dtype).p
            xs[b, i] = oracle.sample_categorical(q, 1.0 - rng.random())[0]
    xs[:, 1] = V + 1
    got = _run_pen(wl, xs, ts, ts, gammas, banned, None, hist, pen_t, pen_t)
    u = pu.philox_uniforms(4, 2, B, g)
    ref = oracle.verify_batch(wl.target.astype(np.float64), wl.draft.astype(np.float64), xs, u,
                              [oracle.Sampler(*s) for s in ts], [oracle.Sampler(*s) for s in ts],
                              banned, None, gammas, hist, pen_t, pen_t, dtype)
    _compare(got, ref, f"zero residual with penalties {dtype}")
    assert np.all(got["flags"] & oracle.FLAG_RESIDUAL_ZERO)
    assert np.all(got["num_accepted"] == 1)
