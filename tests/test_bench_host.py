"""Host logic of bench.py: the parity summary and the pooled oracle baseline
(CPU only; no GPU call)."""

import os
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from lossless_draft_verification_sample_amd import synth  # noqa: E402


def _as_out(refs, torch):
    cat = lambda k: np.concatenate([getattr(r, k) for r in refs])  # noqa: E731
    return SimpleNamespace(tokens=torch.from_numpy(cat("tokens").copy()),
                           num_accepted=torch.from_numpy(cat("num_accepted").copy()),
                           flags=torch.from_numpy(cat("flags").astype(np.int32)))


def test_parity_summary_counts_mismatches():
    import torch
    cfg = synth.config("c5", B=6, V=3001)
    wl = synth.make_workload(cfg)
    xs = np.zeros((cfg.B, cfg.gamma), np.int32)
    refs = []
    base = bench.cpu_baseline(wl, xs, 15, refs)
    assert base["cores"] == 1 and base["value"] > 0
    assert sum(len(r.num_accepted) for r in refs) == cfg.B
    out = _as_out(refs, torch)
    s = bench.parity_summary(cfg, out, refs)
    assert s["requests"] == cfg.B and s["mismatched"] == 0
    assert s["compared"] + s["excluded"] == cfg.B
    out.tokens[2, 0] += 1                      # planted differences in two requests
    out.flags[4] ^= 1
    s = bench.parity_summary(cfg, out, refs)
    margin = np.concatenate([r.margin for r in refs])
    assert s["mismatched"] == int(margin[2] > 1e-10) + int(margin[4] > 1e-10)


def test_parity_summary_greedy():
    import torch
    wl = synth.make_workload(synth.config("c4", B=5, V=2003))
    xs = np.zeros((5, wl.cfg.gamma), np.int32)
    refs = []
    bench.cpu_baseline(wl, xs, 15, refs)
    out = _as_out(refs, torch)
    assert bench.parity_summary(wl.cfg, out, refs)["mismatched"] == 0
    out.num_accepted[0] += 1
    assert bench.parity_summary(wl.cfg, out, refs)["mismatched"] == 1


def test_pooled_oracle_baseline():
    cfg = synth.config("c5", B=4, V=3001)
    wl = synth.make_workload(cfg)
    xs = np.zeros((cfg.B, cfg.gamma), np.int32)
    r = bench.cpu_baseline_pool(wl, xs, max_workers=2)
    assert r["cores"] == 2 and r["value"] > 0 and r["kind"] == "oracle"
