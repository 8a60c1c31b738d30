"""Full-size parity sweep over many Philox offsets (run by hand on a GPU machine;
pytest does not collect it).

    python tests/sweep_parity.py [--offsets c2=1000,c3a=100,c3b=100,c5=100] [--out FILE]

For every configuration and every offset k the HIP path verifies the whole
batch with device Philox uniforms at (seed, k); the float64 oracle verifies the
same batch with the same uniforms, its requests split over up to 16 host
processes. Tokens, accepted counts and flags must be identical except for
requests with a decision within 1e-10 of its edge; the sweep counts decisions
(acceptance tests taken plus one final draw per request) and how many lie
within 1e-10 and within 1e-6 of their edge (counted per request: such a
request holds at least one such decision). Exits non-zero on any mismatch.
"""

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

EXACT_BAND = 1e-10
STATED_BAND = 1e-6


def _worker(conn):
    """Holds one slice of the batch; verifies it for each uniform block sent."""
    import oracle
    tgt, dft, xs, banned, samp = conn.recv()
    tgt = tgt.astype(np.float64)
    dft = dft.astype(np.float64)
    s = oracle.Sampler(*samp)
    while True:
        u = conn.recv()
        if u is None:
            return
        r = oracle.verify_sample(tgt, dft, xs, u, s, s, banned)
        conn.send((r.tokens, r.num_accepted, r.flags, r.margin))


def sweep(name, n_offsets, procs=16):
    import torch
    import lossless_draft_verification_sample_amd as sv
    import parity_util as pu
    wl = pu.make(name)
    cfg = wl.cfg
    xs = pu.stored_proposals(name)
    dev = torch.device("cuda:0")
    t = pu.logits_tensor(wl.target, wl.target_bits, cfg.dtype, dev)
    d = pu.logits_tensor(wl.draft, wl.draft_bits, cfg.dtype, dev)
    toks = torch.from_numpy(xs).to(dev)
    bans = None if wl.banned is None else torch.from_numpy(wl.banned).to(dev)
    samp = pu.sampler_of(cfg)
    n = max(1, min(procs, cfg.B))
    bounds = np.linspace(0, cfg.B, n + 1).astype(int)
    ctx = mp.get_context("spawn")
    workers = []
    for k in range(n):
        sl = slice(bounds[k], bounds[k + 1])
        mine, theirs = ctx.Pipe()
        p = ctx.Process(target=_worker, args=(theirs,), daemon=True)
        p.start()
        mine.send((wl.target[sl], wl.draft[sl], xs[sl],
                   None if wl.banned is None else wl.banned[sl], samp))
        workers.append((p, mine, sl))
    tot = {"config": name, "offsets": n_offsets, "requests": 0, "decisions": 0,
           "mismatched": 0, "requests_within_1e-10": 0, "requests_within_1e-6": 0}
    t0 = time.perf_counter()
    try:
        for off in range(n_offsets):
            out = sv.spec_verify_sample(t, d, toks, samp, samp, banned_ids=bans,
                                        seed=cfg.philox_seed, offset=off, want_lse=False)
            u = pu.philox_uniforms(cfg.philox_seed, off, cfg.B, cfg.gamma)
            for p, c, sl in workers:
                c.send(u[sl])
            parts = []
            for p, c, sl in workers:
                if not c.poll(600):
                    raise RuntimeError("oracle worker timed out")
                parts.append(c.recv())
            rt, rn, rf, rm = (np.concatenate([x[i] for x in parts]) for i in range(4))
            torch.cuda.synchronize()
            gt = out.tokens.cpu().numpy()
            gn = out.num_accepted.cpu().numpy()
            gf = out.flags.cpu().numpy().astype(np.uint32)
            same = (gt == rt).all(axis=1) & (gn == rn) & (gf == rf.astype(np.uint32))
            keep = rm > EXACT_BAND
            tot["requests"] += cfg.B
            tot["decisions"] += int(np.minimum(rn + 1, cfg.gamma).sum() + cfg.B)
            tot["mismatched"] += int((~same & keep).sum())
            tot["requests_within_1e-10"] += int((~keep).sum())
            tot["requests_within_1e-6"] += int((rm <= STATED_BAND).sum())
    finally:
        for p, c, sl in workers:
            try:
                c.send(None)
            except (BrokenPipeError, OSError):
                pass
            p.join(timeout=10)
            if p.is_alive():
                p.terminate()
    tot["seconds"] = round(time.perf_counter() - t0, 1)
    tot["fraction_within_1e-6"] = tot["requests_within_1e-6"] / max(tot["decisions"], 1)
    return tot


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--offsets", default="c2=1000,c3a=100,c3b=100,c5=100")
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    plan = [(k, int(v)) for k, v in (x.split("=") for x in args.offsets.split(","))]
    res = []
    for name, n in plan:
        r = sweep(name, n)
        print(json.dumps(r), flush=True)
        res.append(r)
    if args.out:
        with open(args.out, "w") as f:
            json.dump(res, f, indent=1)
    bad = sum(r["mismatched"] for r in res)
    sys.exit(1 if bad else 0)


if __name__ == "__main__":
    main()
