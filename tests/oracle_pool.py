"""The float64 oracle over a whole batch, its requests split across host
processes, for the full-size parity tests.

Each worker process receives its slice of the batch once, then verifies it for
every block of uniforms it is sent. Workers import only NumPy and the oracle
(never torch or the HIP library), so they start fast and never touch the GPU.
"""

import multiprocessing as mp
import os

import numpy as np

# the host share of one GPU on the boxes the GPU tests run on
MAX_WORKERS = 16


def _worker(conn):
    import oracle
    tgt, dft, xs, banned, tsamp, dsamp = conn.recv()
    tgt = tgt.astype(np.float64)
    dft = dft.astype(np.float64)
    ts, ds = oracle.Sampler(*tsamp), oracle.Sampler(*dsamp)
    while True:
        u = conn.recv()
        if u is None:
            return
        r = oracle.verify_sample(tgt, dft, xs, u, ts, ds, banned)
        conn.send((r.tokens, r.num_accepted, r.flags, r.margin, r.target_lse, r.draft_lse))


class OraclePool:
    """with OraclePool(target, draft, xs, banned, tsamp, dsamp) as pool:
           tokens, num_accepted, flags, margin, target_lse, draft_lse = pool.verify(u)
    target [B, gamma+1, V] and draft [B, gamma, V] as float32 (upcast to
    float64 in the workers), xs [B, gamma], banned [B, n] or None, samplers as
    (temperature, top_k, top_p) tuples, u [B, gamma+1]."""

    def __init__(self, target, draft, xs, banned, tsamp, dsamp, workers=MAX_WORKERS,
                 timeout_s=300.0):
        B = target.shape[0]
        n = max(1, min(workers, os.cpu_count() or 1, B))
        self.bounds = np.linspace(0, B, n + 1).astype(int)
        self.timeout_s = timeout_s
        ctx = mp.get_context("spawn")
        self.workers = []
        try:
            for k in range(n):
                sl = slice(self.bounds[k], self.bounds[k + 1])
                mine, theirs = ctx.Pipe()
                p = ctx.Process(target=_worker, args=(theirs,), daemon=True)
                p.start()
                mine.send((target[sl], draft[sl], xs[sl], None if banned is None else banned[sl],
                           tuple(tsamp), tuple(dsamp)))
                self.workers.append((p, mine))
        except BaseException:
            self.close()
            raise

    def verify(self, u):
        for k, (_, c) in enumerate(self.workers):
            c.send(u[self.bounds[k]:self.bounds[k + 1]])
        parts = []
        for _, c in self.workers:
            if not c.poll(self.timeout_s):
                raise RuntimeError("oracle worker timed out")
            parts.append(c.recv())
        return tuple(np.concatenate([p[i] for p in parts]) for i in range(6))

    def close(self):
        for p, c in self.workers:
            try:
                c.send(None)
            except (BrokenPipeError, OSError):
                pass
        for p, _ in self.workers:
            p.join(timeout=10)
            if p.is_alive():
                p.terminate()
        self.workers = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
