"""Seeded synthetic workloads for the verifier (inputs only).

This module is shared by the parity tests (oracle side and HIP side) and by
bench.py. It holds none of the verifier's arithmetic: it draws logits, ban
lists and the random numbers a drafter would consume, and rounds to bf16.
It imports nothing from the oracle or from the HIP binding.

Workload recipes (sizes from the five benchmark configurations; the pages'
own workloads need models and prompt sets, so these synthetic rows stand in):
  c1   B=1,   gamma=4, V=1000,   fp32, target ~ N(0, 2^2), draft = target + N(0, 0.5^2),
       T=1, no truncation.
  c2   B=8,   gamma=5, V=32000,  bf16, target ~ N(0, 3^2) with 20 distinct random
       ids per row boosted by +8, draft = target + N(0, 1), T=0.7, top-k 50 (p and q).
  c3a  B=64,  gamma=7, V=128256, bf16, target ~ N(0, 3^2) plus Zipf(1.1)-ranked
       boosts 8 * r^-1.1 over a random rank permutation per row, draft noise 0.3, T=1.
  c3b  as c3a with draft noise 1.5 (low acceptance).
  c4   greedy: B=256, gamma=4, V=151936, bf16, target ~ N(0, 2^2); 1% of target rows
       get a second token set exactly equal to the row maximum; the proposal is
       the row argmax with probability 0.7, else a uniform random id.
  c5   B=128, gamma=8, V=151936, bf16, target ~ N(0, 3^2) plus Zipf boosts,
       draft = target + N(0, 1), T=0.8, top-p 0.9, 64 distinct banned ids per
       request applied to p and q.
  c5f32  c5's recipe and seed with float32 logits (not rounded to bf16).
Values are drawn in float32 from NumPy's PCG64 (default_rng(seed)), draft rows
add their noise to the unrounded target row, and bf16 rows are rounded to
nearest-even from float32.
"""

from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    mode: str                 # "sample" or "greedy"
    B: int
    gamma: int
    V: int
    dtype: str                # "bf16" or "f32"
    target_sd: float
    draft_sd: float = 0.0
    boost: str = "none"       # "none" | "random20" | "zipf"
    temperature: float = 1.0
    top_k: int = 0
    top_p: float = 1.0
    n_banned: int = 0
    tie_frac: float = 0.0
    match_prob: float = 0.0
    seed: int = 1000
    philox_seed: int = 0
    philox_offset: int = 0


CONFIGS = {
    "c1": Config("c1", "sample", 1, 4, 1000, "f32", 2.0, 0.5, seed=1001),
    "c2": Config("c2", "sample", 8, 5, 32000, "bf16", 3.0, 1.0, boost="random20",
                 temperature=0.7, top_k=50, seed=1002),
    "c3a": Config("c3a", "sample", 64, 7, 128256, "bf16", 3.0, 0.3, boost="zipf", seed=1003),
    "c3b": Config("c3b", "sample", 64, 7, 128256, "bf16", 3.0, 1.5, boost="zipf", seed=1013),
    "c4": Config("c4", "greedy", 256, 4, 151936, "bf16", 2.0, tie_frac=0.01,
                 match_prob=0.7, seed=1004),
    "c5": Config("c5", "sample", 128, 8, 151936, "bf16", 3.0, 1.0, boost="zipf",
                 temperature=0.8, top_p=0.9, n_banned=64, seed=1005),
    # c5's recipe with float32 logits (not rounded to bf16): the generic path
    "c5f32": Config("c5f32", "sample", 128, 8, 151936, "f32", 3.0, 1.0, boost="zipf",
                    temperature=0.8, top_p=0.9, n_banned=64, seed=1005),
}


def config(name, **overrides):
    """A named configuration, optionally with some fields replaced (smaller B, V, ...)."""
    return replace(CONFIGS[name], **overrides)


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest-even), returned as uint16 bit patterns."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    cfg: Config
    target: np.ndarray              # [B, gamma+1, V] float32 holding the exact logit values
    draft: np.ndarray               # [B, gamma, V] float32 (empty for greedy)
    target_bits: np.ndarray = None  # uint16 bf16 patterns (bf16 only)
    draft_bits: np.ndarray = None
    banned: np.ndarray = None       # [B, n_banned] int32 or None
    proposal_u: np.ndarray = None   # [B, gamma] uniforms a drafter consumes
    match_coin: np.ndarray = None   # greedy: [B, gamma] uniforms deciding argmax vs random
    random_tokens: np.ndarray = None  # greedy: [B, gamma] random proposals
    extra: dict = field(default_factory=dict)

    def target_f64(self, b=slice(None)):
        return self.target[b].astype(np.float64)

    def draft_f64(self, b=slice(None)):
        return self.draft[b].astype(np.float64)


def _boost_rows(rng, rows, cfg):
    n, V = rows.shape
    if cfg.boost == "random20":
        for r in range(n):
            ids = rng.choice(V, 20, replace=False)
            rows[r, ids] += np.float32(8.0)
    elif cfg.boost == "zipf":
        ranked = (8.0 * np.arange(1, V + 1, dtype=np.float64) ** -1.1).astype(np.float32)
        for r in range(n):
            perm = rng.permutation(V)
            rows[r, perm] += ranked


def make_workload(cfg):
    """Draw every input of one configuration from default_rng(cfg.seed)."""
    rng = np.random.default_rng(cfg.seed)
    B, G, V = cfg.B, cfg.gamma, cfg.V
    target = rng.standard_normal((B, G + 1, V), dtype=np.float32)
    target *= np.float32(cfg.target_sd)
    _boost_rows(rng, target.reshape(B * (G + 1), V), cfg)
    if cfg.mode == "sample":
        draft = rng.standard_normal((B, G, V), dtype=np.float32)
        draft *= np.float32(cfg.draft_sd)
        draft += target[:, :G, :]
    else:
        draft = np.zeros((B, 0, V), dtype=np.float32)

    wl = Workload(cfg, target, draft)
    if cfg.dtype == "bf16":
        wl.target_bits = f32_to_bf16_bits(target)
        wl.target = bf16_bits_to_f32(wl.target_bits)
        wl.draft_bits = f32_to_bf16_bits(draft)
        wl.draft = bf16_bits_to_f32(wl.draft_bits)

    if cfg.tie_frac > 0:
        rows = wl.target.reshape(B * (G + 1), V)
        n_tie = max(1, int(round(cfg.tie_frac * rows.shape[0])))
        tie_rows = rng.choice(rows.shape[0], n_tie, replace=False)
        for r in tie_rows:
            top = rows[r].max()
            other = int(rng.integers(V))
            while rows[r, other] == top:
                other = int(rng.integers(V))
            rows[r, other] = top
        if wl.target_bits is not None:
            wl.target_bits = f32_to_bf16_bits(wl.target)
        wl.extra["tie_rows"] = np.sort(tie_rows)

    if cfg.n_banned > 0:
        wl.banned = np.stack([rng.choice(V, cfg.n_banned, replace=False)
                              for _ in range(B)]).astype(np.int32)
    if cfg.mode == "sample":
        wl.proposal_u = 1.0 - rng.random((B, G))          # (0, 1]
    else:
        wl.match_coin = rng.random((B, G))
        wl.random_tokens = rng.integers(0, V, (B, G)).astype(np.int32)
    return wl
