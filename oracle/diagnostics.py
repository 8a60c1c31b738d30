"""Per-position diagnostics of a verification round, float64 CPU oracle.

TEST INFRASTRUCTURE, like the rest of this package: only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may use it.

Pages followed (cited by title and section):
  [ATLAS] "Speculative Decoding - Turn guesses into parallel work":
          "Confidence and verification admission" (the soft label of a
          confidence head is the overlap 1 - TV(p_k, q_k) of the target and
          draft distributions at position k), "Read the benchmark contract"
          (accepted-prefix histograms and conditional acceptance by position),
          "Accepted length is not speed" (c_i, the acceptance probability at
          position i given that the earlier positions survived; survival
          a_j = c_0 ... c_j).
  [DRAFT] "Drafters and Speculative Decoding: Useful Tokens, Correct State",
          "Sampling needs a correction rule": the worked three-token example,
          whose rejection mass 0.40 fixes the overlap 0.60.

Parity status:
  overlap                    pinned: worked example (0.6), the alpha = 0.8
                             family, 1 - TV computed from |p - q|, disjoint and
                             identical supports, and the Monte Carlo acceptance
                             rate of the oracle's own walk.
  position_overlaps          pinned: Monte Carlo conditional acceptance by
                             position of verify_sample on transformed rows.
  accepted_prefix_histogram  pinned: counts against a brute-force loop and
                             the sampled law below.
  conditional_acceptance     pinned: direct per-trial counts.
  prefix_length_law          pinned: closed form (1 - a^(g+1)) / (1 - a) of the
                             expected block length, chi-square of sampled
                             accepted lengths.
"""

import math

import numpy as np

from .verifier import row_distribution


def overlap(p, q):
    """alpha = sum_x min(p(x), q(x)) = 1 - TV(p, q).

    With x drawn from q and accepted with probability min(1, p(x)/q(x)), the
    acceptance probability is sum_x q(x) min(1, p(x)/q(x)) = alpha ([ATLAS]
    "Confidence and verification admission"; [DRAFT] "Sampling needs a
    correction rule"). Summed with math.fsum (correctly rounded).
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    return math.fsum(np.minimum(p, q).tolist())


def position_overlaps(target, draft, target_sampler, draft_sampler, banned=None):
    """alpha[b, i] = overlap(p_i, q_i) of target row i and draft row i, i < gamma,
    after every sampler transform (bans, temperature, top-k, top-p), i.e. the
    same p and q the walk of verify_sample compares.

    Returns (alpha [B, gamma], topp_margin [B, gamma]); the margin is the
    smaller top-p margin of the two rows (inf when top-p is off), so a caller
    can leave out pairs whose kept set sits on a rounding edge.
    """
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    B, G1, V = target.shape
    gamma = G1 - 1
    alpha = np.zeros((B, gamma))
    margin = np.full((B, gamma), math.inf)
    for b in range(B):
        bans = () if banned is None else [t for t in np.asarray(banned[b]).tolist() if t >= 0]
        for i in range(gamma):
            pd = row_distribution(target[b, i], target_sampler, bans)
            qd = row_distribution(draft[b, i], draft_sampler, bans)
            alpha[b, i] = overlap(pd.p, qd.p)
            margin[b, i] = min(pd.topp_margin, qd.topp_margin)
    return alpha, margin


def accepted_prefix_histogram(num_accepted, gamma):
    """counts[n] = number of requests whose walk accepted exactly n proposals,
    n = 0..gamma ([ATLAS] "Read the benchmark contract")."""
    counts = np.zeros(gamma + 1, dtype=np.int64)
    for n in np.asarray(num_accepted).tolist():
        counts[int(n)] += 1
    return counts


def conditional_acceptance(counts):
    """From an accepted-prefix histogram: reached[i] requests examined position
    i (accepted >= i proposals) and accepted[i] of them accepted it (accepted
    > i), i < gamma; accepted / reached estimates c_i ([DRAFT] "Accepted
    length is not speed")."""
    counts = np.asarray(counts, dtype=np.int64)
    gamma = counts.size - 1
    reached = np.array([counts[i:].sum() for i in range(gamma)], dtype=np.int64)
    accepted = np.array([counts[i + 1:].sum() for i in range(gamma)], dtype=np.int64)
    return reached, accepted


def prefix_length_law(alphas):
    """Law of the accepted length n of one request whose proposals are drawn
    from q_i, given the conditional acceptance probabilities c_i = alpha_i:
    P(n = k) = c_0 ... c_{k-1} (1 - c_k) for k < gamma and c_0 ... c_{gamma-1}
    for k = gamma ([ATLAS] "Accepted length is not speed": survival is the
    product of the conditional acceptances)."""
    alphas = [float(a) for a in alphas]
    gamma = len(alphas)
    law = np.zeros(gamma + 1)
    surv = 1.0
    for k in range(gamma):
        law[k] = surv * (1.0 - alphas[k])
        surv *= alphas[k]
    law[gamma] = surv
    return law
