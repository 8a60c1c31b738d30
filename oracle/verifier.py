"""Float64 CPU oracle of the batched speculative-sampling verifier.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import, call or execute anything in this package. The
product path (the HIP library and its Python binding) never touches it, and it
imports nothing from the product.

Everything is plain NumPy in float64 on exact upcasts of the inputs
(bf16 -> fp32 -> fp64 and fp32 -> fp64 are exact). Sampler parameters that the
C interface carries as fp32 (temperature, top_p) are first rounded to fp32 and
then widened, so both sides see the same numbers.

Pages followed (cited by title and section):
  [ATLAS]   "Speculative Decoding - Turn guesses into parallel work":
            "One round and shifted logits", "Exact sampling: account for every
            probability", "Greedy, sampling and the real sampler",
            "Implementation roadmap and tests".
  [DRAFT]   "Drafters and Speculative Decoding: Useful Tokens, Correct State":
            "Greedy verification", "Sampling needs a correction rule",
            "Distribution, seeded output and quality".
  [FUND]    "Speculative Decoding" (specdec fundamentals): "The Loop".
  [STD]     "Speculative Token Decoupling: Asynchronous Verification via
            Flash-Decoding": Equation 3.1 (acceptance min(1, p/q)).

Readings where the pages are silent:
  * transform order: bans -> temperature -> top-k -> top-p -> renormalise;
  * top-k keeps every token whose logit is >= the k-th largest (ties kept);
  * top-p keeps token x when the tempered mass of strictly larger logits is
    < top_p (the crossing token and its exact ties are kept);
  * acceptance: accept iff u * q(x) <= p(x) with u in (0, 1];
  * final draw: smallest token id x (ascending) whose running sum of weights
    reaches u * S;
  * greedy ties: lowest token id;
  * a proposal outside [0, V) or with q(x) = 0 is rejected and flagged.
"""

import math
from dataclasses import dataclass, field

import numpy as np

FLAG_TOKEN_RANGE = 1      # a draft token lies outside [0, V)
FLAG_Q_ZERO = 2           # an examined proposal has q(x) = 0
FLAG_NONFINITE = 4        # NaN or +inf in one of the request's rows
FLAG_EMPTY = 8            # a row of the request has no admissible token
FLAG_RESIDUAL_ZERO = 16   # residual mass was 0 at a rejection; drew from p instead
FLAG_BAD_PARAM = 32       # a per-request draft length or sampler setting is out of range

BOUNDARY_EPS = 1e-6       # a uniform this close to a decision edge is a boundary case


@dataclass(frozen=True)
class Sampler:
    """Per-distribution sampler settings; top_k = 0 and top_p = 1 switch truncation off."""
    temperature: float = 1.0
    top_k: int = 0
    top_p: float = 1.0


def _f32(x):
    return float(np.float32(x))


@dataclass
class RowDist:
    p: np.ndarray            # final probabilities over the vocabulary (float64)
    kept: np.ndarray         # admissible set after every transform
    lse: float               # log-normaliser of the tempered kept logits (-inf if empty)
    nonfinite: bool          # row held NaN or +inf
    empty: bool              # no admissible token
    topp_margin: float = math.inf   # distance of the top-p cut to its edge (inf if off)


def round_to_bf16(x):
    """The bf16 value nearest to float32 x (ties to the even mantissa), as a
    float: the 16 low bits of the float32 pattern are rounded away."""
    bits = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
    lsb = (bits >> 16) & 1
    r = ((bits + 0x7FFF + lsb) >> 16) << 16
    return float(np.array([r & 0xFFFFFFFF], dtype=np.uint32).view(np.float32)[0])


def repetition_penalty(z, theta, dtype):
    """Repetition penalty of one logit: the multiplicative penalty of Keskar et
    al. 2019 ("CTRL", section 4.1) in the sign-aware form inference engines
    use, z / theta for z > 0 and z * theta otherwise, theta >= 1. Computed in
    float32 and, for a bf16 row, rounded to bf16 like any op on a bf16 logits
    tensor, so the penalized logit is a value of the row's own dtype."""
    z32 = np.float32(z)
    t32 = np.float32(theta)
    v = float(z32 / t32) if z32 > 0 else float(z32 * t32)
    return round_to_bf16(v) if dtype == "bf16" else v


def row_distribution(z, sampler, banned_ids=(), penalized=(), penalty=1.0, dtype="f32"):
    """Sampler-transformed distribution of one logit row.

    [ATLAS] "Greedy, sampling and the real sampler" and [DRAFT] "Distribution,
    seeded output and quality": temperature, truncation, bans and repetition
    penalties must live inside p and q. Steps, in order:
      (i)   admissible set K: finite logits that are not banned (-inf = masked);
      (i')  repetition penalty (repetition_penalty) of the admissible tokens in
            `penalized` (each token once), for a row of dtype `dtype`;
      (ii)  tempered logits s = z / T;
      (iii) top-k: keep z >= the k-th largest admissible logit (multiplicity
            counted, ties kept);
      (iv)  top-p on the softmax p' of s over K: keep x when the mass of tokens
            with strictly larger logit is < P;
      (v)   p = softmax of s over the surviving set, lse = m + log Z.
    """
    z = np.asarray(z, dtype=np.float64)
    V = z.size
    T = _f32(sampler.temperature)
    P = _f32(sampler.top_p)
    k = int(sampler.top_k)

    nonfinite = bool(np.any(np.isnan(z) | (z == np.inf)))

    # (i) admissible set
    kept = np.isfinite(z)
    for tok in banned_ids:
        tok = int(tok)
        if 0 <= tok < V:
            kept[tok] = False

    # (i') repetition penalty
    if _f32(penalty) != 1.0:
        z = z.copy()
        for tok in sorted(set(int(t) for t in penalized)):
            if 0 <= tok < V and kept[tok]:
                z[tok] = repetition_penalty(z[tok], penalty, dtype)

    # (ii) temperature
    s = np.full(V, -np.inf)
    s[kept] = z[kept] / T

    # (iii) top-k by value; the threshold is the k-th entry of the descending sort
    if 0 < k < int(kept.sum()):
        desc = np.sort(z[kept])[::-1]
        tau_k = desc[k - 1]
        kept &= z >= tau_k

    # (iv) top-p over the distinct kept values, largest first
    margin = math.inf
    if P < 1.0 and kept.any():
        m1 = s[kept].max()
        e = np.zeros(V)
        e[kept] = np.exp(s[kept] - m1)
        p1 = e / e.sum()
        vals, inverse = np.unique(z[kept], return_inverse=True)   # ascending
        mass = np.bincount(inverse, weights=p1[kept], minlength=vals.size)
        vals, mass = vals[::-1], mass[::-1]                         # descending
        above = np.concatenate(([0.0], np.cumsum(mass)[:-1]))      # mass strictly above
        keep_val = above < P
        n_keep = int(keep_val.sum())           # >= 1 because above[0] = 0 < P
        tau_p = vals[n_keep - 1]
        margin = abs(above[n_keep - 1] - P)
        if n_keep < vals.size:
            margin = min(margin, abs(above[n_keep] - P))
        kept &= z >= tau_p

    # (v) renormalise over the surviving set
    p = np.zeros(V)
    if not kept.any():
        return RowDist(p, kept, -math.inf, nonfinite, True, margin)
    m = s[kept].max()
    e = np.exp(s[kept] - m)
    Z = e.sum()
    p[kept] = e / Z
    return RowDist(p, kept, m + math.log(Z), nonfinite, False, margin)


def sample_categorical(w, u):
    """Inverse-CDF draw from non-negative weights w with u in (0, 1].

    Returns (index, S, boundary_distance). The index is the smallest x whose
    left-to-right running sum C_x satisfies C_x >= u * S, where S = C_{V-1}.
    boundary_distance is how far u lies from the two edges C_{x-1}/S and C_x/S
    of the chosen cell. S = 0 returns index -1.
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    S = float(C[-1]) if C.size else 0.0
    if not S > 0.0:
        return -1, 0.0, math.inf
    t = u * S
    x = int(np.searchsorted(C, t, side="left"))
    if x >= C.size:                      # t above the last sum through rounding
        x = int(np.flatnonzero(w > 0)[-1])
    lo = C[x - 1] if x > 0 else 0.0
    dist = min(abs(u - lo / S), abs(u - C[x] / S))
    return x, S, dist


@dataclass
class SampleResult:
    tokens: np.ndarray            # [B, gamma+1] int32, -1 after the emitted block
    num_accepted: np.ndarray      # [B] int32
    flags: np.ndarray             # [B] uint32
    target_lse: np.ndarray        # [B, gamma+1] float64
    draft_lse: np.ndarray         # [B, gamma] float64
    boundary: np.ndarray          # [B] bool: some decision lay within BOUNDARY_EPS
    accept_prob: np.ndarray = field(default=None)   # [B, gamma] min(1, p/q), nan if not reached
    margin: np.ndarray = field(default=None)        # [B] smallest distance of any decision to its edge


def verify_sample(target, draft, draft_tokens, uniforms, target_sampler, draft_sampler,
                  banned=None):
    """Speculative-sampling verification of B requests.

    target: [B, gamma+1, V] logits; row i is the target distribution after the
            prefix plus proposals 0..i-1, row gamma the bonus distribution
            ([ATLAS] "One round and shifted logits").
    draft:  [B, gamma, V] logits; row i is the distribution proposal i was drawn from.
    draft_tokens: [B, gamma]; uniforms: [B, gamma+1] in (0, 1];
    banned: [B, n] token ids (-1 = padding) or None, applied to p and q.

    Per request ([FUND] "The Loop"; [ATLAS] "Exact sampling"; [STD] Eq. 3.1):
      walk i = 0..gamma-1, accept x_i iff u_i * q_i(x_i) <= p_i(x_i); stop at
      the first rejection n and draw from norm(max(0, p_n - q_n))
      ([DRAFT] "Sampling needs a correction rule"); if all gamma survive draw
      the bonus token from p_gamma.
    """
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    draft_tokens = np.asarray(draft_tokens)
    uniforms = np.asarray(uniforms, dtype=np.float64)
    B, G1, V = target.shape
    gamma = G1 - 1
    assert draft.shape == (B, gamma, V) and draft_tokens.shape == (B, gamma)
    assert uniforms.shape == (B, gamma + 1)

    tokens = np.full((B, gamma + 1), -1, dtype=np.int32)
    num_acc = np.zeros(B, dtype=np.int32)
    flags = np.zeros(B, dtype=np.uint32)
    tlse = np.zeros((B, gamma + 1))
    dlse = np.zeros((B, gamma))
    boundary = np.zeros(B, dtype=bool)
    acc_prob = np.full((B, gamma), np.nan)
    margin = np.full(B, math.inf)

    for b in range(B):
        bans = () if banned is None else [t for t in np.asarray(banned[b]).tolist() if t >= 0]
        pt = [row_distribution(target[b, i], target_sampler, bans) for i in range(gamma + 1)]
        qd = [row_distribution(draft[b, i], draft_sampler, bans) for i in range(gamma)]
        f = 0
        mg = math.inf
        for d in pt + qd:
            if d.nonfinite:
                f |= FLAG_NONFINITE
            if d.empty:
                f |= FLAG_EMPTY
            mg = min(mg, d.topp_margin)
        tlse[b] = [d.lse for d in pt]
        dlse[b] = [d.lse for d in qd]
        out, n, fb, bmg, ap = verify_block([d.p for d in pt], [d.p for d in qd],
                                           draft_tokens[b], uniforms[b])
        tokens[b] = out
        num_acc[b] = n
        flags[b] = f | fb
        margin[b] = min(mg, bmg)
        boundary[b] = margin[b] <= BOUNDARY_EPS
        acc_prob[b] = ap

    return SampleResult(tokens, num_acc, flags, tlse, dlse, boundary, acc_prob, margin)


def accept(u, p_x, q_x):
    """Acceptance test of one proposal: u * q(x) <= p(x), u in (0, 1].

    For q(x) > 0 this accepts with probability min(1, p(x)/q(x))
    ([STD] Eq. 3.1; [ATLAS] "Exact sampling"); it never divides, p >= q always
    accepts (u <= 1) and p = 0 never accepts (u > 0).
    """
    return u * q_x <= p_x


def residual_weights(p, q):
    """Unnormalised correction distribution max(0, p - q)
    ([DRAFT] "Sampling needs a correction rule")."""
    return np.maximum(np.asarray(p, dtype=np.float64) - np.asarray(q, dtype=np.float64), 0.0)


def verify_block(p_rows, q_rows, xs, u):
    """One request's walk over already-transformed distributions.

    p_rows: gamma+1 target distributions; q_rows: gamma draft distributions;
    xs: gamma proposals; u: gamma+1 uniforms. Returns
    (tokens[gamma+1], n_accepted, flags, margin, accept_prob[gamma]), where
    margin is the smallest distance, in units of u, between a uniform the walk
    consumed and the edge of the decision it took (the acceptance threshold
    p/q, or either cumulative edge of the drawn token's cell).
    """
    gamma = len(q_rows)
    V = len(p_rows[0])
    xs = [int(x) for x in xs]
    tokens = np.full(gamma + 1, -1, dtype=np.int32)
    acc_prob = np.full(gamma, np.nan)
    f = 0
    margin = math.inf
    if any(x < 0 or x >= V for x in xs):
        f |= FLAG_TOKEN_RANGE

    # left-to-right acceptance walk, stop at the first rejection
    n = gamma
    for i in range(gamma):
        x = xs[i]
        if x < 0 or x >= V:
            n = i
            break
        p_x = p_rows[i][x]
        q_x = q_rows[i][x]
        if q_x == 0.0:
            f |= FLAG_Q_ZERO
            n = i
            break
        ratio = p_x / q_x
        acc_prob[i] = min(1.0, ratio)
        margin = min(margin, abs(u[i] - ratio))
        if accept(u[i], p_x, q_x):
            tokens[i] = x
        else:
            n = i
            break

    # final draw: residual at the first rejection, bonus when all survived
    if n < gamma:
        w = residual_weights(p_rows[n], q_rows[n])
    else:
        w = p_rows[gamma]
    x, S, dist = sample_categorical(w, u[gamma])
    if n < gamma and x < 0:
        f |= FLAG_RESIDUAL_ZERO
        x, S, dist = sample_categorical(p_rows[n], u[gamma])
    if x < 0:
        f |= FLAG_EMPTY
    margin = min(margin, dist)
    tokens[n] = x
    return tokens, n, f, margin, acc_prob


def greedy_argmax(z, banned_ids=(), penalized=(), penalty=1.0, dtype="f32"):
    """Argmax of one target row for greedy verification ([DRAFT] "Greedy
    verification"; [ATLAS] "Greedy, sampling and the real sampler": bans are
    part of the real sampler). Admissible tokens are those not banned whose
    logit is not NaN; the result is the lowest admissible id holding the
    largest admissible logit (-inf included, so a row of -inf still has an
    argmax), or -1 when nothing is admissible. Tokens in `penalized` compete
    with their repetition_penalty value.
    """
    z = np.asarray(z, dtype=np.float64)
    adm = ~np.isnan(z)
    for tok in banned_ids:
        tok = int(tok)
        if 0 <= tok < z.size:
            adm[tok] = False
    if _f32(penalty) != 1.0:
        z = z.copy()
        for tok in sorted(set(int(t) for t in penalized)):
            if 0 <= tok < z.size and adm[tok] and np.isfinite(z[tok]):
                z[tok] = repetition_penalty(z[tok], penalty, dtype)
    if not adm.any():
        return -1
    m = z[adm].max()
    return int(np.flatnonzero(adm & (z == m))[0])


@dataclass
class GreedyResult:
    tokens: np.ndarray
    num_accepted: np.ndarray
    flags: np.ndarray
    argmax: np.ndarray            # [B, gamma+1] per-row argmax


def verify_greedy(target, draft_tokens, banned=None):
    """Greedy verification ([DRAFT] "Greedy verification"; [ATLAS] "Greedy,
    sampling and the real sampler"): keep proposals while they equal the target
    argmax of their row, emit the argmax at the first mismatch, or the bonus
    argmax of row gamma when all match. The argmax is greedy_argmax: lowest
    token id on exact ties, banned ids (banned[b], -1 = padding) and NaN
    excluded.
    """
    target = np.asarray(target, dtype=np.float64)
    draft_tokens = np.asarray(draft_tokens)
    B, G1, V = target.shape
    gamma = G1 - 1
    tokens = np.full((B, gamma + 1), -1, dtype=np.int32)
    num_acc = np.zeros(B, dtype=np.int32)
    flags = np.zeros(B, dtype=np.uint32)
    am = np.zeros((B, G1), dtype=np.int32)
    for b in range(B):
        f = 0
        bans = () if banned is None else [t for t in np.asarray(banned[b]).tolist() if t >= 0]
        for i in range(G1):
            row = target[b, i]
            if np.any(np.isnan(row) | (row == np.inf)):
                f |= FLAG_NONFINITE
            am[b, i] = greedy_argmax(row, bans)
        xs = [int(x) for x in draft_tokens[b]]
        if any(x < 0 or x >= V for x in xs):
            f |= FLAG_TOKEN_RANGE
        n = gamma
        for i in range(gamma):
            # a proposal outside [0, V) is no token of the row: it never
            # matches, not even the -1 "argmax" of a row with no admissible id
            if not 0 <= xs[i] < V or xs[i] != am[b, i]:
                n = i
                break
            tokens[b, i] = xs[i]
        tokens[b, n] = am[b, n]
        if am[b, n] < 0:
            f |= FLAG_EMPTY
        num_acc[b] = n
        flags[b] = f
    return GreedyResult(tokens, num_acc, flags, am)


def sampler_valid(s, allow_greedy):
    """Range check of one sampler setting (temperature 0 only where a greedy
    request is allowed)."""
    T, k, P = _f32(s.temperature), int(s.top_k), _f32(s.top_p)
    if not math.isfinite(T) or T < 0.0 or (T == 0.0 and not allow_greedy):
        return False
    return k >= 0 and 0.0 < P <= 1.0


def penalty_valid(theta):
    t = _f32(theta)
    return math.isfinite(t) and t >= 1.0


def verify_batch(target, draft, draft_tokens, uniforms, target_samplers, draft_samplers,
                 banned=None, banned_draft=None, gammas=None, history=None, penalties=None,
                 penalties_draft=None, dtype="f32"):
    """A mixed batch: per-request draft lengths, samplers and draft bans.

    target [B, gamma+1, V], draft [B, gamma, V], draft_tokens [B, gamma] and
    uniforms [B, gamma+1] as in verify_sample; target_samplers / draft_samplers
    are lists of B Samplers; banned [B, n] bans the target rows (and the draft
    rows unless banned_draft [B, m] is given, which then bans the draft rows);
    gammas [B] gives each request's number of proposals g_b <= gamma (None: all
    gamma). Request b uses target rows 0..g_b, draft rows 0..g_b-1, proposals
    0..g_b-1, acceptance uniforms u[b, 0..g_b-1] and the final-draw uniform
    u[b, gamma]. A target temperature of 0 makes the request greedy (its draft
    rows and uniforms are unused): the walk of verify_greedy with
    greedy_argmax. A draft length or sampler setting out of range gives flag
    FLAG_BAD_PARAM, no accepted proposal and no token. lse of rows a request
    does not use (and of every row of a greedy request) is NaN.

    Repetition penalties: history [B, H] (-1 = padding) holds each request's
    generated tokens before the round; penalties [B] / penalties_draft [B]
    are the target / draft factors theta >= 1 (None: 1 = off). Row i of a
    request penalizes its history and the proposals x_0 .. x_{i-1} that
    precede position i (the tokens its sampler had seen); `dtype` ("bf16" or
    "f32") is the logits' dtype, in which the penalized values are rounded.

    [ATLAS] "Implementation roadmap and tests" (continuous batching with
    per-request metadata); [ATLAS] "Greedy, sampling and the real sampler".
    """
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    draft_tokens = np.asarray(draft_tokens)
    uniforms = np.asarray(uniforms, dtype=np.float64)
    B, G1, V = target.shape
    gamma = G1 - 1
    tokens = np.full((B, G1), -1, dtype=np.int32)
    num_acc = np.zeros(B, dtype=np.int32)
    flags = np.zeros(B, dtype=np.uint32)
    tlse = np.full((B, G1), np.nan)
    dlse = np.full((B, gamma), np.nan)
    boundary = np.zeros(B, dtype=bool)
    acc_prob = np.full((B, gamma), np.nan)
    margin = np.full(B, math.inf)
    for b in range(B):
        gb = gamma if gammas is None else int(gammas[b])
        ts, ds = target_samplers[b], draft_samplers[b]
        greedy = _f32(ts.temperature) == 0.0
        th_t = 1.0 if penalties is None else float(penalties[b])
        th_d = 1.0 if penalties_draft is None else float(penalties_draft[b])
        if not (0 <= gb <= gamma) or not sampler_valid(ts, True) or not penalty_valid(th_t) or (
                not greedy and (not sampler_valid(ds, False) or not penalty_valid(th_d))):
            flags[b] = FLAG_BAD_PARAM
            continue
        hist = [] if history is None else [int(t) for t in np.asarray(history[b]).tolist() if t >= 0]
        tb = () if banned is None else [t for t in np.asarray(banned[b]).tolist() if t >= 0]
        db = tb if banned_draft is None else [t for t in np.asarray(banned_draft[b]).tolist()
                                              if t >= 0]
        xs = [int(x) for x in draft_tokens[b, :gb]]
        if greedy:
            # verify_greedy's walk over penalized argmaxes
            f = 0
            am = []
            for i in range(gb + 1):
                row = target[b, i]
                if np.any(np.isnan(row) | (row == np.inf)):
                    f |= FLAG_NONFINITE
                am.append(greedy_argmax(row, tb, hist + xs[:i], th_t, dtype))
            if any(x < 0 or x >= V for x in xs):
                f |= FLAG_TOKEN_RANGE
            n = gb
            for i in range(gb):
                if not 0 <= xs[i] < V or xs[i] != am[i]:
                    n = i
                    break
                tokens[b, i] = xs[i]
            tokens[b, n] = am[n]
            if am[n] < 0:
                f |= FLAG_EMPTY
            num_acc[b] = n
            flags[b] = f
            continue
        pt = [row_distribution(target[b, i], ts, tb, hist + xs[:i], th_t, dtype)
              for i in range(gb + 1)]
        qd = [row_distribution(draft[b, i], ds, db, hist + xs[:i], th_d, dtype) for i in range(gb)]
        f = 0
        mg = math.inf
        for d in pt + qd:
            if d.nonfinite:
                f |= FLAG_NONFINITE
            if d.empty:
                f |= FLAG_EMPTY
            mg = min(mg, d.topp_margin)
        tlse[b, :gb + 1] = [d.lse for d in pt]
        dlse[b, :gb] = [d.lse for d in qd]
        u = np.concatenate([uniforms[b, :gb], uniforms[b, gamma:gamma + 1]])
        out, n, fb, bmg, ap = verify_block([d.p for d in pt], [d.p for d in qd], xs, u)
        tokens[b, :gb + 1] = out
        num_acc[b] = n
        flags[b] = f | fb
        margin[b] = min(mg, bmg)
        boundary[b] = margin[b] <= BOUNDARY_EPS
        acc_prob[b, :gb] = ap
    return SampleResult(tokens, num_acc, flags, tlse, dlse, boundary, acc_prob, margin)


def first_token_law(p, q):
    """Exact law of the token emitted at one position, no uniforms involved.

    P(accept x) = q(x) * min(1, p(x)/q(x)) = min(p(x), q(x)); rejection has
    probability 1 - alpha with alpha = sum_x min(p, q), after which the residual
    norm(max(0, p - q)) is drawn ([DRAFT] "Sampling needs a correction rule").
    Returns (law, alpha, residual).
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    accepted = np.minimum(p, q)
    alpha = accepted.sum()
    pos = np.maximum(p - q, 0.0)
    residual = pos / pos.sum() if pos.sum() > 0 else np.zeros_like(p)
    return accepted + (1.0 - alpha) * residual, alpha, residual
