"""Chain KV-commit metadata after one verification round, CPU oracle.

TEST INFRASTRUCTURE, like the rest of this package: only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may use it.

Pages followed (cited by title and section):
  [ATLAS] "Speculative Decoding - Turn guesses into parallel work",
          "Committed tokens versus cached states" (the logical token list and
          the processed KV length differ; a sampled correction or bonus is
          committed before its KV row exists; the convention must be stated).
  [DRAFT] "Drafters and Speculative Decoding: Useful Tokens, Correct State",
          "Committing state after rejection" (the running example: rows
          through the accepted prefix are kept, the rejected suffix becomes
          invalid, the correction stays a pending anchor).

Convention (one request, chain verification):
  before the round  kv_len = K materialised target KV rows; the last
                    committed token (the anchor) is pending, i.e. has no row;
  the target pass   ran the gamma+1 inputs (anchor, x_0, ..., x_{gamma-1}) at
                    positions K .. K+gamma and wrote scratch rows there;
                    slots[j] is the physical KV slot of position K + j;
  after             the anchor's row and the n accepted proposals' rows are
                    committed history: new_kv_len = K + 1 + n; the emitted
                    token tokens[n] (correction or bonus) is the new pending
                    anchor; the rows of x_n .. x_{gamma-1} (positions
                    K+n+1 .. K+gamma) are invalid and their slots are freed,
                    in position order, -1 after them. The logical length
                    (committed tokens) is new_kv_len + 1.

Parity status: pinned by the running example of [DRAFT] "Committing state
after rejection" (tests/golden/commit_example.json) and by the invariants
checked in tests/test_oracle_commit.py (rows kept plus rows freed equal the
rows written; nothing is freed when every proposal survives).
"""

import numpy as np


def commit_chain(tokens, num_accepted, kv_len, slots=None, gammas=None):
    """Per-request commit metadata of one chain verification round.

    tokens [B, gamma+1] and num_accepted [B] as the verifier returns them,
    kv_len [B] materialised rows before the round, slots [B, gamma+1] or None,
    gammas [B] proposals of each request (None: all gamma; the pass then wrote
    rows at positions K .. K+gammas[b] only). Returns (new_kv_len [B], anchor
    [B], n_free [B], free_slots [B, gamma] or None).
    """
    tokens = np.asarray(tokens)
    num_accepted = np.asarray(num_accepted)
    kv_len = np.asarray(kv_len)
    B, G1 = tokens.shape
    gamma = G1 - 1
    new_kv_len = np.zeros(B, dtype=np.int64)
    anchor = np.zeros(B, dtype=np.int64)
    n_free = np.zeros(B, dtype=np.int64)
    free = None if slots is None else np.full((B, gamma), -1, dtype=np.int64)
    for b in range(B):
        n = int(num_accepted[b])
        g = gamma if gammas is None else int(gammas[b])
        if not (0 <= g <= gamma and 0 <= n <= g):
            # not a verifier output: nothing committed, nothing freed
            new_kv_len[b] = int(kv_len[b])
            anchor[b] = -1
            continue
        new_kv_len[b] = int(kv_len[b]) + 1 + n        # anchor row + accepted rows
        anchor[b] = int(tokens[b, n])                  # correction or bonus, pending
        n_free[b] = g - n                              # rows of the rejected proposals
        if free is not None:
            for j in range(n + 1, g + 1):              # positions K+n+1 .. K+g
                free[b, j - (n + 1)] = int(slots[b][j])
    return new_kv_len, anchor, n_free, free
