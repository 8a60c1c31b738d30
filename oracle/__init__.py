"""Float64 CPU oracle of the speculative-sampling verifier.

TEST INFRASTRUCTURE, not product code: only tests/, __graft_entry__.smoke()
and bench.py's cpu_baseline leg may import, call or execute it. It shares no
code with the HIP library or its binding, and imports nothing from them.

Parity status of each function (what pins it to something other than itself):
  philox4x64_10      pinned: NumPy's independent Philox implementation.
  row_distribution   pinned: brute-force threshold search on small rows,
                     math.fsum normaliser, top_k=1 == argmax.
  verify_sample      pinned: three-token worked example of "Drafters and
                     Speculative Decoding" (rejection mass 0.40, residual
                     0.75/0.25/0, final law = p); alpha = 0.8 invariants;
                     closed form (1 - a^(g+1)) / (1 - a) and the survival form by
                     Monte Carlo; chi-square of emitted tokens against p.
  verify_greedy      pinned: brute-force loop over small rows (bans included).
  repetition_penalty pinned: theta = 1 is the identity, sign handling, never
                     raises a logit, bf16 results are bf16 values (round_to_bf16
                     against the bit-level definition and NumPy), and sampled
                     outputs follow the penalized p.
  verify_batch       pinned: each request equals the same request verified
                     alone by verify_sample / verify_greedy on its own rows;
                     a request with g_b proposals equals a gamma = g_b batch.
  first_token_law    pinned: the worked example's printed numbers.
  commit_chain       pinned: the running example of "Committing state after
                     rejection" (tests/golden/commit_example.json) and the
                     row-partition invariants.
  diagnostics        per-position overlap 1 - TV, accepted-prefix histogram,
                     conditional acceptance, accepted-length law; each pin is
                     listed in oracle/diagnostics.py.
Parity unpinned (fixed by convention only, not by anything the pages print):
the uniform layout, the tie rules of top-k, top-p and greedy, and the actual
numbers of the alpha = 0.8 example (only its invariants are printed).
"""

from . import commit, diagnostics  # noqa: F401
from .commit import commit_chain  # noqa: F401
from .diagnostics import (  # noqa: F401
    accepted_prefix_histogram,
    conditional_acceptance,
    overlap,
    position_overlaps,
    prefix_length_law,
)
from .philox import philox4x64_10, uniform, uniforms, word_to_uniform  # noqa: F401
from .verifier import (  # noqa: F401
    BOUNDARY_EPS,
    FLAG_BAD_PARAM,
    FLAG_EMPTY,
    FLAG_NONFINITE,
    FLAG_Q_ZERO,
    FLAG_RESIDUAL_ZERO,
    FLAG_TOKEN_RANGE,
    GreedyResult,
    RowDist,
    SampleResult,
    Sampler,
    accept,
    first_token_law,
    greedy_argmax,
    repetition_penalty,
    residual_weights,
    round_to_bf16,
    row_distribution,
    sample_categorical,
    penalty_valid,
    sampler_valid,
    verify_batch,
    verify_block,
    verify_greedy,
    verify_sample,
)
