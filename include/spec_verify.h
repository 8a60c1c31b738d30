/*
 * spec_verify.h - C interface of a lossless speculative-sampling verifier for
 * AMD MI355X (gfx950).
 *
 * The operation is one verification round of speculative decoding for a batch
 * of B independent requests:
 *   - "Speculative Decoding - Turn guesses into parallel work", section "One
 *     round and shifted logits": the drafter proposes gamma tokens together with
 *     their proposal distributions q; one target pass yields gamma+1 target
 *     distributions p (row i judges proposal i, row gamma serves the bonus token).
 *   - same page, section "Exact sampling: account for every probability", and
 *     "Speculative Token Decoupling ..." Equation 3.1: proposal i is accepted with
 *     probability min(1, p_i(x_i) / q_i(x_i)); here: accept iff u_i * q_i(x_i) <=
 *     p_i(x_i) with u_i uniform on (0, 1].
 *   - "Drafters and Speculative Decoding: Useful Tokens, Correct State", section
 *     "Sampling needs a correction rule": at the first rejection the replacement
 *     is drawn from norm(max(0, p - q)); every later proposal is discarded.
 *   - "Speculative Decoding" (specdec fundamentals), section "The Loop": if all
 *     gamma proposals survive, one bonus token is drawn from p_gamma; every round
 *     emits between 1 and gamma+1 tokens.
 *   - "Speculative Decoding - Turn guesses into parallel work", section "Greedy,
 *     sampling and the real sampler": temperature, truncation and token bans are
 *     part of p and q, and the greedy variant accepts while the proposal equals
 *     the target argmax ("Drafters and Speculative Decoding", section "Greedy
 *     verification").
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is caller-owned memory. Logits, tokens, outputs and
 *     workspace are DEVICE pointers on the current HIP device; sampler structs
 *     are passed by value. The library allocates no device memory, frees
 *     nothing, and keeps no pointer after returning.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream)
 *     and never synchronise. Outputs are valid once the stream has reached the
 *     call. Outputs must not alias inputs; concurrent calls need distinct
 *     outputs and workspaces.
 *   - Argument errors are detected on the host before anything is launched and
 *     return a negative SV_E* code; nothing is written in that case. Problems
 *     that can only be seen in the data are reported per request through the
 *     SV_FLAG_* bits of out_flags.
 *   - Logit rows are contiguous with row stride V elements. A logit of -inf
 *     marks a token as impossible. NaN and +inf are data errors (flag
 *     SV_FLAG_NONFINITE); the tokens of such a request are unspecified.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Sampler settings of one distribution (target or draft may differ).
 *   temperature: > 0 and finite; logits are divided by it.
 *   top_k:       0 = off; otherwise keep every token whose logit is >= the
 *                k-th largest admissible logit (ties kept, so more than k
 *                tokens may survive). k >= number of admissible tokens is off.
 *   top_p:       1.0 = off; otherwise in (0, 1): keep token x when the tempered
 *                probability mass of tokens with a strictly larger logit is
 *                < top_p (the crossing token and its exact ties are kept).
 * Order of transforms: bans, temperature, top-k, top-p, renormalise. */
typedef struct {
  float temperature;
  int32_t top_k;
  float top_p;
} sv_sampler;

/* Return codes. */
#define SV_OK 0
#define SV_EINVAL (-1)     /* null required pointer, bad size or sampler field */
#define SV_EDTYPE (-2)     /* dtype not SV_F32 / SV_BF16 */
#define SV_EWORKSPACE (-3) /* workspace NULL or smaller than spec_verify_workspace_bytes */
#define SV_ESIZE (-4)      /* sizes overflow the supported index ranges */
#define SV_EHIP (-5)       /* a HIP launch or runtime call failed */
#define SV_ESCRATCH (-6)   /* spec_verify_sample_noalloc: the sizes need more workspace
                              than SV_NOALLOC_SCRATCH_BYTES */

/* Per-request flag bits written to out_flags. */
#define SV_FLAG_TOKEN_RANGE 1u    /* some draft token lies outside [0, V) */
#define SV_FLAG_Q_ZERO 2u         /* the proposal that ended the walk has q(x) = 0 */
#define SV_FLAG_NONFINITE 4u      /* NaN or +inf in one of the request's rows */
#define SV_FLAG_EMPTY 8u          /* a row has no admissible token; see out_tokens */
#define SV_FLAG_RESIDUAL_ZERO 16u /* residual mass was 0 at a rejection; drawn from p */
#define SV_FLAG_BAD_PARAM 32u     /* a per-request setting of sv_requests is out of range */

/* Largest n_banned (and sv_requests.n_banned_draft) accepted. */
#define SV_MAX_BANNED 2048
/* Largest sv_requests.n_history accepted. A row penalizes at most
 * SV_MAX_HISTORY + 63 distinct ids (its history and the proposals before it);
 * the kernels keep them in an on-chip hash set of 4096 slots that this bound
 * keeps at most half full. */
#define SV_MAX_HISTORY 1984

/* Per-request settings of a mixed batch ("Speculative Decoding - Turn guesses
 * into parallel work", section "Implementation roadmap and tests": continuous
 * batching keeps per-request metadata on the GPU). Every array is DEVICE
 * memory of B entries (banned_draft: B rows of n_banned_draft); a NULL array
 * keeps the call-wide value. Passed to spec_verify_sample by host pointer.
 *   gamma         proposals of each request, 0 <= gamma[b] <= gamma: request b
 *                 uses target rows 0..gamma[b], draft rows and draft tokens
 *                 0..gamma[b]-1, acceptance uniforms (slots) 0..gamma[b]-1 and
 *                 the final-draw uniform of slot gamma; its out_tokens row has
 *                 at most gamma[b]+1 tokens.
 *   target        target sampler of each request. Temperature 0 makes the
 *                 request greedy: proposals are kept while they equal the
 *                 argmax of their target row (banned_ids applied, NaN excluded,
 *                 lowest id on ties), as in spec_verify_greedy; its draft rows
 *                 and uniforms are not read.
 *   draft         draft sampler of each request (ignored for greedy requests).
 *   banned_draft  [B][n_banned_draft] bans of the draft rows; banned_ids then
 *                 applies to the target rows only (same list rules).
 *   history       [B][n_history] tokens each request generated before this
 *                 round (-1 or ids outside [0, V) are padding), for the
 *                 repetition penalty; n_history <= SV_MAX_HISTORY.
 *   penalty       [B] repetition penalty theta >= 1 of the target rows (1:
 *                 off); penalty_draft [B] likewise for the draft rows. Row i
 *                 of a request penalizes its history and the proposals
 *                 x_0 .. x_{i-1} before position i (the tokens its sampler had
 *                 seen), each id once, banned ids excepted: a logit z becomes
 *                 z / theta if z > 0, else z * theta (Keskar et al. 2019,
 *                 "CTRL", section 4.1, sign-aware form), computed in float32
 *                 and rounded to bf16 for bf16 logits; the penalty comes after
 *                 the bans and before temperature and truncation.
 * A request whose gamma[b], sampler fields or penalties are out of range (the
 * ranges of sv_sampler; temperature 0 only as a target; a penalty below 1 or
 * not finite) is not verified: flag
 * SV_FLAG_BAD_PARAM, no accepted proposal, out_tokens row all -1. Rows a
 * request does not use report NaN in out_target_lse / out_draft_lse, and so
 * do the rows of greedy requests; out_overlap is NaN at positions a request
 * does not have and for greedy requests. */
typedef struct {
  const int32_t* gamma;
  const sv_sampler* target;
  const sv_sampler* draft;
  const int32_t* banned_draft;
  int32_t n_banned_draft;
  const int32_t* history;
  int32_t n_history;
  const float* penalty;
  const float* penalty_draft;
} sv_requests;

/* Workspace bytes needed by spec_verify_sample for these sizes (0 when B < 1,
 * gamma outside [1, 63], V < 1 or the sizes overflow the supported index
 * ranges). The workspace needs no initialisation and may be reused by later
 * calls on the same stream; calls that run concurrently need separate
 * workspaces. */
size_t spec_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t V);

/* Speculative-sampling verification.
 *   target_logits  [B][gamma+1][V] of dtype; row i is the target distribution
 *                  after the prefix and proposals 0..i-1, row gamma the bonus row.
 *   draft_logits   [B][gamma][V] of dtype; row i is the distribution proposal i
 *                  was sampled from (it must be the distribution that actually
 *                  produced the token, after the drafter's own transforms).
 *   draft_tokens   [B][gamma] int32 proposals.
 *   banned_ids     [B][n_banned] int32 token ids removed from p AND q of every
 *                  row of the request; -1 or any id outside [0, V) is padding;
 *                  duplicates are allowed. NULL only when n_banned == 0.
 *   target, draft  sampler settings for p and q respectively.
 *   requests       per-request settings of a mixed batch (sv_requests above),
 *                  or NULL for a batch that shares gamma, samplers and bans.
 *   seed, offset   select the uniforms when `uniforms` is NULL: for request b
 *                  and slot j (j < gamma: acceptance of proposal j; j == gamma:
 *                  the single final draw) u = ((r >> 11) + 1) * 2^-53 with r the
 *                  first output word of Philox4x64-10 at counter (j, b, offset, 0)
 *                  and key (seed, 0) (Salmon et al., SC'11).
 *   uniforms       [B][gamma+1] double in (0, 1] used instead of Philox, or NULL.
 * Outputs:
 *   out_tokens       [B][gamma+1] int32: the n accepted proposals, then the
 *                    correction (n < gamma) or bonus (n == gamma) token, then -1
 *                    padding. The emitted token is -1 when the distribution it
 *                    must be drawn from is empty (SV_FLAG_EMPTY).
 *   out_num_accepted [B] int32 n in [0, gamma].
 *   out_flags        [B] uint32 SV_FLAG_* bits, or NULL.
 *   out_target_lse   [B][gamma+1] float log-normaliser of each tempered target
 *                    row over its kept set (-inf if empty), or NULL.
 *   out_draft_lse    [B][gamma] float, same for the draft rows, or NULL.
 *   out_overlap      [B][gamma] double, or NULL (then not computed): the overlap
 *                    sum_x min(p_i(x), q_i(x)) = 1 - TV(p_i, q_i) of target row
 *                    i and draft row i after every sampler transform; with x_i
 *                    drawn from q_i it is the probability that proposal i is
 *                    accepted once the walk reaches it ("Speculative
 *                    Decoding - Turn guesses into parallel work", sections
 *                    "Confidence and verification admission" and "Accepted
 *                    length is not speed"). 0 when either row is empty; unspecified for a
 *                    request flagged SV_FLAG_NONFINITE. Computing it reads the
 *                    rows 0..gamma-1 once more (only the kept groups of the
 *                    other row when one of the two is truncated).
 *   out_accept_hist  [gamma+1] uint32, or NULL: out_accept_hist[n] = number of
 *                    requests of this call with n accepted proposals (an
 *                    accepted-prefix histogram, same page, section "Read the
 *                    benchmark contract"). Overwritten by each call. Requests
 *                    that reached position i number sum_{n >= i} hist[n], and
 *                    sum_{n > i} hist[n] of them accepted it.
 *   workspace        device scratch of at least spec_verify_workspace_bytes(...)
 *                    bytes, 256-byte aligned.
 * Limits: 1 <= B, 1 <= gamma <= 63, 1 <= V < 2^31, B*(2*gamma+1) < 2^31,
 * n_banned <= SV_MAX_BANNED; logit pointers aligned to their element size. */
int spec_verify_sample(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                       const int32_t* draft_tokens, const int32_t* banned_ids,
                       int32_t n_banned, int32_t B, int32_t gamma, int32_t V,
                       sv_sampler target, sv_sampler draft, const sv_requests* requests,
                       uint64_t seed, uint64_t offset,
                       const double* uniforms, int32_t* out_tokens, int32_t* out_num_accepted,
                       uint32_t* out_flags, float* out_target_lse, float* out_draft_lse,
                       double* out_overlap, uint32_t* out_accept_hist,
                       void* workspace, size_t workspace_bytes, void* stream);

/* spec_verify_sample without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Arguments, outputs and errors are those of
 * spec_verify_sample; the workspace is a static device array of
 * SV_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held until
 * the process ends. The call allocates nothing. When
 * spec_verify_workspace_bytes exceeds SV_NOALLOC_SCRATCH_BYTES, the call runs
 * without the final draw's lists of kept tokens (the last part of that size:
 * 388 bytes per request and 2048-token sub-chunk), with the same outputs;
 * sizes whose remaining workspace still exceeds the array return SV_ESCRATCH
 * (c5-sized batches, B = 128, gamma = 8, V = 151936, need about 4.0 MB with
 * the lists and 0.3 MB without). The first call on a device resolves that
 * device's array address (SV_EHIP if it cannot). Every call on one GPU shares its array: calls that
 * may overlap on one GPU (different streams, or different host threads)
 * race and must be serialised by the caller; calls in order on one stream are
 * safe. Nothing needs clearing: every call initialises what it reads. */
#define SV_NOALLOC_SCRATCH_BYTES (8u << 20)
int spec_verify_sample_noalloc(const void* target_logits, const void* draft_logits,
                               sv_dtype dtype, const int32_t* draft_tokens,
                               const int32_t* banned_ids, int32_t n_banned, int32_t B,
                               int32_t gamma, int32_t V, sv_sampler target, sv_sampler draft,
                               const sv_requests* requests, uint64_t seed, uint64_t offset,
                               const double* uniforms, int32_t* out_tokens,
                               int32_t* out_num_accepted, uint32_t* out_flags,
                               float* out_target_lse, float* out_draft_lse, double* out_overlap,
                               uint32_t* out_accept_hist, void* stream);

/* Greedy verification ("Drafters and Speculative Decoding", section "Greedy
 * verification"): proposal i is kept while it equals the argmax of target row i
 * (largest logit, lowest token id on exact ties, -0 == +0); the first mismatch
 * emits that row's argmax, and if all gamma match the argmax of row gamma is
 * appended. Needs no workspace: out_tokens doubles as scratch.
 *   target_logits [B][gamma+1][V], draft_tokens [B][gamma];
 *   banned_ids [B][n_banned] ids that are never an argmax (the sampler's bans
 *   are part of greedy decoding too: "Speculative Decoding - Turn guesses into
 *   parallel work", section "Greedy, sampling and the real sampler"); same list
 *   rules as for spec_verify_sample; NULL only when n_banned == 0;
 *   out_tokens [B][gamma+1] (n matches, argmax, then -1), out_num_accepted [B],
 *   out_flags [B] or NULL (SV_FLAG_TOKEN_RANGE, SV_FLAG_NONFINITE, and
 *   SV_FLAG_EMPTY when the emitted token's row has no admissible id: that token
 *   is then -1),
 *   out_accept_hist [gamma+1] or NULL: accepted-prefix histogram of the call,
 *   as for spec_verify_sample.
 * NaN logits are not candidates and are flagged; a row whose admissible
 * logits are all -inf has the lowest such id as its argmax. */
int spec_verify_greedy(const void* target_logits, sv_dtype dtype, const int32_t* draft_tokens,
                       const int32_t* banned_ids, int32_t n_banned,
                       int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens,
                       int32_t* out_num_accepted, uint32_t* out_flags,
                       uint32_t* out_accept_hist, void* stream);

/* Chain KV-commit metadata of one verification round ("Speculative Decoding -
 * Turn guesses into parallel work", section "Committed tokens versus cached
 * states"; "Drafters and Speculative Decoding: Useful Tokens, Correct State",
 * section "Committing state after rejection"), from the outputs of
 * spec_verify_sample or spec_verify_greedy, on the same stream.
 * gamma_b [B] (device) gives each request's number of proposals as in
 * sv_requests (NULL: all gamma); below, gamma stands for gamma_b[b].
 * Convention: before the round request b has kv_len[b] = K materialised target
 * KV rows, and its last committed token (the anchor) is pending: it has no row
 * yet. The verification pass ran the gamma+1 inputs (anchor, x_0, ...,
 * x_{gamma-1}) at positions K .. K+gamma and wrote their rows; slots[b][j] is
 * the physical KV slot of position K + j. After the round:
 *   new_kv_len[b] = K + 1 + n   the anchor's row and the n accepted rows are
 *                               committed history (logical length = new_kv_len + 1);
 *   anchor[b] = out_tokens[b][n]  the correction or bonus token, pending until
 *                               the next pass computes its row (-1 if the
 *                               verifier emitted none, see SV_FLAG_EMPTY);
 *   n_free[b] = gamma - n       rows of the rejected proposals x_n .. x_{gamma-1};
 *   free_slots[b][0 .. gamma-n-1] = slots[b][n+1 .. gamma], then -1.
 * Pointers: out_tokens [B][gamma+1], out_num_accepted [B], kv_len [B] (inputs,
 * device); new_kv_len [B], anchor [B] (required outputs); n_free [B] or NULL;
 * free_slots [B][gamma] or NULL, which needs slots [B][gamma+1]. A request
 * whose accepted count lies outside [0, gamma_b[b]], or whose gamma_b[b] lies
 * outside [0, gamma], is left unchanged (new_kv_len =
 * kv_len, anchor -1, nothing freed). The caller keeps kv_len + gamma + 1 within
 * int32. Returns SV_EINVAL for a missing required pointer, free_slots without
 * slots, B < 1 or gamma outside [1, 63]; SV_ESIZE if B*(gamma+1) overflows. */
int spec_verify_commit(const int32_t* out_tokens, const int32_t* out_num_accepted,
                       const int32_t* kv_len, const int32_t* slots, const int32_t* gamma_b,
                       int32_t B, int32_t gamma,
                       int32_t* new_kv_len, int32_t* anchor, int32_t* n_free,
                       int32_t* free_slots, void* stream);

/* Static description of a status code. */
const char* spec_verify_strerror(int status);


#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
