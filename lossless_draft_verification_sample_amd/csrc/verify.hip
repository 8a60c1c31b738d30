// Acceptance walk and final draw of spec_verify_sample, in one kernel.
//
// Acceptance ("Speculative Decoding - Turn guesses into parallel work", section
// "Exact sampling: account for every probability"; "Speculative Token
// Decoupling ..." Equation 3.1): proposal i of a request is accepted iff
// u_i * q_i(x_i) <= p_i(x_i), walking left to right and stopping at the first
// rejection. p_i(x_i) and q_i(x_i) come from the row statistics pass, which
// evaluates them in fp64 next to each row's normaliser.
//
// Final draw ("Drafters and Speculative Decoding: Useful Tokens, Correct State",
// section "Sampling needs a correction rule"; "Speculative Decoding"
// fundamentals, section "The Loop"): at the first rejection n the token is
// drawn from norm(max(0, p_n - q_n)); if every proposal survived it is drawn
// from p_gamma. The draw is an inverse CDF in ascending token order: the
// smallest x whose running weight sum reaches u * S. Only the one (or two)
// selected rows per request are read again.
//
// Work split: each request gets `nwg` workgroups, each owning `spw` consecutive
// sub-chunks of DRAW_SUB tokens. Every workgroup repeats the (tiny) acceptance
// walk to learn n, sums the draw weights of its sub-chunks and publishes them
// (at a truncated target row of a plain batch, with a list of each sub-chunk's
// weighted tokens when it has at most DRAW_LIST); the last workgroup of the
// request to finish (an arrival counter) locates the sub-chunk holding u * S,
// picks the token from its list or rescans it, and writes the outputs.

#include <climits>
#include <type_traits>

#include "sv_launch.hpp"
#include "sv_rowio.hpp"

namespace sv {

constexpr int DR_THREADS = 256;
constexpr int DR_NW = DR_THREADS / WAVE;
static_assert(DR_NW == DRAW_WAVES, "the host sizes dense draw splits by this");
// bf16 rows are read with nontemporal loads (measured faster in this kernel;
// fp32 rows, slower)
template <typename Elem>
constexpr bool DR_NT = sizeof(Elem) == 2;
constexpr int GPL = DRAW_SUB / GRP / WAVE;   // groups per lane when a wave owns a sub-chunk
static_assert(DRAW_SUB == DR_THREADS * GRP, "one group of GRP logits per thread per sub-chunk");

struct DrawRow {
  const void* trow;
  const void* drow;   // nullptr for the bonus draw
  RowStat ts, ds;
  double tinv, dinv;  // 1/T of both rows
  float tcut;         // no target token below this is kept (+inf: empty row)
};

// The rows of the final draw of request b after n acceptances: the target row
// n, and the draft row n at a rejection (n < the request's draft length g).
// Their statistics come from the acceptance walk, which has loaded them.
__device__ __forceinline__ DrawRow draw_row(const DrawArgs& a, int b, int n, const ReqInfo& rq,
                                            const RowStat& ts, const RowStat& ds) {
  const int g = a.gamma, G1 = g + 1;
  DrawRow r;
  const int64_t V = a.V;
  const size_t es = a.bf16 ? 2 : 4;
  r.trow = (const char*)a.target + ((int64_t)b * G1 + n) * V * es;
  r.ts = ts;
  r.tinv = 1.0 / (double)rq.st.temperature;
  r.tcut = (r.ts.flags & FLAG_EMPTY) ? INFINITY : r.ts.tau;
  if (n < rq.g) {
    r.drow = (const char*)a.draft + ((int64_t)b * g + n) * V * es;
    r.ds = ds;
    r.dinv = 1.0 / (double)rq.sd.temperature;
  } else {
    r.drow = nullptr;
  }
  return r;
}

// p(x) of a token whose target logit zt is kept.
__device__ __forceinline__ double tok_p(const DrawRow& r, float zt, const double* tab) {
  return exp_tab(fma((double)zt, r.tinv, -r.ts.lse), tab);
}

// Draw weight of one token whose target logit zt is kept: w(x) = max(0, p - q)
// at a rejection, p for the bonus draw. (Skipping the exps where the draft's
// log-probability is at least the target's saves nothing: some lane of the
// wave needs them.)
__device__ __forceinline__ double tok_w(const DrawRow& r, float zt, float zd, const double* tab) {
  const double p = exp_tab(fma((double)zt, r.tinv, -r.ts.lse), tab);
  if (!r.drow) return p;
  // zd belongs to a token that is not banned (its target logit is kept)
  const double q = is_kept(zd, r.ds, false) ? exp_tab(fma((double)zd, r.dinv, -r.ds.lse), tab)
                                            : 0.0;
  return p > q ? p - q : 0.0;
}

// Bit e set when token e of the group is kept in the target row; only those
// tokens have p > 0, hence w > 0. `banned` holds one bit per token.
template <typename Elem>
__device__ __forceinline__ uint32_t kept_mask(const DrawRow& r, const Group<Elem>& tg,
                                              uint32_t banned) {
  uint32_t m = 0u;
#pragma unroll
  for (int e = 0; e < GRP; ++e)
    m |= (is_kept(group_val<Elem>(tg, e), r.ts, (banned >> e) & 1u) ? 1u : 0u) << e;
  return m;
}

// Sum of w over the kept tokens of a group.
template <typename Elem>
__device__ __forceinline__ double group_wsum(const DrawRow& r, const Group<Elem>& tg,
                                             const Group<Elem>& dg, uint32_t km, const double* tab) {
  double sw = 0.0;
#pragma unroll
  for (int e = 0; e < GRP; ++e)
    if ((km >> e) & 1u) sw += tok_w(r, group_val<Elem>(tg, e), r.drow ? group_val<Elem>(dg, e) : 0.0f, tab);
  return sw;
}

// Sum of p over the kept tokens of a group.
template <typename Elem>
__device__ __forceinline__ double group_psum(const DrawRow& r, const Group<Elem>& tg, uint32_t km,
                                             const double* tab) {
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < GRP; ++e)
    if ((km >> e) & 1u) s += tok_p(r, group_val<Elem>(tg, e), tab);
  return s;
}

// Per-token draw weights of a group: w, or p when `use_p` (0 outside the mask).
template <typename Elem>
__device__ __forceinline__ void group_values(const DrawRow& r, const Group<Elem>& tg,
                                             const Group<Elem>& dg, uint32_t km, const double* tab,
                                             bool use_p, double (&v)[GRP]) {
#pragma unroll
  for (int e = 0; e < GRP; ++e) {
    v[e] = 0.0;
    if ((km >> e) & 1u)
      v[e] = use_p ? tok_p(r, group_val<Elem>(tg, e), tab)
                   : tok_w(r, group_val<Elem>(tg, e), r.drow ? group_val<Elem>(dg, e) : 0.0f, tab);
  }
}

// Outcome of the acceptance walk of one request, computed by every wave.
struct Walk {
  int n;           // accepted proposals; the final token goes to slot n
  uint32_t flags;
  double u_final;  // uniform of the final draw
  int32_t x;       // proposal of this lane (lanes < gamma)
  RowStat ts, ds;  // statistics of target row n and draft row n (the draw's rows)
};

// Lane `src`'s RowStat (src wave-uniform), in scalar registers.
__device__ __forceinline__ RowStat rowstat_from_lane(const RowStat& v, int src) {
  RowStat r;
  r.m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.m), src));
  r.tau = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v.tau), src));
  r.lse = readlane_f64(v.lse, src);
  r.flags = (uint32_t)__builtin_amdgcn_readlane((int)v.flags, src);
  r.path = (uint32_t)__builtin_amdgcn_readlane((int)v.path, src);
  r.px = readlane_f64(v.px, src);
  return r;
}

// gq: the request's draft length (proposals 0..gq-1 and target rows 0..gq are
// its own); the final-draw uniform is slot gamma whatever gq is.
__device__ __forceinline__ Walk accept_walk(const DrawArgs& a, int b, int gq) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int g = a.gamma, G1 = g + 1, RPR = 2 * g + 1;
  const RowStat* st = a.stats + (int64_t)b * RPR;
  uint32_t rf = 0u;
  double p = 0.0, q = 0.0, u = 0.0;
  int32_t x = -1;
  RowStat t{}, d{};
  // loads for every position of the call (all in range), so that they need
  // not wait for a mixed batch's per-request draft length; then masked by it
  if (lane <= g) {
    u = a.uniforms[(int64_t)b * G1 + lane];
    t = st[lane];
  }
  if (lane < g) {
    d = st[G1 + lane];
    x = a.draft_tokens[(int64_t)b * g + lane];
  }
  if (lane <= gq) {
    rf |= t.flags;
    p = t.px;
  }
  if (lane < gq) {
    rf |= d.flags;
    q = d.px;
  } else {
    x = -1;
  }
  rf &= FLAG_NONFINITE | FLAG_EMPTY;
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) rf |= __shfl_xor(rf, off, WAVE);
  const bool range = lane < gq && (x < 0 || x >= a.V);
  const bool qzero = lane < gq && !range && !(q > 0.0);
  const bool acc = lane < gq && !range && !qzero && u * q <= p;
  const uint64_t accm = __ballot(acc);
  const uint64_t rangem = __ballot(range);
  const uint64_t qzm = __ballot(qzero);
  Walk w;
  w.n = __ffsll((unsigned long long)~accm) - 1;   // lane gq never accepts: n <= gq
  w.flags = rf;
  if (rangem) w.flags |= FLAG_TOKEN_RANGE;
  if (w.n < gq && ((qzm >> w.n) & 1ull)) w.flags |= FLAG_Q_ZERO;
  w.u_final = readlane_f64(u, g);
  w.x = x;
  w.ts = rowstat_from_lane(t, w.n);
  w.ds = rowstat_from_lane(d, w.n);
  return w;
}

constexpr int DR_QCAP = 4 * WAVE;   // queued kept tokens per wave: one batch of 4 reads per lane
static_assert(DRAW_LIST <= WAVE, "a sub-chunk's list is read by one wave, one entry per lane");

// A listed token of the selected sub-chunk, placed in token order.
struct ListTok {
  int32_t x;
  int32_t pad;
  double w;
};

struct DrawShared {
  double etab[256];
  union {
    KeptTok kt[DR_NW][WAVE];          // bonus draws and untruncated targets
    QueuedTok q[DR_NW][DR_QCAP];      // rejections at a truncated target
    ListTok lt[DRAW_LIST];            // the selection's list, after the stream
  };
  uint32_t bm[DRAW_SPW_MAX * DRAW_SUB / 32];
  uint32_t bmd[DRAW_SPW_MAX * DRAW_SUB / 32];   // draft-only bans (mixed batches)
  uint32_t bmp[DRAW_SPW_MAX * DRAW_SUB / 32];   // repetition-penalized ids (mixed batches)
  double scr[2 * DR_NW];
  int32_t iscr[2 * DR_NW];
  int32_t last;
  int32_t sel_sub, sel_x;
  double sel_before;
};

// Outputs of a request of a mixed batch that needs no draw, written by one
// wave: a request with settings out of range (nothing accepted, no token), or
// a greedy request (the walk of greedy verification over the argmaxes that
// the row pass left in the target rows' RowStat).
__device__ __forceinline__ void finish_without_draw(const DrawArgs& a, int b, const ReqInfo& rq) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int g = a.gamma, G1 = g + 1, RPR = 2 * g + 1;
  int32_t* ot = a.out_tokens + (int64_t)b * G1;
  if (rq.bad) {
    if (lane < G1) ot[lane] = -1;
    if (lane == 0) {
      a.out_num_accepted[b] = 0;
      if (a.out_flags) a.out_flags[b] = FLAG_BAD_PARAM;
      if (a.accept_hist) atomicAdd(&a.accept_hist[0], 1u);
    }
    return;
  }
  const RowStat* st = a.stats + (int64_t)b * RPR;
  uint32_t rf = 0u;
  int32_t am = -1, x = -1;
  bool match = false;
  if (lane <= rq.g) {
    const RowStat t = st[lane];
    rf = t.flags & FLAG_NONFINITE;
    am = (int32_t)t.path;
    match = t.px == 1.0;
  }
  if (lane < rq.g) x = a.draft_tokens[(int64_t)b * g + lane];
  const bool range = lane < rq.g && (x < 0 || x >= a.V);
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) rf |= __shfl_xor(rf, off, WAVE);
  const uint64_t mm = __ballot(lane < rq.g && match && !range);
  const int n = __ffsll((unsigned long long)~mm) - 1;   // <= rq.g
  uint32_t flags = rf;
  if (__ballot(range)) flags |= FLAG_TOKEN_RANGE;
  const int32_t token = __shfl(am, n, WAVE);
  if (token < 0) flags |= FLAG_EMPTY;
  if (lane < G1) ot[lane] = lane < n ? x : (lane == n ? token : -1);
  if (lane == 0) {
    a.out_num_accepted[b] = n;
    if (a.out_flags) a.out_flags[b] = flags;
    if (a.accept_hist) atomicAdd(&a.accept_hist[n], 1u);
  }
}

// Sets the logits of the banned tokens of a group (bit e: token e) to -inf.
template <typename Elem>
__device__ __forceinline__ void mask_group(Group<Elem>& g, uint32_t bits) {
  if (!bits) return;
#pragma unroll
  for (int e = 0; e < GRP; ++e) {
    if ((bits >> e) & 1u) {
      if constexpr (sizeof(Elem) == 2) {
        const int sh = 16 * (e & 1);
        g.w[0][e >> 1] = (g.w[0][e >> 1] & ~(0xFFFFu << sh)) | (0xFF80u << sh);
      } else {
        g.w[e >> 2][e & 3] = 0xFF800000u;
      }
    }
  }
}

// MIXED: per-request draft lengths, samplers (greedy requests included),
// draft ban lists and repetition penalties; the plain variant carries none of
// that logic. Plain batches also choose at launch (DR_*): whether the
// kept-token lists are in use (the workspace holds them; a run-time test of
// the pointer instead cost c5's draw 2 µs), or whether the target sampler
// truncates nothing, so that the code for truncated rows is left out (c3a
// and c3b 0.4-0.5 µs faster). The bf16 MIXED variant is held to 128 VGPRs
// (four waves per SIMD, so all workgroups of a launch stay resident).
constexpr int DR_NOLIST = 0, DR_LISTS = 1, DR_UNTRUNC = 2;
template <typename Elem, bool MIXED, int KIND>
__global__ __launch_bounds__(DR_THREADS, sizeof(Elem) == 2 ? (MIXED ? 4 : 1) : 2)
void draw_kernel(DrawArgs a) {
  __shared__ DrawShared sh;
  const int tid = threadIdx.x, wv = tid / WAVE, lane = tid & (WAVE - 1);
  // A plain batch's grid is part-major (part p of every request before part
  // p + 1: the draws finish closer together); a mixed batch's stays
  // request-major, so that the workgroups of a heavy request start together.
  const int nreq = (int)(gridDim.x / (unsigned)a.nwg);
  const int b = MIXED ? blockIdx.x / a.nwg : blockIdx.x % nreq;
  const int part = MIXED ? blockIdx.x % a.nwg : blockIdx.x / nreq;
  const int g = a.gamma, G1 = g + 1;
  const int sub0 = part * a.spw;
  const int nsl = min(a.spw, a.nsub - sub0);
  const int tok0 = sub0 * DRAW_SUB;
  const int nb = a.banned ? a.n_banned : 0;
  const int32_t* bl = a.banned ? a.banned + (int64_t)b * a.n_banned : nullptr;
  const int32_t ban0 = tid < nb ? bl[tid] : -1;
  ReqInfo rq;
  if constexpr (MIXED) {
    rq = request_info(a.req, b, g, a.st, a.sd);
    if (rq.bad || rq.greedy) {
      if (part == 0 && wv == 0) finish_without_draw(a, b, rq);
      return;
    }
  } else {
    rq.g = g;
    rq.st = a.st;
    rq.sd = a.sd;
    rq.greedy = false;
    rq.bad = false;
  }
  // the draft rows' own ban list, if the batch has one
  const int dnb = (MIXED && a.req.banned_d) ? a.req.n_banned_d : 0;
  const int32_t* dbl = dnb ? a.req.banned_d + (int64_t)b * a.req.n_banned_d : nullptr;
  const int32_t dban0 = tid < dnb ? dbl[tid] : -1;

  exp_table_fill(sh.etab);
  const Walk wk = accept_walk(a, b, rq.g);
  const DrawRow r = draw_row(a, b, wk.n, rq, wk.ts, wk.ds);
  const bool dmask = dnb > 0 && r.drow;
  if (dmask) mark_bans(sh.bmd, nsl * DRAW_SUB, dbl, dnb, dban0, tok0, a.V);
  // repetition penalty of the draw's rows: the history and the n accepted
  // proposals that precede position n
  const int H = (MIXED && a.req.history) ? a.req.n_history : 0;
  const int32_t* hist = H ? a.req.history + (int64_t)b * a.req.n_history : nullptr;
  const int32_t* props = a.draft_tokens + (int64_t)b * g;
  const bool tpen = MIXED && rq.pt != 1.0f && H + wk.n > 0;
  const bool dpen = MIXED && r.drow && rq.pd != 1.0f && H + wk.n > 0;
  if (tpen || dpen) mark_pen(sh.bmp, nsl * DRAW_SUB, hist, H, props, wk.n, tok0, a.V);
  if (nb > 0)
    mark_bans(sh.bm, nsl * DRAW_SUB, bl, nb, ban0, tok0, a.V);   // also publishes etab
  else
    __syncthreads();                                               // publishes etab

  // Weight sums of the workgroup's sub-chunks: wave wv owns sub-chunks wv,
  // wv + DR_NW, ...; lane l reads groups l, l + 64, l + 128, l + 192 of a
  // sub-chunk, so every load instruction covers 1 KiB of the row, and the wave
  // issues the loads of its next sub-chunk before it works on the current one.
  // Only tokens kept in the target row carry weight.
  // - At a rejection with a truncated target row (few kept tokens, spread
  //   thinly) the draft logits are needed only at the kept tokens: the wave
  //   queues them in LDS in token order and reads the draft row at the queued
  //   positions in one batch of independent loads, when the queue would
  //   overflow or its sub-chunks end; the sums then go to their sub-chunks.
  // - Otherwise (the bonus draw, or an untruncated target whose draft row is
  //   streamed alongside) the weights come from registers: through a per-wave
  //   compaction when at most 64 tokens are kept, in place when more are.
  // (a target sampler that truncates nothing leaves tau at -inf)
  const bool sparse = KIND != DR_UNTRUNC && r.ts.tau > -INFINITY;
  // kept-token lists of the sub-chunks for the selection (truncated target
  // rows of plain batches, when the workspace holds them; in mixed batches
  // they measured slower)
  static_assert(!MIXED || KIND == DR_NOLIST, "mixed batches take the general variant");
  const bool listing = KIND == DR_LISTS && sparse;
  const bool queued = sparse && r.drow;
  // the kept tokens of the wave's groups of one sub-chunk, and their number
  auto sub_mask = [&](int sbase, const Group<Elem>(&tg)[GPL], uint32_t(&km)[GPL]) {
    uint32_t cnt = 0u;
#pragma unroll
    for (int k = 0; k < GPL; ++k) {
      const int x0 = sbase + (lane + k * WAVE) * GRP;
      km[k] = x0 < a.V ? kept_mask<Elem>(r, tg[k], nb > 0 ? bm_group(sh.bm, x0 - tok0) : 0u) : 0u;
      cnt += (uint32_t)__popc(km[k]);
    }
    return cnt;
  };
  // Appends (x, w) of the lanes with `on` set to sub-chunk c's list at
  // positions base, base + 1, ... in lane order (stores past DRAW_LIST are
  // dropped); returns the new length. Same publication as the sums.
  auto list_put = [&](int64_t c, int base, bool on, int32_t x, double w) {
    const uint64_t m = __ballot(on);
    const int j = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (on && j < DRAW_LIST) {
      __hip_atomic_store(&a.lx[c * DRAW_LIST + j], x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.lw[c * DRAW_LIST + j], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return base + (int)__popcll(m);
  };
  // the weight sum of those kept tokens from registers, added to sw
  auto sub_sums = [&](int sbase, const Group<Elem>(&tg)[GPL], const Group<Elem>(&dg)[GPL],
                      const uint32_t(&km)[GPL], uint32_t cnt, double& sw, int& nl) {
    const uint32_t incl = wave_scan_dpp(cnt, 0u, [](uint32_t x, uint32_t y) { return x + y; });
    const uint32_t total = lane63(incl);
    nl = 0;
    if (total == 0u) return;
    if (total <= (uint32_t)WAVE) {
      uint32_t pos = incl - cnt;
#pragma unroll
      for (int k = 0; k < GPL; ++k) {
        for (uint32_t m = km[k]; m; m &= m - 1u) {   // one iteration per kept token
          const int e = __ffs(m) - 1;
          KeptTok t;
          t.x = sbase + (lane + k * WAVE) * GRP + e;
          t.zt = group_val_dyn<Elem>(tg[k], e);
          t.zd = r.drow ? group_val_dyn<Elem>(dg[k], e) : 0.0f;
          t.pad = 0;
          sh.kt[wv][pos++] = t;
        }
      }
      wave_sync_lds();
      int32_t x = -1;
      double w = 0.0;
      if ((uint32_t)lane < total) {
        const KeptTok t = sh.kt[wv][lane];
        x = t.x;
        w = tok_w(r, t.zt, t.zd, sh.etab);
        sw += w;
      }
      wave_sync_lds();
      if (listing) nl = list_put((int64_t)b * a.nsub + sbase / DRAW_SUB, 0, w > 0.0, x, w);
    } else {
#pragma unroll
      for (int k = 0; k < GPL; ++k)
        if (km[k]) sw += group_wsum<Elem>(r, tg[k], dg[k], km[k], sh.etab);
      nl = DRAW_LIST + 1;
    }
  };
  // A sub-chunk's weight sum goes out as soon as its wave has it. At a
  // rejection, a sub-chunk without residual mass also publishes its p sum
  // (lane_p() gives the lane's part, computed only then): when no sub-chunk
  // has any, the draw falls back to p and finds every p sum published. (Made
  // by the selecting workgroup alone instead, c5's 75 p sums took 50-90 µs.)
  // Publication
  // without a release fence: agent-scope atomic stores, which the hardware
  // writes through to the device-coherent level; every writer waits for its
  // stores to complete before the barrier that precedes the arrival ticket,
  // so they are visible device-wide before the ticket is taken. The reader
  // uses agent-scope atomic loads. (A release on the ticket would also write
  // back the whole L2, once per workgroup, for nothing.)
  // When listing, next to the sum goes the length nl of the sub-chunk's list
  // of tokens with w > 0 (DRAW_LIST + 1: not listed), so that the selection
  // can pick from the list instead of reading the sub-chunk again.
  // (Untruncated rows keep nearly every token: no lists.)
  auto publish = [&](int sl, double sw, int nl, auto&& lane_p) {
    sw = wave_total(sw);
    const bool need_p = r.drow != nullptr && !(sw > 0.0);
    double sp = 0.0;
    if (need_p) sp = wave_total(lane_p());
    if (lane == 0) {
      const int64_t c = (int64_t)b * a.nsub + sub0 + sl;
      __hip_atomic_store(&a.sums[c].w, sw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (listing) __hip_atomic_store(&a.lcount[c], nl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (need_p) __hip_atomic_store(&a.sums[c].p, sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  // The wave's sub-chunks, specialised by how the draft row is read: 0 =
  // queued reads at a truncated target, 1 = none (bonus draw), 2 = streamed.
  auto run = [&](auto mode_c) {
    constexpr int MODE = decltype(mode_c)::value;
    Group<Elem> tn[GPL], dn[GPL];   // the wave's next sub-chunk, in flight
    auto issue = [&](int sl) {
      const int sbase = tok0 + sl * DRAW_SUB;
#pragma unroll
      for (int k = 0; k < GPL; ++k) {
        const int x0 = sbase + (lane + k * WAVE) * GRP;
        if (x0 < a.V) {
          load_group<Elem, DR_NT<Elem>>(r.trow, x0, a.V, a.vec, tn[k]);
          if constexpr (MODE == 2) load_group<Elem, DR_NT<Elem>>(r.drow, x0, a.V, a.vec, dn[k]);
        }
      }
    };
    // queued tokens and the wave's sub-chunks they belong to (pend_lo ..
    // pend_hi, step DR_NW; wave-uniform)
    int qlen = 0, pend_lo = 0, pend_hi = -1;
    auto flush = [&]() {
      constexpr int QU = DR_QCAP / WAVE;
      wave_sync_lds();
      int qx[QU];
      float qt[QU], qd[QU];
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        const int j = u * WAVE + lane;
        qx[u] = -1;
        qt[u] = 0.0f;
        qd[u] = 0.0f;
        if (j < qlen) {
          const QueuedTok t = sh.q[wv][j];
          qx[u] = t.x;
          qt[u] = t.z;
          qd[u] = load_logit<Elem>(r.drow, t.x);
        }
      }
      if (dmask) {
#pragma unroll
        for (int u = 0; u < QU; ++u) {
          const int o = qx[u] - tok0;
          if (qx[u] >= 0 && ((sh.bmd[o >> 5] >> (o & 31)) & 1u)) qd[u] = -INFINITY;
        }
      }
      if (dpen) {
#pragma unroll
        for (int u = 0; u < QU; ++u) {
          const int o = qx[u] - tok0;
          if (qx[u] >= 0 && ((sh.bmp[o >> 5] >> (o & 31)) & 1u) && qd[u] > -INFINITY &&
              qd[u] < INFINITY)
            qd[u] = pen_apply(qd[u], rq.pd, sizeof(Elem) == 2);
        }
      }
      double qw[QU];
#pragma unroll
      for (int u = 0; u < QU; ++u) qw[u] = qx[u] >= 0 ? tok_w(r, qt[u], qd[u], sh.etab) : 0.0;
      for (int sl = pend_lo; sl <= pend_hi; sl += DR_NW) {
        const int lo = tok0 + sl * DRAW_SUB;
        const int64_t c = (int64_t)b * a.nsub + sub0 + sl;
        double sw = 0.0;
        int nl = 0;
#pragma unroll
        for (int u = 0; u < QU; ++u) {
          if (u * WAVE >= qlen) break;
          const bool in = qx[u] >= lo && qx[u] < lo + DRAW_SUB;
          if (in) sw += qw[u];
          if (listing) nl = list_put(c, nl, in && qw[u] > 0.0, qx[u], qw[u]);
        }
        publish(sl, sw, nl, [&]() {
          // from the queue in LDS (the registers of the batch are not kept for this)
          double sp = 0.0;
          for (int j = lane; j < qlen; j += WAVE) {
            const QueuedTok t = sh.q[wv][j];
            if (t.x >= lo && t.x < lo + DRAW_SUB) sp += tok_p(r, t.z, sh.etab);
          }
          return sp;
        });
      }
      wave_sync_lds();
      qlen = 0;
      pend_hi = -1;
    };
    if (wv < nsl) issue(wv);
    for (int sl = wv; sl < nsl; sl += DR_NW) {
      const int sbase = tok0 + sl * DRAW_SUB;
      Group<Elem> tg[GPL], dg[GPL];
#pragma unroll
      for (int k = 0; k < GPL; ++k) {
        const int o = sbase + (lane + k * WAVE) * GRP - tok0;
        tg[k] = tn[k];
        if (tpen && sbase + (lane + k * WAVE) * GRP < a.V)
          penalize_group<Elem>(tg[k], bm_group(sh.bmp, o), rq.pt);
        if constexpr (MODE == 2) {
          dg[k] = dn[k];
          if (dmask) mask_group<Elem>(dg[k], bm_group(sh.bmd, o));
          if (dpen && sbase + (lane + k * WAVE) * GRP < a.V)
            penalize_group<Elem>(dg[k], bm_group(sh.bmp, o), rq.pd);
        }
      }
      if (sl + DR_NW < nsl) issue(sl + DR_NW);
      uint32_t km[GPL];
      const uint32_t cnt = sub_mask(sbase, tg, km);
      auto lane_p = [&]() {
        double sp = 0.0;
#pragma unroll
        for (int k = 0; k < GPL; ++k)
          if (km[k]) sp += group_psum<Elem>(r, tg[k], km[k], sh.etab);
        return sp;
      };
      if constexpr (MODE != 0) {
        double sw = 0.0;
        int nl;
        sub_sums(sbase, tg, dg, km, cnt, sw, nl);
        publish(sl, sw, nl, lane_p);
      } else {
        const uint32_t incl = wave_scan_dpp(cnt, 0u, [](uint32_t x, uint32_t y) { return x + y; });
        const int total = (int)lane63(incl);
        if (pend_hi >= 0 && qlen + total > DR_QCAP) flush();
        if (total > DR_QCAP) {
          // more kept tokens than the queue holds: draft groups where needed,
          // evaluated in place
#pragma unroll
          for (int k = 0; k < GPL; ++k) {
            if (!km[k]) continue;
            const int x0 = sbase + (lane + k * WAVE) * GRP;
            load_group<Elem, DR_NT<Elem>>(r.drow, x0, a.V, a.vec, dg[k]);
            if (dmask) mask_group<Elem>(dg[k], bm_group(sh.bmd, x0 - tok0));
            if (dpen) penalize_group<Elem>(dg[k], bm_group(sh.bmp, x0 - tok0), rq.pd);
          }
          double sw = 0.0;
#pragma unroll
          for (int k = 0; k < GPL; ++k)
            if (km[k]) sw += group_wsum<Elem>(r, tg[k], dg[k], km[k], sh.etab);
          publish(sl, sw, DRAW_LIST + 1, lane_p);
          continue;
        }
        // one iteration per kept token of the lane (the wave runs as many as
        // its busiest lane needs, usually one or two)
        int pos = qlen + (int)(incl - cnt);
#pragma unroll
        for (int k = 0; k < GPL; ++k) {
          for (uint32_t m = km[k]; m; m &= m - 1u) {
            const int e = __ffs(m) - 1;
            QueuedTok t;
            t.x = sbase + (lane + k * WAVE) * GRP + e;
            t.z = group_val_dyn<Elem>(tg[k], e);
            sh.q[wv][pos++] = t;
          }
        }
        qlen += total;
        if (pend_hi < 0) pend_lo = sl;
        pend_hi = sl;
      }
    }
    if constexpr (MODE == 0) {
      if (pend_hi >= 0) flush();
    }
  };
  if (queued)
    run(std::integral_constant<int, 0>{});
  else if (!r.drow)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 2>{});
  __builtin_amdgcn_s_waitcnt(0);   // this wave's sums have landed
  // the last workgroup of the request to arrive performs the selection
  __syncthreads();
  if (tid == 0)
    sh.last = __hip_atomic_fetch_add(&a.tickets[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              a.nwg - 1;
  __syncthreads();
  if (!sh.last) return;

  const int n = wk.n;
  uint32_t flags = wk.flags;
  ChunkSums* cs = a.sums + (int64_t)b * a.nsub;
  auto ld = [](double* x) { return __hip_atomic_load(x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto ldi = [](int32_t* x) { return __hip_atomic_load(x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  // Per-token values of sub-chunk s0, one group of GRP tokens per thread: w,
  // or p when use_p (0 outside the target's kept set). The sub-chunk's bitmaps
  // are built here, with barriers: every thread calls this.
  auto sub_values = [&](int s0, bool use_p, double(&v)[GRP]) {
    const int x0 = s0 + tid * GRP;
    Group<Elem> tg, dg;
    if (x0 < a.V) {
      load_group<Elem, DR_NT<Elem>>(r.trow, x0, a.V, a.vec, tg);
      if (r.drow && !use_p) load_group<Elem, DR_NT<Elem>>(r.drow, x0, a.V, a.vec, dg);
    }
    if (dmask && !use_p) {
      mark_bans(sh.bmd, DRAW_SUB, dbl, dnb, dban0, s0, a.V);
      if (x0 < a.V) mask_group<Elem>(dg, bm_group(sh.bmd, x0 - s0));
    }
    if (tpen || (dpen && !use_p)) {
      mark_pen(sh.bmp, DRAW_SUB, hist, H, props, n, s0, a.V);
      if (x0 < a.V) {
        if (tpen) penalize_group<Elem>(tg, bm_group(sh.bmp, x0 - s0), rq.pt);
        if (dpen && !use_p) penalize_group<Elem>(dg, bm_group(sh.bmp, x0 - s0), rq.pd);
      }
    }
    if (nb > 0) mark_bans(sh.bm, DRAW_SUB, bl, nb, ban0, s0, a.V);
    const uint32_t km = x0 < a.V ? kept_mask<Elem>(r, tg, nb > 0 ? bm_group(sh.bm, x0 - s0) : 0u) : 0u;
    group_values<Elem>(r, tg, dg, km, sh.etab, use_p, v);
  };
  // every thread sums a contiguous run of sub-chunks, read once; one block
  // scan gives the prefix before each run and the total
  const int per = (a.nsub + DR_THREADS - 1) / DR_THREADS;
  const int k0 = tid * per, k1 = min(k0 + per, a.nsub);
  double loc = 0.0, before, S, unused0, unused1;
  for (int c = k0; c < k1; ++c) loc += ld(&cs[c].w);
  block_excl_scan2<DR_THREADS>(loc, 0.0, sh.scr, before, unused0, S, unused1);
  // Fall back to p when the residual has no mass (p and q then agree on every
  // token): the stream published the p sum of every sub-chunk (none had
  // residual mass), before the arrival tickets.
  bool use_p = false;
  if (!(S > 0.0) && n < g) {
    flags |= FLAG_RESIDUAL_ZERO;
    use_p = true;
    loc = 0.0;
    for (int c = k0; c < k1; ++c) loc += ld(&cs[c].p);
    block_excl_scan2<DR_THREADS>(loc, 0.0, sh.scr, before, unused0, S, unused1);
  }
  int32_t token = -1;
  if (!(S > 0.0)) {
    flags |= FLAG_EMPTY;
  } else {
    const double t = wk.u_final * S;
    // the sub-chunk holding t: the first thread whose run reaches t searches its
    // run; when rounding leaves t above every prefix, the last sub-chunk with
    // weight is taken
    int cand, lastw;
    block_first_last<DR_THREADS>(loc > 0.0 && before + loc >= t, loc > 0.0, sh.iscr, cand, lastw);
    const int who = cand < DR_THREADS ? cand : lastw;
    if (tid == who) {
      double run = before;
      int sel = -1;
      double selb = 0.0;
      for (int c = k0; c < k1; ++c) {
        // a run of one sub-chunk: its value is the run's sum, already loaded
        const double v = per == 1 ? loc : ld(use_p ? &cs[c].p : &cs[c].w);
        if (v > 0.0) {
          sel = c;                  // the last sub-chunk with weight unless one reaches t
          selb = run;
          if (run + v >= t) break;
        }
        run += v;
      }
      sh.sel_sub = sel;
      sh.sel_before = selb;
    }
    if (who < 0 && tid == 0) sh.sel_sub = -1;
    __syncthreads();
  }
  if (S > 0.0 && sh.sel_sub < 0) flags |= FLAG_EMPTY;   // no sub-chunk with weight
  // The selected sub-chunk's residual weights come from its list when the
  // stream listed them: wave 0 loads the list (with its length), puts it in
  // token order and picks; otherwise the sub-chunk is read again.
  const int sel = S > 0.0 ? sh.sel_sub : -1;
  const int64_t csel = (int64_t)b * a.nsub + sel;
  int nl = DRAW_LIST + 1;
  int32_t lxv = INT_MAX;
  double lwv = 0.0;
  if (S > 0.0 && sel >= 0 && !use_p && listing) {
    nl = ldi(&a.lcount[csel]);
    if (wv == 0 && lane < DRAW_LIST) {
      lxv = ldi(&a.lx[csel * DRAW_LIST + lane]);
      lwv = ld(&a.lw[csel * DRAW_LIST + lane]);
    }
  }
  if (S > 0.0 && sel >= 0 && nl <= DRAW_LIST) {
    if (wv == 0) {
      const double tl = wk.u_final * S - sh.sel_before;
      const bool on = lane < nl;
      if (!on) lxv = INT_MAX;            // listed ids are distinct and below V
      int rank = 0;
#pragma unroll
      for (int j = 0; j < DRAW_LIST; ++j) rank += __shfl(lxv, j, WAVE) < lxv ? 1 : 0;
      if (on) {
        sh.lt[rank].x = lxv;
        sh.lt[rank].w = lwv;
      }
      wave_sync_lds();
      int32_t sx = -1;
      double sw = 0.0;
      if (on) {
        sx = sh.lt[lane].x;
        sw = sh.lt[lane].w;
      }
      const double incl = wave_incl_scan(sw);
      // the first listed token reaching tl; the last one when rounding leaves
      // tl above the list's total
      const uint64_t reach = __ballot(on && incl >= tl);
      const uint64_t has = __ballot(on);
      const int pl = reach ? __ffsll((unsigned long long)reach) - 1
                           : (has ? 63 - __clzll((long long)has) : -1);
      token = pl >= 0 ? __shfl(sx, pl, WAVE) : -1;
    }
  } else if (S > 0.0 && sel >= 0) {
    const int s0 = sel * DRAW_SUB;
    const double tl = wk.u_final * S - sh.sel_before;
    const int x0 = s0 + tid * GRP;
    double v[GRP];
    sub_values(s0, use_p, v);
    double lsum = 0.0;
#pragma unroll
    for (int e = 0; e < GRP; ++e) lsum += v[e];
    double cb, dummy, ctot, dtot;
    block_excl_scan2<DR_THREADS>(lsum, 0.0, sh.scr, cb, dummy, ctot, dtot);
    int xc, xl;
    block_first_last<DR_THREADS>(lsum > 0.0 && cb + lsum >= tl, lsum > 0.0, sh.iscr, xc, xl);
    const int whot = xc < DR_THREADS ? xc : xl;   // a sub-chunk chosen here has weight
    if (tid == whot) {
      double run = cb;
      int pick = -1;
      for (int e = 0; e < GRP; ++e) {
        if (v[e] > 0.0) {
          pick = x0 + e;            // the last token with weight unless one reaches tl
          if (run + v[e] >= tl) break;
        }
        run += v[e];
      }
      sh.sel_x = pick;
    }
    if (whot < 0 && tid == 0) sh.sel_x = -1;
    __syncthreads();
    token = sh.sel_x;
  }
  int32_t* ot = a.out_tokens + (int64_t)b * G1;
  if (tid < G1) ot[tid] = tid < n ? wk.x : (tid == n ? token : -1);
  if (tid == 0) {
    a.out_num_accepted[b] = n;
    if (a.out_flags) a.out_flags[b] = flags;
    if (a.accept_hist) atomicAdd(&a.accept_hist[n], 1u);
  }
}

int launch_draw(const DrawArgs& a, int B, hipStream_t st) {
  const dim3 grid((unsigned)(a.nwg * B)), block(DR_THREADS);
  const bool mixed = a.req.gammas || a.req.ts || a.req.ds || a.req.banned_d || a.req.pen_t ||
                     a.req.pen_d || a.req.history;
  const bool untrunc = a.st.top_k == 0 && a.st.top_p >= 1.0f;
  const int kind = untrunc ? DR_UNTRUNC : (a.lcount ? DR_LISTS : DR_NOLIST);
  if (a.bf16) {
    if (mixed)
      hipLaunchKernelGGL((draw_kernel<uint16_t, true, DR_NOLIST>), grid, block, 0, st, a);
    else if (kind == DR_UNTRUNC)
      hipLaunchKernelGGL((draw_kernel<uint16_t, false, DR_UNTRUNC>), grid, block, 0, st, a);
    else if (kind == DR_LISTS)
      hipLaunchKernelGGL((draw_kernel<uint16_t, false, DR_LISTS>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((draw_kernel<uint16_t, false, DR_NOLIST>), grid, block, 0, st, a);
  } else {
    if (mixed)
      hipLaunchKernelGGL((draw_kernel<float, true, DR_NOLIST>), grid, block, 0, st, a);
    else if (kind == DR_UNTRUNC)
      hipLaunchKernelGGL((draw_kernel<float, false, DR_UNTRUNC>), grid, block, 0, st, a);
    else if (kind == DR_LISTS)
      hipLaunchKernelGGL((draw_kernel<float, false, DR_LISTS>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((draw_kernel<float, false, DR_NOLIST>), grid, block, 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
