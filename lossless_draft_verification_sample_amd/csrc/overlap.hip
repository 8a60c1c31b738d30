// Per-position overlap of the target and draft distributions of a request:
// alpha_i = sum_x min(p_i(x), q_i(x)) = 1 - TV(p_i, q_i), for i < gamma.
//
// "Speculative Decoding - Turn guesses into parallel work", section
// "Confidence and verification admission": this overlap is the soft label of a
// confidence head; with x drawn from q_i and the acceptance rule of "Drafters
// and Speculative Decoding: Useful Tokens, Correct State", section "Sampling
// needs a correction rule", it is the probability that proposal i is accepted
// once the walk reaches it (first page, section "Accepted length is not
// speed": the conditional acceptance c_i).
//
// p_i and q_i are the sampler-transformed rows the walk compares (bans,
// temperature, top-k, top-p), so a token contributes only when it is kept in
// both rows; the row statistics pass supplies each row's threshold and
// normaliser. Because exp is monotone, min(p, q) = exp(min(s_t - lse_t,
// s_d - lse_d)): one fp64 exp per token kept in both rows.
//
// Work split: each (request, position) pair gets `parts` workgroups over
// consecutive sub-chunks of DRAW_SUB tokens; a wave owns whole sub-chunks and
// issues the loads of its next sub-chunk before it works on the current one. A
// truncated row keeps few tokens: it is streamed in full, its kept tokens are
// queued in LDS, and the other row is read only at the queued positions, in one
// batch of independent loads when the queue fills or the wave's sub-chunks end
// (so no load waits on another inside the stream). Sums are fixed-order (queue
// order, lanes, waves, parts), so the result does not depend on scheduling;
// with several parts the last workgroup of a pair to arrive adds the partial
// sums in part order.

#include "sv_launch.hpp"
#include "sv_rowio.hpp"

namespace sv {

// bf16 rows are streamed with nontemporal loads (measured faster, and the
// next kernels find the caches less disturbed)
template <typename Elem>
constexpr bool OV_NT = sizeof(Elem) == 2;

constexpr int OV_THREADS = 256;
constexpr int OV_NW = OV_THREADS / WAVE;
constexpr int OV_GPL = DRAW_SUB / GRP / WAVE;   // groups per lane when a wave owns a sub-chunk

constexpr int OV_QCAP = 4 * WAVE;   // queued kept tokens per wave: one batch of 4 loads per lane

// The bitmaps of mixed batches take LDS only in the MIXED variant.
template <bool MIXED>
struct OverlapShared {
  static constexpr int BMW = OV_SPW_MAX * DRAW_SUB / 32;
  double etab[256];
  QueuedTok q[OV_NW][OV_QCAP];
  uint32_t bm[BMW];                  // bans of the target row (of both rows unless the
                                     // draft rows have their own list)
  uint32_t bmd[MIXED ? BMW : 1];     // the draft rows' own bans
  uint32_t bmp[MIXED ? BMW : 1];     // repetition-penalized ids
  double w[OV_NW];
};



// What the streaming loop needs to know about one (request, position) pair.
struct OvPair {
  const void* trow;
  const void* drow;
  RowStat ts, ds;
  double tinv, dinv;  // 1/T of both rows
  int V, tok0, nsl, nb;
  int dnb;            // bans in the draft rows' own list
  bool sep;           // the draft rows have their own ban list (bmd)
  bool vec;
  bool tpen, dpen;    // the target / draft logits of the ids in bmp are penalized
  float pt, pd;       // their repetition penalties
};

// The wave's sum of min(p, q) over its sub-chunks wv, wv + OV_NW, ... .
// LEAD 0: the target row is truncated and leads: it is read in full and the
// draft row only where the target keeps a token; LEAD 1: the reverse; LEAD 2:
// neither is truncated and both rows are read in full.
template <typename Elem, int LEAD, typename Shared>
__device__ __forceinline__ double ov_stream(const OvPair& r, Shared& sh, int wv, int lane) {
  constexpr bool FULL_T = LEAD != 1, FULL_D = LEAD != 0;
  auto term = [&](float zt, float zd) {
    const double lt = fma((double)zt, r.tinv, -r.ts.lse);
    const double ld = fma((double)zd, r.dinv, -r.ds.lse);
    return exp_tab(fmin(lt, ld), sh.etab);
  };
  // ban bits of the eight tokens at offset o of the workgroup's range, per side
  auto tbits = [&](int o) -> uint32_t { return r.nb > 0 ? bm_group(sh.bm, o) : 0u; };
  auto dbits = [&](int o) -> uint32_t {
    return r.sep ? (r.dnb > 0 ? bm_group(sh.bmd, o) : 0u) : tbits(o);
  };
  // the other row's bans need a test of their own only when the lists differ
  auto obits = [&](int o) -> uint32_t { return !r.sep ? 0u : LEAD == 1 ? tbits(o) : dbits(o); };
  // the repetition penalty of the ids marked in bmp, per side
  auto pen_bits = [&](int o) -> uint32_t { return bm_group(sh.bmp, o); };
  const bool lpen = LEAD == 1 ? r.dpen : r.tpen, open_ = LEAD == 1 ? r.tpen : r.dpen;
  const float lth = LEAD == 1 ? r.pd : r.pt, oth = LEAD == 1 ? r.pt : r.pd;
  const void* lrow = LEAD == 1 ? r.drow : r.trow;   // leading row
  const void* orow = LEAD == 1 ? r.trow : r.drow;   // the other row
  const RowStat& ls = LEAD == 1 ? r.ds : r.ts;
  const RowStat& os = LEAD == 1 ? r.ts : r.ds;
  double acc = 0.0;
  // the other row's logits at the n queued tokens: lane l takes entries l,
  // l + 64, ...; all loads are issued before any is used
  auto flush = [&](int n) {
    wave_sync_lds();
    float zl[OV_QCAP / WAVE], zo[OV_QCAP / WAVE];
#pragma unroll
    for (int u = 0; u < OV_QCAP / WAVE; ++u) {
      const int j = u * WAVE + lane;
      zo[u] = -INFINITY;
      zl[u] = -INFINITY;
      if (j < n) {
        const QueuedTok t = sh.q[wv][j];
        zl[u] = t.z;
        zo[u] = load_logit<Elem>(orow, t.x);
        if (open_) {
          const int o = t.x - r.tok0;
          if (((sh.bmp[o >> 5] >> (o & 31)) & 1u) && zo[u] > -INFINITY && zo[u] < INFINITY)
            zo[u] = pen_apply(zo[u], oth, sizeof(Elem) == 2);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < OV_QCAP / WAVE; ++u) {
      const int j = u * WAVE + lane;
      if (j >= n) continue;
      bool ob = false;
      if (r.sep) {
        const int o = sh.q[wv][j].x - r.tok0;
        ob = (obits(o & ~7) >> (o & 7)) & 1u;
      }
      if (is_kept(zo[u], os, ob)) acc += LEAD == 1 ? term(zo[u], zl[u]) : term(zl[u], zo[u]);
    }
    wave_sync_lds();
  };

  Group<Elem> tn[OV_GPL], dn[OV_GPL];   // the next sub-chunk, in flight
  auto issue = [&](int sl) {
    const int sbase = r.tok0 + sl * DRAW_SUB;
#pragma unroll
    for (int k = 0; k < OV_GPL; ++k) {
      const int x0 = sbase + (lane + k * WAVE) * GRP;
      if (x0 < r.V) {
        if constexpr (FULL_T) load_group<Elem, OV_NT<Elem>>(r.trow, x0, r.V, r.vec, tn[k]);
        if constexpr (FULL_D) load_group<Elem, OV_NT<Elem>>(r.drow, x0, r.V, r.vec, dn[k]);
      }
    }
  };
  int qlen = 0;   // wave-uniform
  if (wv < r.nsl) issue(wv);
  for (int sl = wv; sl < r.nsl; sl += OV_NW) {
    const int sbase = r.tok0 + sl * DRAW_SUB;
    Group<Elem> tg[OV_GPL], dg[OV_GPL];
#pragma unroll
    for (int k = 0; k < OV_GPL; ++k) {
      const int x0 = sbase + (lane + k * WAVE) * GRP;
      if constexpr (FULL_T) {
        tg[k] = tn[k];
        if (r.tpen && x0 < r.V) penalize_group<Elem>(tg[k], pen_bits(x0 - r.tok0), r.pt);
      }
      if constexpr (FULL_D) {
        dg[k] = dn[k];
        if (r.dpen && x0 < r.V) penalize_group<Elem>(dg[k], pen_bits(x0 - r.tok0), r.pd);
      }
    }
    if (sl + OV_NW < r.nsl) issue(sl + OV_NW);
    // kept in the leading row (in both rows when neither leads); bans apply to
    // both rows alike, so they are tested once
    uint32_t km[OV_GPL];
#pragma unroll
    for (int k = 0; k < OV_GPL; ++k) {
      const int x0 = sbase + (lane + k * WAVE) * GRP;
      uint32_t m = 0u;
      if (x0 < r.V) {
        const int o = x0 - r.tok0;
        const uint32_t ban = LEAD == 1 ? dbits(o) : tbits(o);
        const uint32_t ban2 = LEAD == 2 ? obits(o) : 0u;   // draft bans, dense pairs
#pragma unroll
        for (int e = 0; e < GRP; ++e) {
          const bool bn = (ban >> e) & 1u;
          bool kept;
          if constexpr (LEAD == 0)
            kept = is_kept(group_val<Elem>(tg[k], e), r.ts, bn);
          else if constexpr (LEAD == 1)
            kept = is_kept(group_val<Elem>(dg[k], e), r.ds, bn);
          else
            kept = is_kept(group_val<Elem>(tg[k], e), r.ts, bn) &&
                   is_kept(group_val<Elem>(dg[k], e), r.ds, (ban2 >> e) & 1u);
          m |= (kept ? 1u : 0u) << e;
        }
      }
      km[k] = m;
    }
    if constexpr (LEAD == 2) {
#pragma unroll
      for (int k = 0; k < OV_GPL; ++k) {
        if (!km[k]) continue;
#pragma unroll
        for (int e = 0; e < GRP; ++e)
          if ((km[k] >> e) & 1u) acc += term(group_val<Elem>(tg[k], e), group_val<Elem>(dg[k], e));
      }
    } else {
      uint32_t cnt = 0u;
#pragma unroll
      for (int k = 0; k < OV_GPL; ++k) cnt += (uint32_t)__popc(km[k]);
      const uint32_t incl = wave_scan_dpp(cnt, 0u, [](uint32_t x, uint32_t y) { return x + y; });
      const int total = (int)lane63(incl);
      if (total == 0) continue;
      if (qlen + total > OV_QCAP) {
        flush(qlen);
        qlen = 0;
      }
      if (total <= OV_QCAP) {
        // queue the kept tokens in ascending token order of the wave's groups,
        // one iteration per kept token of the lane (the wave runs as many as
        // its busiest lane needs)
        int pos = qlen + (int)(incl - cnt);
#pragma unroll
        for (int k = 0; k < OV_GPL; ++k) {
          const Group<Elem>& lg = LEAD == 1 ? dg[k] : tg[k];
          for (uint32_t m = km[k]; m; m &= m - 1u) {
            const int e = __ffs(m) - 1;
            QueuedTok t;
            t.x = sbase + (lane + k * WAVE) * GRP + e;
            t.z = group_val_dyn<Elem>(lg, e);
            sh.q[wv][pos++] = t;
          }
        }
        qlen += total;
      } else {
        // a sub-chunk that keeps more tokens than the queue holds: read the
        // other row's groups where needed and evaluate in place
#pragma unroll
        for (int k = 0; k < OV_GPL; ++k) {
          if (!km[k]) continue;
          const int x0 = sbase + (lane + k * WAVE) * GRP;
          Group<Elem> og;
          load_group<Elem, OV_NT<Elem>>(orow, x0, r.V, r.vec, og);
          if (open_) penalize_group<Elem>(og, pen_bits(x0 - r.tok0), oth);
          const Group<Elem>& lg = LEAD == 1 ? dg[k] : tg[k];
          const uint32_t ob = obits(x0 - r.tok0);
#pragma unroll
          for (int e = 0; e < GRP; ++e) {
            const float zo = group_val<Elem>(og, e), zl = group_val<Elem>(lg, e);
            if (((km[k] >> e) & 1u) && is_kept(zo, os, (ob >> e) & 1u))
              acc += LEAD == 1 ? term(zo, zl) : term(zl, zo);
          }
        }
      }
    }
  }
  if constexpr (LEAD != 2) {
    if (qlen > 0) flush(qlen);
  }
  (void)ls;
  return acc;
}

// MIXED: per-request draft lengths, samplers and draft ban lists; a pair the
// request does not have (beyond its draft length, or a greedy request, or one
// with settings out of range) gets NaN.
template <typename Elem, bool MIXED>
__global__ __launch_bounds__(OV_THREADS) void overlap_kernel(OverlapArgs a) {
  __shared__ OverlapShared<MIXED> sh;
  const int tid = threadIdx.x, wv = tid / WAVE, lane = tid & (WAVE - 1);
  // part-major grid in a plain batch (part p of every pair before part p + 1)
  const int npairs = (int)(gridDim.x / (unsigned)a.parts);
  const int pair = MIXED ? blockIdx.x / a.parts : blockIdx.x % npairs;
  const int part = MIXED ? blockIdx.x % a.parts : blockIdx.x / npairs;
  const int g = a.gamma, G1 = g + 1, RPR = 2 * g + 1;
  const int b = pair / g, i = pair % g;
  ReqInfo rq;
  if constexpr (MIXED) {
    rq = request_info(a.req, b, g, a.st, a.sd);
    if (rq.bad || rq.greedy || i >= rq.g) {
      if (part == 0 && tid == 0) a.out_overlap[pair] = __builtin_nan("");
      return;
    }
  } else {
    rq.st = a.st;
    rq.sd = a.sd;
  }
  OvPair r;
  r.V = a.V;
  r.vec = a.vec != 0;
  r.ts = a.stats[(int64_t)b * RPR + i];
  r.ds = a.stats[(int64_t)b * RPR + G1 + i];
  r.trow = (const Elem*)a.target + ((int64_t)b * G1 + i) * a.V;
  r.drow = (const Elem*)a.draft + ((int64_t)b * g + i) * a.V;
  r.tinv = 1.0 / (double)rq.st.temperature;
  r.dinv = 1.0 / (double)rq.sd.temperature;
  const int sub0 = part * a.spp;
  r.tok0 = sub0 * DRAW_SUB;
  // an empty row has p (or q) = 0 everywhere: the overlap is 0
  const bool empty = ((r.ts.flags | r.ds.flags) & FLAG_EMPTY) != 0u;
  r.nsl = empty ? 0 : min(a.spp, a.nsub - sub0);
  r.nb = (a.banned && !empty) ? a.n_banned : 0;
  const int32_t* bl = r.nb ? a.banned + (int64_t)b * a.n_banned : nullptr;
  const int32_t ban0 = tid < r.nb ? bl[tid] : -1;
  r.sep = MIXED && a.req.banned_d != nullptr;
  // repetition penalty of the pair's rows: the history and the proposals
  // before position i
  const int H = (MIXED && a.req.history) ? a.req.n_history : 0;
  r.pt = MIXED ? rq.pt : 1.0f;
  r.pd = MIXED ? rq.pd : 1.0f;
  r.tpen = MIXED && !empty && r.pt != 1.0f && H + i > 0;
  r.dpen = MIXED && !empty && r.pd != 1.0f && H + i > 0;
  r.dnb = (r.sep && !empty) ? a.req.n_banned_d : 0;
  const int32_t* dbl = r.dnb ? a.req.banned_d + (int64_t)b * a.req.n_banned_d : nullptr;
  const int32_t dban0 = tid < r.dnb ? dbl[tid] : -1;

  exp_table_fill(sh.etab);
  if (r.dnb > 0) mark_bans(sh.bmd, r.nsl * DRAW_SUB, dbl, r.dnb, dban0, r.tok0, r.V);
  if (r.tpen || r.dpen) {
    // the pair's penalized ids in the workgroup's range (as mark_pen, written
    // out here: the shared helper crashed this compiler's inliner in this kernel)
    const int len = r.nsl * DRAW_SUB;
    for (int k = tid; k < len / 32; k += OV_THREADS) sh.bmp[k] = 0u;
    __syncthreads();
    for (int j = tid; j < H + i; j += OV_THREADS) {
      const int32_t id = j < H ? a.req.history[(int64_t)b * a.req.n_history + j]
                               : a.draft_tokens[(int64_t)b * g + (j - H)];
      if (id >= r.tok0 && id < r.V && id - r.tok0 < len) {
        const int o = id - r.tok0;
        atomicOr(&sh.bmp[o >> 5], 1u << (o & 31));
      }
    }
    __syncthreads();
  }
  if (r.nb > 0)
    mark_bans(sh.bm, r.nsl * DRAW_SUB, bl, r.nb, ban0, r.tok0, r.V);   // also publishes etab
  else
    __syncthreads();                                                  // publishes etab

  double acc;
  if (r.ts.tau > -INFINITY)
    acc = ov_stream<Elem, 0>(r, sh, wv, lane);
  else if (r.ds.tau > -INFINITY)
    acc = ov_stream<Elem, 1>(r, sh, wv, lane);
  else
    acc = ov_stream<Elem, 2>(r, sh, wv, lane);
  acc = wave_total(acc);
  if (lane == 0) sh.w[wv] = acc;
  __syncthreads();
  if (tid != 0) return;
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < OV_NW; ++w) s += sh.w[w];
  if (a.parts == 1) {
    a.out_overlap[pair] = s;
    return;
  }
  // Partial sums are published as agent-scope atomic stores, which write
  // through to the device-coherent level; the writer waits for them before it
  // takes its ticket, and the last arrival reads them with agent-scope atomic
  // loads (no cache-wide release needed).
  double* pp = a.partial + (int64_t)pair * a.parts;
  __hip_atomic_store(pp + part, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  const int arrived =
      __hip_atomic_fetch_add(&a.tickets[pair], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (arrived != a.parts - 1) return;
  double tot = 0.0;
  for (int c = 0; c < a.parts; ++c)
    tot += __hip_atomic_load(pp + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  a.out_overlap[pair] = tot;
}

int launch_overlap(const OverlapArgs& a, int bf16, int pairs, hipStream_t st) {
  const dim3 grid((unsigned)(pairs * a.parts)), block(OV_THREADS);
  const bool mixed = a.req.gammas || a.req.ts || a.req.ds || a.req.banned_d || a.req.pen_t ||
                     a.req.pen_d || a.req.history;
  if (bf16) {
    if (mixed)
      hipLaunchKernelGGL((overlap_kernel<uint16_t, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((overlap_kernel<uint16_t, false>), grid, block, 0, st, a);
  } else {
    if (mixed)
      hipLaunchKernelGGL((overlap_kernel<float, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((overlap_kernel<float, false>), grid, block, 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
