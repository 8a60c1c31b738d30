// Per-position overlap of the target and draft distributions of a request:
// alpha_i = sum_x min(p_i(x), q_i(x)) = 1 - TV(p_i, q_i), for i < gamma.
//
// "Drafters and Speculative Decoding: Useful Tokens, Correct State", section
// "Confidence and verification admission": this overlap is the soft label of a
// confidence head; with x drawn from q_i and the acceptance rule of section
// "Sampling needs a correction rule" it is the probability that proposal i is
// accepted once the walk reaches it ("Accepted length is not speed": the
// conditional acceptance c_i).
//
// p_i and q_i are the sampler-transformed rows the walk compares (bans,
// temperature, top-k, top-p), so a token contributes only when it is kept in
// both rows; the row statistics pass supplies each row's threshold and
// normaliser. Because exp is monotone, min(p, q) = exp(min(s_t - lse_t,
// s_d - lse_d)): one fp64 exp per token kept in both rows.
//
// Work split: each (request, position) pair gets `parts` workgroups over
// consecutive sub-chunks of DRAW_SUB tokens; a wave owns whole sub-chunks. A
// truncated row keeps few tokens: it is read in full and the other row only in
// the groups where it keeps something. Sums are fixed-order (lanes, waves,
// parts), so the result does not depend on scheduling; with several parts the
// last workgroup of a pair to arrive adds the partial sums in part order.

#include "sv_launch.hpp"
#include "sv_rowio.hpp"

namespace sv {

constexpr int OV_THREADS = 256;
constexpr int OV_NW = OV_THREADS / WAVE;
constexpr int OV_GPL = DRAW_SUB / GRP / WAVE;   // groups per lane when a wave owns a sub-chunk

struct OverlapShared {
  double etab[256];
  KeptTok kt[OV_NW][WAVE];
  uint32_t bm[OV_SPW_MAX * DRAW_SUB / 32];
  double w[OV_NW];
};

template <typename Elem>
__global__ __launch_bounds__(OV_THREADS) void overlap_kernel(OverlapArgs a) {
  __shared__ OverlapShared sh;
  const int tid = threadIdx.x, wv = tid / WAVE, lane = tid & (WAVE - 1);
  const int pair = blockIdx.x / a.parts, part = blockIdx.x % a.parts;
  const int g = a.gamma, G1 = g + 1, RPR = 2 * g + 1;
  const int b = pair / g, i = pair % g;
  const int V = a.V;
  const RowStat ts = a.stats[(int64_t)b * RPR + i];
  const RowStat ds = a.stats[(int64_t)b * RPR + G1 + i];
  const Elem* trow = (const Elem*)a.target + ((int64_t)b * G1 + i) * V;
  const Elem* drow = (const Elem*)a.draft + ((int64_t)b * g + i) * V;
  const double tinv = 1.0 / (double)a.t_temp, dinv = 1.0 / (double)a.d_temp;
  const int sub0 = part * a.spp;
  const int nsl = min(a.spp, a.nsub - sub0);
  const int tok0 = sub0 * DRAW_SUB;
  // an empty row has p (or q) = 0 everywhere: the overlap is 0
  const bool empty = ((ts.flags | ds.flags) & FLAG_EMPTY) != 0u;
  const int nb = (a.banned && !empty) ? a.n_banned : 0;
  const int32_t* bl = nb ? a.banned + (int64_t)b * a.n_banned : nullptr;
  const int32_t ban0 = tid < nb ? bl[tid] : -1;

  exp_table_fill(sh.etab);
  if (nb > 0)
    mark_bans(sh.bm, nsl * DRAW_SUB, bl, nb, ban0, tok0, V);   // also publishes etab
  else
    __syncthreads();                                            // publishes etab

  // 0: the target row is truncated and leads; 1: the draft row leads; 2: both dense
  const int lead = ts.tau > -INFINITY ? 0 : (ds.tau > -INFINITY ? 1 : 2);
  auto term = [&](float zt, float zd) {
    const double lt = fma((double)zt, tinv, -ts.lse);
    const double ld = fma((double)zd, dinv, -ds.lse);
    return exp_tab(fmin(lt, ld), sh.etab);
  };

  double acc = 0.0;
  const int nsl_used = empty ? 0 : nsl;
  for (int sl = wv; sl < nsl_used; sl += OV_NW) {
    const int sbase = tok0 + sl * DRAW_SUB;
    Group<Elem> tg[OV_GPL], dg[OV_GPL];
    uint32_t km[OV_GPL];
#pragma unroll
    for (int k = 0; k < OV_GPL; ++k) {
      const int x0 = sbase + (lane + k * WAVE) * GRP;
      if (x0 < V) {
        if (lead != 1) load_group<Elem>(trow, x0, V, a.vec, tg[k]);
        if (lead != 0) load_group<Elem>(drow, x0, V, a.vec, dg[k]);
      }
    }
    // kept in the leading row (both rows when dense); bans apply to both rows
    // alike, so they are tested once
#pragma unroll
    for (int k = 0; k < OV_GPL; ++k) {
      const int x0 = sbase + (lane + k * WAVE) * GRP;
      uint32_t m = 0u;
      if (x0 < V) {
        const uint32_t ban = nb > 0 ? bm_group(sh.bm, x0 - tok0) : 0u;
#pragma unroll
        for (int e = 0; e < GRP; ++e) {
          const bool bn = (ban >> e) & 1u;
          bool kept;
          if (lead == 0)
            kept = is_kept(group_val<Elem>(tg[k], e), ts, bn);
          else if (lead == 1)
            kept = is_kept(group_val<Elem>(dg[k], e), ds, bn);
          else
            kept = is_kept(group_val<Elem>(tg[k], e), ts, bn) &&
                   is_kept(group_val<Elem>(dg[k], e), ds, false);
          m |= (kept ? 1u : 0u) << e;
        }
      }
      km[k] = m;
    }
    // the other row, only where the leading row keeps a token
    if (lead != 2) {
#pragma unroll
      for (int k = 0; k < OV_GPL; ++k) {
        if (!km[k]) continue;
        const int x0 = sbase + (lane + k * WAVE) * GRP;
        uint32_t m = 0u;
        if (lead == 0) {
          load_group<Elem>(drow, x0, V, a.vec, dg[k]);
#pragma unroll
          for (int e = 0; e < GRP; ++e)
            m |= (is_kept(group_val<Elem>(dg[k], e), ds, false) ? 1u : 0u) << e;
        } else {
          load_group<Elem>(trow, x0, V, a.vec, tg[k]);
#pragma unroll
          for (int e = 0; e < GRP; ++e)
            m |= (is_kept(group_val<Elem>(tg[k], e), ts, false) ? 1u : 0u) << e;
        }
        km[k] &= m;
      }
    }
    uint32_t cnt = 0u;
#pragma unroll
    for (int k = 0; k < OV_GPL; ++k) cnt += (uint32_t)__popc(km[k]);
    const uint32_t incl = wave_scan_dpp(cnt, 0u, [](uint32_t x, uint32_t y) { return x + y; });
    const uint32_t total = lane63(incl);
    if (total == 0u) continue;
    if (total <= (uint32_t)WAVE) {
      // few tokens kept in both rows: queue them so that lane k evaluates the
      // k-th one
      uint32_t pos = incl - cnt;
#pragma unroll
      for (int k = 0; k < OV_GPL; ++k) {
        if (!km[k]) continue;
#pragma unroll
        for (int e = 0; e < GRP; ++e) {
          if ((km[k] >> e) & 1u) {
            KeptTok t;
            t.x = sbase + (lane + k * WAVE) * GRP + e;
            t.zt = group_val<Elem>(tg[k], e);
            t.zd = group_val<Elem>(dg[k], e);
            t.pad = 0;
            sh.kt[wv][pos++] = t;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if ((uint32_t)lane < total) {
        const KeptTok t = sh.kt[wv][lane];
        acc += term(t.zt, t.zd);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
#pragma unroll
      for (int k = 0; k < OV_GPL; ++k) {
        if (!km[k]) continue;
#pragma unroll
        for (int e = 0; e < GRP; ++e)
          if ((km[k] >> e) & 1u) acc += term(group_val<Elem>(tg[k], e), group_val<Elem>(dg[k], e));
      }
    }
  }
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
  const dim3 grid((unsigned)(pairs * a.parts));
  if (bf16)
    hipLaunchKernelGGL(overlap_kernel<uint16_t>, grid, dim3(OV_THREADS), 0, st, a);
  else
    hipLaunchKernelGGL(overlap_kernel<float>, grid, dim3(OV_THREADS), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
