// Ban-list preparation, acceptance walk and final draw of spec_verify_sample.
//
// Acceptance ("Speculative Decoding - Turn guesses into parallel work", section
// "Exact sampling: account for every probability"; "Speculative Token
// Decoupling ..." Equation 3.1): proposal i of a request is accepted iff
// u_i * q_i(x_i) <= p_i(x_i), walking left to right and stopping at the first
// rejection. p and q are recomputed in fp64 from the gathered logits and the
// row statistics.
//
// Final draw ("Drafters and Speculative Decoding: Useful Tokens, Correct State",
// section "Sampling needs a correction rule"; "Speculative Decoding"
// fundamentals, section "The Loop"): at the first rejection n the token is
// drawn from norm(max(0, p_n - q_n)); if every proposal survived it is drawn
// from p_gamma. The draw is an inverse CDF in ascending token order: the
// smallest x whose running weight sum reaches u * S. Only the one (or two)
// selected rows per request are read again. The vocabulary is cut into chunks:
// one kernel sums each chunk's weights, a second one locates the chunk holding
// u * S and scans just that chunk.

#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

// ------------------------------------------------------------------ ban lists

constexpr int BP_THREADS = 256;
constexpr int BP_MAX = 2048;

__global__ __launch_bounds__(BP_THREADS) void ban_prep_kernel(BanPrepArgs a) {
  __shared__ int32_t s[BP_MAX];
  __shared__ uint32_t scr[BP_THREADS / WAVE];
  const int b = blockIdx.x, tid = threadIdx.x;
  int np = 1;
  while (np < a.n_banned) np <<= 1;
  for (int j = tid; j < np; j += BP_THREADS) {
    int32_t v = INT32_MAX;
    if (j < a.n_banned) {
      const int32_t id = a.banned[(int64_t)b * a.n_banned + j];
      if (id >= 0 && id < a.V) v = id;
    }
    s[j] = v;
  }
  __syncthreads();
  // bitonic sort, ascending
  for (int k = 2; k <= np; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < np; i += BP_THREADS) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const int32_t x = s[i], y = s[ixj];
          const bool up = (i & k) == 0;
          if (up ? (x > y) : (x < y)) {
            s[i] = y;
            s[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  // keep the first of every run of equal valid ids, compacted in order
  const int per = (np + BP_THREADS - 1) / BP_THREADS;
  const int j0 = tid * per;
  uint32_t keep = 0;
  for (int j = j0; j < j0 + per && j < np; ++j)
    keep += (s[j] != INT32_MAX && (j == 0 || s[j] != s[j - 1])) ? 1u : 0u;
  uint32_t total;
  uint32_t pos = block_excl_scan<BP_THREADS>(keep, scr, &total);
  for (int j = j0; j < j0 + per && j < np; ++j) {
    if (s[j] != INT32_MAX && (j == 0 || s[j] != s[j - 1]))
      a.ban_sorted[(int64_t)b * a.n_banned + pos++] = s[j];
  }
  if (tid == 0) a.ban_count[b] = (int32_t)total;
}

int launch_ban_prep(const BanPrepArgs& a, int B, hipStream_t st) {
  hipLaunchKernelGGL(ban_prep_kernel, dim3(B), dim3(BP_THREADS), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float load_logit(const void* base, int bf16, int64_t idx) {
  if (bf16) return bf16_to_f32(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

__device__ __forceinline__ bool is_kept(float z, const RowStat& s, bool banned) {
  return !banned && !(s.flags & FLAG_EMPTY) && z > -INFINITY && z < INFINITY && z >= s.tau;
}

// ------------------------------------------------------------------ acceptance

__global__ __launch_bounds__(WAVE) void accept_kernel(AcceptArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int g = a.gamma, G1 = g + 1, RPR = 2 * g + 1;
  const RowStat* st = a.stats + (int64_t)b * RPR;
  const int nb = a.ban_count ? a.ban_count[b] : 0;
  const int32_t* bans = a.ban_sorted ? a.ban_sorted + (int64_t)b * a.ban_stride : nullptr;

  uint32_t rf = 0;
  for (int r = lane; r < RPR; r += WAVE) rf |= st[r].flags & (FLAG_NONFINITE | FLAG_EMPTY);
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) rf |= __shfl_xor(rf, off, WAVE);

  int32_t x = -1;
  bool acc = false, range = false, qzero = false;
  if (lane < g) {
    x = a.draft_tokens[(int64_t)b * g + lane];
    range = x < 0 || x >= a.V;
    if (!range) {
      const float zt = load_logit(a.target, a.bf16, ((int64_t)b * G1 + lane) * a.V + x);
      const float zd = load_logit(a.draft, a.bf16, ((int64_t)b * g + lane) * a.V + x);
      const bool banned = nb > 0 && in_sorted(bans, nb, x);
      const RowStat ts = st[lane], ds = st[G1 + lane];
      const double p = is_kept(zt, ts, banned) ? exp((double)zt / (double)a.t_temp - ts.lse) : 0.0;
      const double q = is_kept(zd, ds, banned) ? exp((double)zd / (double)a.d_temp - ds.lse) : 0.0;
      const double u = a.uniforms ? a.uniforms[(int64_t)b * G1 + lane]
                                  : philox_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)lane);
      qzero = !(q > 0.0);
      acc = !qzero && u * q <= p;
    }
  }
  const uint64_t accm = __ballot(acc);
  const uint64_t rangem = __ballot(range);
  const uint64_t qzm = __ballot(qzero && !range);
  int n = __ffsll((unsigned long long)~accm) - 1;
  if (n > g) n = g;
  uint32_t flags = rf;
  if (rangem) flags |= FLAG_TOKEN_RANGE;
  if (n < g && ((qzm >> n) & 1ull)) flags |= FLAG_Q_ZERO;
  if (lane < n) a.out_tokens[(int64_t)b * G1 + lane] = x;
  if (lane == 0) {
    a.out_num_accepted[b] = n;
    ReqState rs;
    rs.n = n;
    rs.flags = flags;
    rs.u_final = a.uniforms ? a.uniforms[(int64_t)b * G1 + g]
                            : philox_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)g);
    a.req[b] = rs;
  }
}

int launch_accept(const AcceptArgs& a, int B, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(WAVE), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------------ final draw

constexpr int DR_THREADS = 256;
constexpr int GRP = 8;                                   // logits per group
constexpr int GPT = DRAW_CHUNK / GRP / DR_THREADS;       // groups per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DrawRow {
  const void* trow;
  const void* drow;   // nullptr for the bonus draw
  RowStat ts, ds;
  double tinv, dinv;  // 1/T of both rows
};

__device__ __forceinline__ DrawRow draw_row(const DrawArgs& a, int b, int n) {
  const int g = a.gamma, G1 = g + 1, RPR = 2 * g + 1;
  DrawRow r;
  const int64_t V = a.V;
  const size_t es = a.bf16 ? 2 : 4;
  r.trow = (const char*)a.target + ((int64_t)b * G1 + n) * V * es;
  r.ts = a.stats[(int64_t)b * RPR + n];
  r.tinv = 1.0 / (double)a.t_temp;
  if (n < g) {
    r.drow = (const char*)a.draft + ((int64_t)b * g + n) * V * es;
    r.ds = a.stats[(int64_t)b * RPR + G1 + n];
    r.dinv = 1.0 / (double)a.d_temp;
  } else {
    r.drow = nullptr;
  }
  return r;
}

// Eight consecutive logits starting at x0, as raw bits (-inf beyond the row).
template <typename Elem>
struct Group {
  u32x4 w[sizeof(Elem) == 2 ? 1 : 2];
};

template <typename Elem>
__device__ __forceinline__ void load_group(const void* row, int x0, int V, bool vec, Group<Elem>& g) {
  const Elem* e = (const Elem*)row;
  if constexpr (sizeof(Elem) == 2) {
    if (vec) {
      g.w[0] = *(const u32x4*)(e + x0);   // V % 8 == 0 on this path
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = x0 + 2 * j < V ? (uint32_t)e[x0 + 2 * j] : 0xFF80u;
        const uint32_t hi = x0 + 2 * j + 1 < V ? (uint32_t)e[x0 + 2 * j + 1] : 0xFF80u;
        g.w[0][j] = lo | (hi << 16);
      }
    }
  } else {
    if (vec) {
      const u32x4* p = (const u32x4*)(e + x0);
      g.w[0] = p[0];                       // V % 4 == 0 on this path
      g.w[1] = x0 + 4 < V ? p[1] : (u32x4)(0xFF800000u);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        g.w[j >> 2][j & 3] = x0 + j < V ? __float_as_uint(e[x0 + j]) : 0xFF800000u;
    }
  }
}

template <typename Elem>
__device__ __forceinline__ float group_val(const Group<Elem>& g, int j) {
  if constexpr (sizeof(Elem) == 2) return bf16_to_f32((g.w[0][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
  return __uint_as_float(g.w[j >> 2][j & 3]);
}

// p(x) and the draw weight of token x: max(0, p - q) at a rejection, p for the
// bonus draw. fp64 throughout (exp of an fp64 argument), so the running sums
// of the inverse CDF carry no fp32 error.
__device__ __forceinline__ void pair_weight(const DrawRow& r, float zt, float zd, bool banned,
                                            double& w, double& p) {
  p = is_kept(zt, r.ts, banned) ? exp_neg((double)zt * r.tinv - r.ts.lse) : 0.0;
  if (r.drow) {
    const double q = is_kept(zd, r.ds, banned) ? exp_neg((double)zd * r.dinv - r.ds.lse) : 0.0;
    w = p > q ? p - q : 0.0;
  } else {
    w = p;
  }
}

// Marks the banned ids of [c0, c0 + len) in an LDS bitmap of len / 32 words.
__device__ __forceinline__ void range_bans(uint32_t* bm, int len, const int32_t* bans, int nb,
                                           int c0) {
  for (int k = threadIdx.x; k < len / 32; k += blockDim.x) bm[k] = 0u;
  __syncthreads();
  if (nb > 0) {
    const int lo = lower_bound(bans, nb, c0);
    const int hi = lower_bound(bans, nb, c0 + len);
    for (int j = lo + (int)threadIdx.x; j < hi; j += blockDim.x) {
      const int o = bans[j] - c0;
      atomicOr(&bm[o >> 5], 1u << (o & 31));
    }
  }
  __syncthreads();
}

__device__ __forceinline__ bool bm_test(const uint32_t* bm, int o) {
  return (bm[o >> 5] >> (o & 31)) & 1u;
}

// One workgroup per (request, DRAW_CHUNK tokens): weight sums per DRAW_SUB.
// Group j of thread t covers tokens c0 + j*DRAW_SUB + 8t .. +8, so sub-chunk j
// is exactly the j-th group of every thread and the loads are coalesced.
template <typename Elem>
__global__ __launch_bounds__(DR_THREADS) void residual_partial_kernel(DrawArgs a) {
  static_assert(DRAW_SUB == DR_THREADS * GRP && GPT == SUB_PER_CHUNK, "draw tiling");
  __shared__ uint32_t bm[DRAW_CHUNK / 32];
  __shared__ double scr[2 * SUB_PER_CHUNK][DR_THREADS / WAVE];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / a.nchunk, c = blockIdx.x % a.nchunk;
  const ReqState rs = a.req[b];
  const DrawRow r = draw_row(a, b, rs.n);
  const int nb = a.ban_count ? a.ban_count[b] : 0;
  const int32_t* bans = a.ban_sorted ? a.ban_sorted + (int64_t)b * a.ban_stride : nullptr;
  const int c0 = c * DRAW_CHUNK;
  const bool vec = a.vec;
  // every load of this thread in flight before any use
  Group<Elem> tg[GPT], dg[GPT];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const int x0 = c0 + j * DRAW_SUB + tid * GRP;
    if (x0 < a.V) {
      load_group<Elem>(r.trow, x0, a.V, vec, tg[j]);
      if (r.drow) load_group<Elem>(r.drow, x0, a.V, vec, dg[j]);
    }
  }
  range_bans(bm, DRAW_CHUNK, bans, nb, c0);
  double sw[GPT], sp[GPT];
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    sw[j] = 0.0;
    sp[j] = 0.0;
    const int x0 = c0 + j * DRAW_SUB + tid * GRP;
    if (x0 < a.V) {
#pragma unroll
      for (int e = 0; e < GRP; ++e) {
        double w, p;
        pair_weight(r, group_val<Elem>(tg[j], e), r.drow ? group_val<Elem>(dg[j], e) : 0.0f,
                    bm_test(bm, x0 - c0 + e), w, p);
        sw[j] += w;
        sp[j] += p;
      }
    }
  }
  // per-sub-chunk block sums in a fixed order
  const int wv = tid / WAVE, lane = tid & (WAVE - 1);
#pragma unroll
  for (int j = 0; j < GPT; ++j) {
    const double a0 = wave_sum(sw[j]), a1 = wave_sum(sp[j]);
    if (lane == 0) {
      scr[2 * j][wv] = a0;
      scr[2 * j + 1][wv] = a1;
    }
  }
  __syncthreads();
  if (tid < GPT) {
    const int sub = c * SUB_PER_CHUNK + tid;
    if (sub < a.nsub) {
      double w = 0.0, p = 0.0;
#pragma unroll
      for (int k = 0; k < DR_THREADS / WAVE; ++k) {
        w += scr[2 * tid][k];
        p += scr[2 * tid + 1][k];
      }
      ChunkSums cs;
      cs.w = w;
      cs.p = p;
      a.sums[(int64_t)b * a.nsub + sub] = cs;
    }
  }
}

int launch_residual_partial(const DrawArgs& a, int B, hipStream_t st) {
  if (a.bf16)
    hipLaunchKernelGGL(residual_partial_kernel<uint16_t>, dim3(a.nchunk * B), dim3(DR_THREADS), 0, st, a);
  else
    hipLaunchKernelGGL(residual_partial_kernel<float>, dim3(a.nchunk * B), dim3(DR_THREADS), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// One workgroup per request: locate the sub-chunk holding u * S from the
// partial sums, then rescan those DRAW_SUB tokens (8 per thread, in id order).
template <typename Elem>
__global__ __launch_bounds__(DR_THREADS) void residual_select_kernel(DrawArgs a) {
  __shared__ uint32_t bm[DRAW_SUB / 32];
  __shared__ double scr[DR_THREADS / WAVE];
  __shared__ int32_t sel_sub, sel_x;
  __shared__ double sel_before;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int g = a.gamma, G1 = g + 1;
  const ReqState rs = a.req[b];
  const int n = rs.n;
  uint32_t flags = rs.flags;
  const ChunkSums* cs = a.sums + (int64_t)b * a.nsub;

  // totals; fall back to p when the residual has no mass
  double tw = 0.0, tp = 0.0;
  for (int c = tid; c < a.nsub; c += DR_THREADS) {
    tw += cs[c].w;
    tp += cs[c].p;
  }
  tw = block_sum<DR_THREADS>(tw, scr);
  tp = block_sum<DR_THREADS>(tp, scr);
  bool use_p = false;
  double S = tw;
  if (!(tw > 0.0) && n < g) {
    flags |= FLAG_RESIDUAL_ZERO;
    use_p = true;
    S = tp;
  }
  int32_t token = -1;
  if (!(S > 0.0)) {
    flags |= FLAG_EMPTY;
  } else {
    const double t = rs.u_final * S;
    // sub-chunk holding t: per-thread contiguous runs, a block scan, and the
    // first thread whose run reaches t searches its run
    const int per = (a.nsub + DR_THREADS - 1) / DR_THREADS;
    const int k0 = tid * per;
    double loc = 0.0;
    for (int c = k0; c < k0 + per && c < a.nsub; ++c) loc += use_p ? cs[c].p : cs[c].w;
    double tot;
    const double before = block_excl_scan<DR_THREADS>(loc, scr, &tot);
    const int cand = block_min<DR_THREADS>((loc > 0.0 && before + loc >= t) ? tid : DR_THREADS,
                                           (int*)scr);
    if (tid == 0) {
      sel_sub = -1;
      sel_before = 0.0;
    }
    __syncthreads();
    if (tid == cand) {
      double run = before;
      for (int c = k0; c < k0 + per && c < a.nsub; ++c) {
        const double v = use_p ? cs[c].p : cs[c].w;
        if (v > 0.0) {
          sel_sub = c;              // the last sub-chunk with weight unless one reaches t
          sel_before = run;
          if (run + v >= t) break;
        }
        run += v;
      }
    }
    __syncthreads();
    if (sel_sub < 0 && tid == 0) {
      // t above every prefix through rounding: the last sub-chunk with weight
      double run = 0.0;
      for (int c = 0; c < a.nsub; ++c) {
        const double v = use_p ? cs[c].p : cs[c].w;
        if (v > 0.0) {
          sel_sub = c;
          sel_before = run;
        }
        run += v;
      }
    }
    __syncthreads();
    const int s0 = sel_sub * DRAW_SUB;
    const double tl = t - sel_before;
    const DrawRow r = draw_row(a, b, n);
    const int nb = a.ban_count ? a.ban_count[b] : 0;
    const int32_t* bans = a.ban_sorted ? a.ban_sorted + (int64_t)b * a.ban_stride : nullptr;
    const int x0 = s0 + tid * GRP;
    Group<Elem> tg, dg;
    if (x0 < a.V) {
      load_group<Elem>(r.trow, x0, a.V, a.vec, tg);
      if (r.drow) load_group<Elem>(r.drow, x0, a.V, a.vec, dg);
    }
    range_bans(bm, DRAW_SUB, bans, nb, s0);
    double v[GRP];
    double lsum = 0.0;
#pragma unroll
    for (int e = 0; e < GRP; ++e) {
      v[e] = 0.0;
      if (x0 + e < a.V) {
        double w, p;
        pair_weight(r, group_val<Elem>(tg, e), r.drow ? group_val<Elem>(dg, e) : 0.0f,
                    bm_test(bm, x0 - s0 + e), w, p);
        v[e] = use_p ? p : w;
      }
      lsum += v[e];
    }
    double ctot;
    const double cb = block_excl_scan<DR_THREADS>(lsum, scr, &ctot);
    const int xc = block_min<DR_THREADS>((lsum > 0.0 && cb + lsum >= tl) ? tid : DR_THREADS,
                                         (int*)scr);
    const int xl = block_max<DR_THREADS>(lsum > 0.0 ? tid : -1, (int*)scr);
    const int who = xc < DR_THREADS ? xc : xl;   // a sub-chunk chosen here has weight
    if (tid == 0) sel_x = -1;
    __syncthreads();
    if (tid == who) {
      double run = cb;
      int pick = -1;
      for (int e = 0; e < GRP; ++e) {
        if (v[e] > 0.0) {
          pick = x0 + e;            // the last token with weight unless one reaches tl
          if (run + v[e] >= tl) break;
        }
        run += v[e];
      }
      sel_x = pick;
    }
    __syncthreads();
    token = sel_x;
  }
  if (tid == 0) {
    a.out_tokens[(int64_t)b * G1 + n] = token;
    for (int j = n + 1; j < G1; ++j) a.out_tokens[(int64_t)b * G1 + j] = -1;
    if (a.out_flags) a.out_flags[b] = flags;
  }
}

int launch_residual_select(const DrawArgs& a, int B, hipStream_t st) {
  if (a.bf16)
    hipLaunchKernelGGL(residual_select_kernel<uint16_t>, dim3(B), dim3(DR_THREADS), 0, st, a);
  else
    hipLaunchKernelGGL(residual_select_kernel<float>, dim3(B), dim3(DR_THREADS), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
