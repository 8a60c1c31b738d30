// Shared device-side definitions of the verifier kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr uint32_t FLAG_TOKEN_RANGE = 1u;
constexpr uint32_t FLAG_Q_ZERO = 2u;
constexpr uint32_t FLAG_NONFINITE = 4u;
constexpr uint32_t FLAG_EMPTY = 8u;
constexpr uint32_t FLAG_RESIDUAL_ZERO = 16u;
constexpr uint32_t FLAG_BAD_PARAM = 32u;

constexpr int WAVE = 64;

// Statistics of one sampler-transformed logit row, produced by row_stats and
// consumed by the draw kernel. A token x of the row is kept iff it is not
// banned, its logit z is finite and z >= tau.
struct alignas(16) RowStat {
  float m;         // largest kept logit (-inf for an empty row)
  float tau;       // truncation threshold on the logit value (-inf: none)
  double lse;      // log sum_{kept} exp(z / T)   (-inf for an empty row)
  uint32_t flags;  // FLAG_NONFINITE | FLAG_EMPTY
  uint32_t path;   // 0 = count histogram, 1 = generic streaming path; for the
                   // target row of a greedy request: its argmax (-1: none)
  double px;       // probability of the row's proposal token (target row i < gamma:
                   // p_i(x_i); draft row i: q_i(x_i)); 0 when it has none
};

// Partial sums of one vocabulary sub-chunk for the final draw.
struct alignas(16) ChunkSums {
  double w;  // sum of max(0, p - q) (bonus draw: sum of p)
  double p;  // sum of p (fallback when the residual mass is zero)
};

// Sampler settings as the kernels use them.
struct SamplerDev {
  float temperature;
  int32_t top_k;
  float top_p;
  float pad;
};

// Per-request sampler as the caller lays it out (sv_sampler of the C interface).
struct SamplerReq {
  float temperature;
  int32_t top_k;
  float top_p;
};

// Per-request settings of a mixed batch: device arrays, nullptr = call-wide.
struct ReqArgs {
  const int32_t* gammas;      // [B] proposals of each request, 0..gamma
  const SamplerReq* ts;       // [B] target samplers (temperature 0: greedy request)
  const SamplerReq* ds;       // [B] draft samplers
  const int32_t* banned_d;    // [B][n_banned_d] bans of the draft rows, or nullptr
  int n_banned_d;
  const int32_t* history;     // [B][n_history] generated tokens before the round, or nullptr
  int n_history;
  const float* pen_t;         // [B] repetition penalty of the target rows, or nullptr (1)
  const float* pen_d;         // [B] repetition penalty of the draft rows, or nullptr (1)
};

// One request's resolved settings.
struct ReqInfo {
  int g;             // proposals
  SamplerDev st, sd;
  bool greedy;       // target temperature 0
  bool bad;          // a setting out of range: the request is not verified
  float pt, pd;      // repetition penalties of the target and draft rows (1: none)
};

// Repetition penalty of one finite logit (Keskar et al. 2019, "CTRL", section
// 4.1, in its sign-aware form): z / theta for z > 0, z * theta otherwise,
// theta >= 1, in IEEE float32; for bf16 rows the result is rounded to bf16
// (nearest, ties to even), as an op on a bf16 logits tensor would round it.
__device__ __forceinline__ float pen_apply(float z, float theta, bool to_bf16) {
  float v = z > 0.0f ? z / theta : z * theta;
  if (to_bf16) {
    const uint32_t b = __float_as_uint(v);
    v = __uint_as_float((b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u);
  }
  return v;
}

__device__ __forceinline__ bool sampler_in_range(const SamplerDev& s, bool allow_greedy) {
  const float T = s.temperature;
  if (!(T >= 0.0f) || !(T < INFINITY) || (T == 0.0f && !allow_greedy)) return false;
  return s.top_k >= 0 && s.top_p > 0.0f && s.top_p <= 1.0f;
}

__device__ __forceinline__ ReqInfo request_info(const ReqArgs& q, int b, int gamma,
                                                const SamplerDev& st, const SamplerDev& sd) {
  ReqInfo r;
  r.g = q.gammas ? q.gammas[b] : gamma;
  r.st = st;
  r.sd = sd;
  if (q.ts) {
    const SamplerReq t = q.ts[b];
    r.st.temperature = t.temperature;
    r.st.top_k = t.top_k;
    r.st.top_p = t.top_p;
  }
  if (q.ds) {
    const SamplerReq t = q.ds[b];
    r.sd.temperature = t.temperature;
    r.sd.top_k = t.top_k;
    r.sd.top_p = t.top_p;
  }
  r.greedy = r.st.temperature == 0.0f;
  r.pt = q.pen_t ? q.pen_t[b] : 1.0f;
  r.pd = q.pen_d ? q.pen_d[b] : 1.0f;
  const bool pt_ok = r.pt >= 1.0f && r.pt < INFINITY, pd_ok = r.pd >= 1.0f && r.pd < INFINITY;
  r.bad = r.g < 0 || r.g > gamma || !sampler_in_range(r.st, true) || !pt_ok ||
          (!r.greedy && (!sampler_in_range(r.sd, false) || !pd_ok));
  if (r.bad) r.g = 0;
  return r;
}

// Lane `src`'s double (src wave-uniform), in scalar registers.
__device__ __forceinline__ double readlane_f64(double v, int src) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Order-preserving unsigned keys: a < b  <=>  key(a) < key(b) for non-NaN values,
// with -0 and +0 given the key of +0 so that they tie.
__device__ __forceinline__ uint32_t f32_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float f32_from_key(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11): ten rounds of two 64x64->128-bit products with the
// published multipliers, the key bumped by the published Weyl constants between
// rounds. Returns output word 0 of the block.
__device__ __forceinline__ uint64_t philox4x64_10_w0(uint64_t c0, uint64_t c1, uint64_t c2,
                                                     uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

// Uniform in (0, 1] for request b, slot j: counter (j, b, offset, 0), key (seed, 0).
__device__ __forceinline__ double philox_uniform(uint64_t seed, uint64_t offset, uint32_t b,
                                                 uint32_t j) {
  const uint64_t r = philox4x64_10_w0(j, b, offset, 0, seed, 0);
  return (double)((r >> 11) + 1) * 0x1.0p-53;
}

// exp(a) in fp64 for a <= about 0 (log-probabilities), to a few ulp, with no
// table and no memory access. Cody-Waite reduction a = k * (ln2 / 2) + r with
// |r| <= ln2 / 4 (ln2/2 split into a head and a tail); e^r - 1 from its
// degree-10 Taylor polynomial (remainder ~1e-16 relative); then
// e^a = 2^(k >> 1) * (k odd ? sqrt 2 : 1) * e^r.
__device__ __forceinline__ double exp_neg(double a) {
  a = fmax(a, -1000.0);                                   // exp(-1000) is 0 in fp64
  const double kf = rint(a * 0x1.71547652b82fep+1);       // 2 / ln2
  double r = fma(-kf, 0x1.62e42fefa39efp-2, a);           // head of ln2 / 2
  r = fma(-kf, 0x1.abc9e3b39803fp-57, r);                 // tail of ln2 / 2
  double q = fma(r, 1.0 / 3628800.0, 1.0 / 362880.0);
  q = fma(q, r, 1.0 / 40320.0);
  q = fma(q, r, 1.0 / 5040.0);
  q = fma(q, r, 1.0 / 720.0);
  q = fma(q, r, 1.0 / 120.0);
  q = fma(q, r, 1.0 / 24.0);
  q = fma(q, r, 1.0 / 6.0);
  q = fma(q, r, 0.5);
  q = fma(q, r, 1.0);
  q *= r;                                                 // e^r - 1
  const int k = (int)kf;
  const double t = (k & 1) ? 0x1.6a09e667f3bcdp+0 : 1.0;  // sqrt 2
  return ldexp(fma(t, q, t), k >> 1);
}

// ---------------------------------------------------------------- reductions

// Wave64 scans through DPP lane moves, which stay in the VALU and never queue
// behind LDS traffic. Inclusive scan: Hillis-Steele inside each row of 16 lanes
// (row_shr 1, 2, 4, 8), then lane 15 of rows 0 and 2 is broadcast into rows 1
// and 3 (row_bcast:15, row mask 0xA) and lane 31 into rows 2 and 3
// (row_bcast:31, row mask 0xC). Lanes whose source is outside the row, or whose
// row is masked, receive `ident`.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v, uint32_t ident) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int32_t dpp_move(int32_t v, int32_t ident) {
  return __builtin_amdgcn_update_dpp(ident, v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_move(double v, double ident) {
  const uint64_t b = (uint64_t)__double_as_longlong(v), o = (uint64_t)__double_as_longlong(ident);
  const uint32_t lo = dpp_move<CTRL, ROWMASK>((uint32_t)b, (uint32_t)o);
  const uint32_t hi = dpp_move<CTRL, ROWMASK>((uint32_t)(b >> 32), (uint32_t)(o >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_scan_dpp(T x, T ident, Op op) {
  x = op(x, dpp_move<0x111, 0xF>(x, ident));
  x = op(x, dpp_move<0x112, 0xF>(x, ident));
  x = op(x, dpp_move<0x114, 0xF>(x, ident));
  x = op(x, dpp_move<0x118, 0xF>(x, ident));
  x = op(x, dpp_move<0x142, 0xA>(x, ident));
  x = op(x, dpp_move<0x143, 0xC>(x, ident));
  return x;
}
// Value of lane 63 (the wave total after an inclusive scan).
__device__ __forceinline__ uint32_t lane63(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ int32_t lane63(int32_t v) { return __builtin_amdgcn_readlane(v, 63); }
__device__ __forceinline__ double lane63(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, WAVE);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) {
    T o = __shfl_xor(v, off, WAVE);
    v = o > v ? o : v;
  }
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) {
    T o = __shfl_xor(v, off, WAVE);
    v = o < v ? o : v;
  }
  return v;
}
// Inclusive prefix sum over the wave in lane order.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    T o = __shfl_up(v, off, WAVE);
    if (lane >= off) v += o;
  }
  return v;
}

// Block-wide reductions for NT threads; `scratch` holds at least NT/WAVE
// elements of T. All threads get the result. Fixed combination order, so the
// result does not depend on timing.
template <int NT, typename T>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
  constexpr int NW = NT / WAVE;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  T s = scratch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) s += scratch[i];
  return s;
}
template <int NT, typename T>
__device__ __forceinline__ T block_max(T v, T* scratch) {
  constexpr int NW = NT / WAVE;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  T s = scratch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) s = scratch[i] > s ? scratch[i] : s;
  return s;
}
template <int NT, typename T>
__device__ __forceinline__ T block_min(T v, T* scratch) {
  constexpr int NW = NT / WAVE;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  v = wave_min(v);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  T s = scratch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) s = scratch[i] < s ? scratch[i] : s;
  return s;
}
// Exclusive prefix sum over the block in thread order; *total gets the sum.
template <int NT, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* scratch, T* total) {
  constexpr int NW = NT / WAVE;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  T incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == WAVE - 1) scratch[w] = incl;
  __syncthreads();
  T before = T(0), all = T(0);
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) before += scratch[i];
    all += scratch[i];
  }
  *total = all;
  return before + incl - v;
}

// Exclusive prefix sums over the block, in thread order, of two values at
// once, with both totals. `scr` holds 2 * NT / WAVE doubles.
template <int NT>
__device__ __forceinline__ void block_excl_scan2(double x, double y, double* scr, double& px,
                                                 double& py, double& tx, double& ty) {
  constexpr int NW = NT / WAVE;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  const auto add = [](double u, double v) { return u + v; };
  const double ix = wave_scan_dpp(x, 0.0, add), iy = wave_scan_dpp(y, 0.0, add);
  __syncthreads();
  if (lane == WAVE - 1) {
    scr[w] = ix;
    scr[NW + w] = iy;
  }
  __syncthreads();
  double bx = 0.0, by = 0.0, ax = 0.0, ay = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) {
      bx += scr[i];
      by += scr[NW + i];
    }
    ax += scr[i];
    ay += scr[NW + i];
  }
  px = bx + ix - x;
  py = by + iy - y;
  tx = ax;
  ty = ay;
}

// Lowest thread index whose `f` holds (NT if none) and highest whose `l` holds
// (-1 if none), for the whole block. `scr` holds 2 * NT / WAVE ints.
template <int NT>
__device__ __forceinline__ void block_first_last(bool f, bool l, int* scr, int& first, int& last) {
  constexpr int NW = NT / WAVE;
  const int w = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  const uint64_t bf = __ballot(f), bl = __ballot(l);
  __syncthreads();
  if (lane == 0) {
    scr[w] = bf ? w * WAVE + __ffsll((unsigned long long)bf) - 1 : NT;
    scr[NW + w] = bl ? w * WAVE + 63 - __clzll((long long)bl) : -1;
  }
  __syncthreads();
  first = NT;
  last = -1;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    first = scr[i] < first ? scr[i] : first;
    last = scr[NW + i] > last ? scr[NW + i] : last;
  }
}

}  // namespace sv
