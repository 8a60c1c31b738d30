// Greedy verification ("Drafters and Speculative Decoding: Useful Tokens,
// Correct State", section "Greedy verification"; "Speculative Decoding - Turn
// guesses into parallel work", section "Greedy, sampling and the real sampler"):
// a proposal survives while it equals the argmax of its target row; the first
// mismatch emits that row's argmax; if all gamma match, the argmax of row gamma
// is appended. Ties go to the lowest token id (-0 and +0 tie).
//
// greedy_argmax: one workgroup per target row streams the row once with 16-byte
// loads; each lane keeps the first position of its largest value (lanes visit
// their positions in increasing order, so a strict > keeps the lowest id), and
// the workgroup merges (value, id) pairs. The argmax is parked in out_tokens,
// which greedy_scan then rewrites into the emitted block.

#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

constexpr int GA_THREADS = 512;
constexpr int GA_UNROLL = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

struct ArgBest {
  float v;
  int32_t i;
};

__device__ __forceinline__ void arg_take(ArgBest& a, float v, int32_t i) {
  if (v > a.v) {
    a.v = v;
    a.i = i;
  }
}

// (value desc, id asc) merge of two candidates; id INT32_MAX means none.
__device__ __forceinline__ ArgBest arg_merge(ArgBest a, ArgBest b) {
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

template <typename Elem>
__device__ __forceinline__ float g_val(const Elem* p, int i);
template <>
__device__ __forceinline__ float g_val<uint16_t>(const uint16_t* p, int i) {
  return bf16_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float g_val<float>(const float* p, int i) {
  return p[i];
}

template <typename Elem>
__global__ __launch_bounds__(GA_THREADS) void greedy_argmax_kernel(GreedyArgs a) {
  constexpr int PER = 16 / sizeof(Elem);
  __shared__ float sv_[GA_THREADS / WAVE];
  __shared__ int32_t si_[GA_THREADS / WAVE];
  __shared__ uint32_t su_[GA_THREADS / WAVE];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int V = a.V;
  const Elem* rowp = (const Elem*)a.target + (int64_t)row * V;

  ArgBest best{-INFINITY, INT32_MAX};
  uint32_t expmax = 0;   // largest exponent field seen (all ones: inf or NaN present)
  const uintptr_t addr = (uintptr_t)rowp;
  int head = (int)(((16u - (addr & 15u)) & 15u) / sizeof(Elem));
  if (head > V) head = V;
  const int nchunk = (V - head) / PER;
  const int tail0 = head + nchunk * PER;
  if (tid < head) arg_take(best, g_val<Elem>(rowp, tid), tid);
  const u32x4* body = (const u32x4*)(rowp + head);
  for (int k0 = tid; k0 < nchunk; k0 += GA_THREADS * GA_UNROLL) {
    u32x4 v[GA_UNROLL];
#pragma unroll
    for (int u = 0; u < GA_UNROLL; ++u) {
      const int k = k0 + u * GA_THREADS;
      if (k < nchunk) v[u] = __builtin_nontemporal_load(body + k);
    }
#pragma unroll
    for (int u = 0; u < GA_UNROLL; ++u) {
      const int k = k0 + u * GA_THREADS;
      if (k < nchunk) {
        const int id0 = head + k * PER;
        if constexpr (sizeof(Elem) == 2) {
          u16x2 e = __builtin_bit_cast(u16x2, v[u][0] & 0x7F807F80u);
          e = __builtin_elementwise_max(e, __builtin_bit_cast(u16x2, v[u][1] & 0x7F807F80u));
          e = __builtin_elementwise_max(e, __builtin_bit_cast(u16x2, v[u][2] & 0x7F807F80u));
          e = __builtin_elementwise_max(e, __builtin_bit_cast(u16x2, v[u][3] & 0x7F807F80u));
          expmax = max(expmax, max((uint32_t)e[0], (uint32_t)e[1]));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            arg_take(best, __uint_as_float(v[u][j] << 16), id0 + 2 * j);
            arg_take(best, __uint_as_float(v[u][j] & 0xFFFF0000u), id0 + 2 * j + 1);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            expmax = max(expmax, (v[u][j] >> 23) & 0xFFu);
            arg_take(best, __uint_as_float(v[u][j]), id0 + j);
          }
        }
      }
    }
  }
  if (tid < V - tail0) arg_take(best, g_val<Elem>(rowp, tail0 + tid), tail0 + tid);
  if (tid < head || tid < V - tail0) {
    // head and tail elements also count for the exponent check
    const float hv = tid < head ? g_val<Elem>(rowp, tid) : 0.0f;
    const float tv = tid < V - tail0 ? g_val<Elem>(rowp, tail0 + tid) : 0.0f;
    if (!(fabsf(hv) < INFINITY) || !(fabsf(tv) < INFINITY)) expmax = 0xFFFFFFFFu;
  }

  // merge across the wave, then across waves
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) {
    ArgBest o{__shfl_xor(best.v, off, WAVE), __shfl_xor(best.i, off, WAVE)};
    best = arg_merge(best, o);
  }
  const int w = tid / WAVE, lane = tid & (WAVE - 1);
  if (lane == 0) {
    sv_[w] = best.v;
    si_[w] = best.i;
  }
  __syncthreads();
  ArgBest blk{sv_[0], si_[0]};
#pragma unroll
  for (int k = 1; k < GA_THREADS / WAVE; ++k) blk = arg_merge(blk, ArgBest{sv_[k], si_[k]});

  // inf or NaN somewhere (the all-ones exponent): look at the row again
  const bool is_bf = sizeof(Elem) == 2;
  const uint32_t allones = is_bf ? 0x7F80u : 0xFFu;
  const uint32_t seen = block_max<GA_THREADS>(expmax, su_);
  uint32_t nonfinite = 0;
  if (seen >= allones) {
    uint32_t bad = 0;
    int32_t first_ninf = INT32_MAX;
    for (int i = tid; i < V; i += GA_THREADS) {
      const float z = g_val<Elem>(rowp, i);
      if (z != z || z == INFINITY) bad = 1u;
      if (z == -INFINITY && i < first_ninf) first_ninf = i;
    }
    nonfinite = block_max<GA_THREADS>(bad, su_);
    const int32_t fn = block_min<GA_THREADS>(first_ninf, si_);
    // a row of -inf (and NaN) only: the lowest -inf position is the argmax
    if (blk.i == INT32_MAX) blk.i = fn;
  }
  if (blk.i == INT32_MAX) blk.i = 0;   // only NaN: unspecified, flagged
  if (tid == 0) a.out_tokens[row] = blk.i | (int32_t)(nonfinite << 31);
  if (row == 0 && a.accept_hist && tid <= a.gamma) a.accept_hist[tid] = 0u;
}

int launch_greedy_argmax(const GreedyArgs& a, hipStream_t st) {
  const int rows = a.B * (a.gamma + 1);
  if (a.bf16)
    hipLaunchKernelGGL(greedy_argmax_kernel<uint16_t>, dim3(rows), dim3(GA_THREADS), 0, st, a);
  else
    hipLaunchKernelGGL(greedy_argmax_kernel<float>, dim3(rows), dim3(GA_THREADS), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ __launch_bounds__(WAVE) void greedy_scan_kernel(GreedyArgs a) {
  const int b = blockIdx.x * WAVE + threadIdx.x;
  if (b >= a.B) return;
  const int g = a.gamma, G1 = g + 1;
  int32_t* out = a.out_tokens + (int64_t)b * G1;
  const int32_t* xs = a.draft_tokens + (int64_t)b * g;
  uint32_t flags = 0;
  int n = g;
  for (int i = 0; i < g; ++i) {
    const int32_t x = xs[i];
    if (x < 0 || x >= a.V) flags |= FLAG_TOKEN_RANGE;
    if (n == g && x != (out[i] & 0x7FFFFFFF)) n = i;
  }
  for (int i = 0; i < G1; ++i) {
    const int32_t e = out[i];
    if (e < 0) flags |= FLAG_NONFINITE;
    const int32_t am = e & 0x7FFFFFFF;
    out[i] = i <= n ? am : -1;
  }
  a.out_num_accepted[b] = n;
  if (a.out_flags) a.out_flags[b] = flags;
  if (a.accept_hist) atomicAdd(&a.accept_hist[n], 1u);
}

int launch_greedy_scan(const GreedyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(greedy_scan_kernel, dim3((a.B + WAVE - 1) / WAVE), dim3(WAVE), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
