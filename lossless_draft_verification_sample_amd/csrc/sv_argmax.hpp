// Argmax of one logit row for greedy verification ("Drafters and Speculative
// Decoding: Useful Tokens, Correct State", section "Greedy verification"): the
// largest logit, the lowest token id on exact ties (-0 and +0 tie), NaN and
// banned ids excluded. One workgroup of NT threads streams the row once with
// 16-byte loads; each lane keeps the first position of its largest value
// (lanes visit their positions in increasing order, so a strict > keeps the
// lowest id) and the workgroup merges (value, id) pairs. Bans and penalties are
// consulted only when that winner is banned or penalized: the row is then
// streamed again with a set lookup whenever a value beats a lane's best.
#pragma once

#include <type_traits>

#include "sv_bans.hpp"
#include "sv_common.hpp"

namespace sv {

struct ArgBest {
  float v;
  int32_t i;
};

// (value desc, id asc) merge of two candidates; id INT32_MAX means none.
__device__ __forceinline__ ArgBest arg_merge(ArgBest a, ArgBest b) {
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

template <typename Elem>
__device__ __forceinline__ float am_val(const Elem* p, int i) {
  if constexpr (sizeof(Elem) == 2) return bf16_to_f32(p[i]);
  return p[i];
}

// Result of row_argmax: the argmax id (-1 when no token is admissible) and
// whether the row holds NaN or +inf.
struct ArgResult {
  int32_t arg;
  bool nonfinite;
};

// `tab` is the LDS hash set of the request's banned ids (used only when BANS
// and tab is set). With PEN, the ids in the hash set `ptab` (when set) compete
// with their repetition-penalized logit (pen_apply with `theta`); the penalty
// never raises a logit, so in the checking pass it is applied only when a
// value beats the lane's best. The scratch arrays hold NT / WAVE entries each. Every thread gets the
// result.
template <typename Elem, int NT, int UNROLL, bool BANS, bool PEN = false>
__device__ ArgResult row_argmax(const Elem* rowp, int V, const uint32_t* tab, float* sv,
                                int32_t* si, uint32_t* su, const uint32_t* ptab = nullptr,
                                float theta = 1.0f) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  constexpr int PER = 16 / sizeof(Elem);
  const int tid = threadIdx.x;
  uint32_t expmax = 0;   // largest exponent field seen (all ones: inf or NaN present)
  const uintptr_t addr = (uintptr_t)rowp;
  int head = (int)(((16u - (addr & 15u)) & 15u) / sizeof(Elem));
  if (head > V) head = V;
  const int nchunk = (V - head) / PER;
  const int tail0 = head + nchunk * PER;
  const u32x4* body = (const u32x4*)(rowp + head);

  // One pass over the row, merged over the workgroup. With CHECK, a value that
  // beats the lane's best is looked up in the ban and penalty sets; without,
  // every value competes as it is.
  auto pass = [&](auto check_c) -> ArgBest {
    constexpr bool CHECK = decltype(check_c)::value;
    ArgBest best{-INFINITY, INT32_MAX};
    auto take = [&](float v, int32_t i) {
      if (v > best.v) {
        if constexpr (CHECK) {
          if (BANS && tab && ht_has(tab, i)) return;
          if (PEN && ptab && ht_has(ptab, i)) {
            v = pen_apply(v, theta, sizeof(Elem) == 2);
            if (!(v > best.v)) return;
          }
        }
        best.v = v;
        best.i = i;
      }
    };
    if (tid < head) take(am_val<Elem>(rowp, tid), tid);
    // Software-pipelined stream: while one buffer of UNROLL chunks is scanned,
    // the loads of the other are in flight.
    constexpr int STEP = NT * UNROLL;
    u32x4 va[UNROLL], vb[UNROLL];
    auto ld = [&](u32x4 (&v)[UNROLL], int k0) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int k = k0 + u * NT;
        if (k < nchunk) v[u] = __builtin_nontemporal_load(body + k);
      }
    };
    auto scan = [&](const u32x4 (&v)[UNROLL], int k0) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int k = k0 + u * NT;
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
              take(__uint_as_float(v[u][j] << 16), id0 + 2 * j);
              take(__uint_as_float(v[u][j] & 0xFFFF0000u), id0 + 2 * j + 1);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              expmax = max(expmax, (v[u][j] >> 23) & 0xFFu);
              take(__uint_as_float(v[u][j]), id0 + j);
            }
          }
        }
      }
    };
    int k0 = tid;
    if (k0 < nchunk) ld(va, k0);
    while (k0 < nchunk) {
      if (k0 + STEP < nchunk) ld(vb, k0 + STEP);
      scan(va, k0);
      k0 += STEP;
      if (k0 >= nchunk) break;
      if (k0 + STEP < nchunk) ld(va, k0 + STEP);
      scan(vb, k0);
      k0 += STEP;
    }
    if (tid < V - tail0) take(am_val<Elem>(rowp, tail0 + tid), tail0 + tid);
    if (tid < head || tid < V - tail0) {
      // head and tail elements also count for the exponent check
      const float hv = tid < head ? am_val<Elem>(rowp, tid) : 0.0f;
      const float tv = tid < V - tail0 ? am_val<Elem>(rowp, tail0 + tid) : 0.0f;
      if (!(fabsf(hv) < INFINITY) || !(fabsf(tv) < INFINITY)) expmax = 0xFFFFFFFFu;
    }
    // merge across the wave, then across waves
#pragma unroll
    for (int off = WAVE / 2; off > 0; off >>= 1) {
      ArgBest o{__shfl_xor(best.v, off, WAVE), __shfl_xor(best.i, off, WAVE)};
      best = arg_merge(best, o);
    }
    const int w = tid / WAVE, lane = tid & (WAVE - 1);
    __syncthreads();   // the scratch may still be read by a previous caller or pass
    if (lane == 0) {
      sv[w] = best.v;
      si[w] = best.i;
    }
    __syncthreads();
    ArgBest blk{sv[0], si[0]};
#pragma unroll
    for (int k = 1; k < NT / WAVE; ++k) blk = arg_merge(blk, ArgBest{sv[k], si[k]});
    return blk;
  };

  // Sets are looked up only if the plain argmax is banned or penalized. A
  // ban removes values and a penalty never raises one, so a plain winner
  // that is in neither set is also the lowest-id largest admissible value.
  ArgBest blk = pass(std::false_type{});
  if constexpr (BANS || PEN) {
    const bool hit = blk.i != INT32_MAX && ((BANS && tab && ht_has(tab, blk.i)) ||
                                            (PEN && ptab && ht_has(ptab, blk.i)));
    if (hit) blk = pass(std::true_type{});
  }

  // inf or NaN somewhere (the all-ones exponent): look at the row again
  const uint32_t allones = sizeof(Elem) == 2 ? 0x7F80u : 0xFFu;
  const uint32_t seen = block_max<NT>(expmax, su);
  bool nonfinite = false;
  if (seen >= allones) {
    uint32_t bad = 0;
    int32_t first_ninf = INT32_MAX;
    for (int i = tid; i < V; i += NT) {
      const float z = am_val<Elem>(rowp, i);
      if (z != z || z == INFINITY) bad = 1u;
      if (z == -INFINITY && i < first_ninf && !(BANS && tab && ht_has(tab, i))) first_ninf = i;
    }
    nonfinite = block_max<NT>(bad, su) != 0u;
    const int32_t fn = block_min<NT>(first_ninf, si);
    // only -inf (and NaN) among the admissible tokens: the lowest -inf id
    if (blk.i == INT32_MAX) blk.i = fn;
  }
  return ArgResult{blk.i == INT32_MAX ? -1 : blk.i, nonfinite};
}

}  // namespace sv
