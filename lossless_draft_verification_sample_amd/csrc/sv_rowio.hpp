// Row access shared by the kernels that re-read logit rows after the row
// statistics pass (final draw, overlap): groups of eight logits, the kept test
// against a row's statistics, LDS ban bitmaps, a table-driven fp64 exp and the
// per-wave queue of kept tokens.
#pragma once

#include "sv_common.hpp"

namespace sv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int GRP = 8;   // logits per group

// Token with logit z is kept in a row with statistics s: admissible (finite,
// not banned) and at or above the row's truncation threshold.
__device__ __forceinline__ bool is_kept(float z, const RowStat& s, bool banned) {
  return !banned && !(s.flags & FLAG_EMPTY) && z > -INFINITY && z < INFINITY && z >= s.tau;
}

// Eight consecutive logits starting at x0, as raw bits (-inf beyond the row).
template <typename Elem>
struct Group {
  u32x4 w[sizeof(Elem) == 2 ? 1 : 2];
};

// NT: the aligned bf16 load is nontemporal.
template <typename Elem, bool NT = false>
__device__ __forceinline__ void load_group(const void* row, int x0, int V, bool vec, Group<Elem>& g) {
  const Elem* e = (const Elem*)row;
  if constexpr (sizeof(Elem) == 2) {
    if (vec) {
      const u32x4* p = (const u32x4*)(e + x0);   // V % 8 == 0 on this path
      g.w[0] = NT ? __builtin_nontemporal_load(p) : *p;
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

// group_val for an index known only at run time: selects instead of a
// dynamically indexed register array (which would go through scratch).
template <typename Elem>
__device__ __forceinline__ float group_val_dyn(const Group<Elem>& g, int j) {
  if constexpr (sizeof(Elem) == 2) {
    const uint32_t d01 = (j & 2) ? g.w[0][1] : g.w[0][0];
    const uint32_t d23 = (j & 2) ? g.w[0][3] : g.w[0][2];
    const uint32_t d = (j & 4) ? d23 : d01;
    return bf16_to_f32((j & 1) ? d >> 16 : d & 0xFFFFu);
  } else {
    const bool hi = (j & 4) != 0;
    const uint32_t d0 = hi ? g.w[1][0] : g.w[0][0], d1 = hi ? g.w[1][1] : g.w[0][1];
    const uint32_t d2 = hi ? g.w[1][2] : g.w[0][2], d3 = hi ? g.w[1][3] : g.w[0][3];
    const uint32_t d01 = (j & 1) ? d1 : d0;
    const uint32_t d23 = (j & 1) ? d3 : d2;
    return __uint_as_float((j & 2) ? d23 : d01);
  }
}

// exp(a) in fp64 for a <= about 0, table-driven (P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989): a = (256 k' + j) ln2 / 256 + r with
// |r| <= ln2 / 512, so e^a = 2^k' * 2^(j/256) * e^r; 2^(j/256) comes from a
// 256-entry LDS table and e^r - 1 from its degree-4 Taylor polynomial
// (remainder below 4e-17 relative). Error a few ulp.
__device__ __forceinline__ double exp_tab(double a, const double* tab) {
  a = fmax(a, -1000.0);                                    // exp(-1000) is 0 in fp64
  const double kf = rint(a * 0x1.71547652b82fep+8);        // 256 / ln2
  double r = fma(-kf, 0x1.62e42fef80000p-9, a);            // head of ln2 / 256 (34 bits)
  r = fma(-kf, 0x1.1cf79abc9e3b4p-44, r);                  // tail of ln2 / 256
  double q = fma(r, 1.0 / 24.0, 1.0 / 6.0);
  q = fma(q, r, 0.5);
  q = fma(q, r, 1.0);
  q *= r;                                                  // e^r - 1
  const int k = (int)kf;
  const double t = tab[k & 255];
  return ldexp(fma(t, q, t), k >> 8);
}

// The 2^(j/256) table of exp_tab, filled by the first 256 threads.
__device__ __forceinline__ void exp_table_fill(double* tab) {
  if (threadIdx.x < 256) tab[threadIdx.x] = exp2((double)threadIdx.x * (1.0 / 256.0));
}

// Marks the banned ids that fall in [c0, c0 + len) in an LDS bitmap of len / 32
// words. The list is raw: ids outside [0, V) are padding and duplicates set the
// same bit. `first` is element threadIdx.x of the list, loaded by the caller.
__device__ __forceinline__ void mark_bans(uint32_t* bm, int len, const int32_t* bl, int nb,
                                          int32_t first, int c0, int V) {
  for (int k = threadIdx.x; k < len / 32; k += blockDim.x) bm[k] = 0u;
  __syncthreads();
  for (int j = threadIdx.x; j < nb; j += blockDim.x) {
    const int32_t id = j == (int)threadIdx.x ? first : bl[j];
    if (id >= c0 && id < V && id - c0 < len) {
      const int o = id - c0;
      atomicOr(&bm[o >> 5], 1u << (o & 31));
    }
  }
  __syncthreads();
}

// Ban bits of the eight tokens at offset o (a multiple of 8) of the bitmap.
__device__ __forceinline__ uint32_t bm_group(const uint32_t* bm, int o) {
  return (bm[o >> 5] >> (o & 31)) & 0xFFu;
}

__device__ __forceinline__ double wave_total(double v) {
  return lane63(wave_scan_dpp(v, 0.0, [](double x, double y) { return x + y; }));
}

// A kept token of a wave's sub-chunk, queued for dense evaluation.
struct alignas(16) KeptTok {
  int32_t x;
  float zt, zd;
  int32_t pad;
};

// Marks, in an LDS bitmap of len / 32 words over [c0, c0 + len), the ids a row
// penalizes: entries 0..H-1 of `hist` and the proposals props[0..np-1] (ids
// outside [0, V) are padding, duplicates set the same bit).
__device__ __forceinline__ void mark_pen(uint32_t* bm, int len, const int32_t* hist, int H,
                                         const int32_t* props, int np, int c0, int V) {
  for (int k = threadIdx.x; k < len / 32; k += blockDim.x) bm[k] = 0u;
  __syncthreads();
  for (int j = threadIdx.x; j < H + np; j += blockDim.x) {
    const int32_t id = j < H ? hist[j] : props[j - H];
    if (id >= c0 && id < V && id - c0 < len) {
      const int o = id - c0;
      atomicOr(&bm[o >> 5], 1u << (o & 31));
    }
  }
  __syncthreads();
}

// Replaces the finite logits of the marked tokens of a group (bit e: token e)
// by their repetition-penalized value.
template <typename Elem>
__device__ __forceinline__ void penalize_group(Group<Elem>& g, uint32_t bits, float theta) {
  if (!bits) return;
#pragma unroll
  for (int e = 0; e < GRP; ++e) {
    if (!((bits >> e) & 1u)) continue;
    const float z = group_val<Elem>(g, e);
    if (!(z > -INFINITY && z < INFINITY)) continue;
    const uint32_t v = __float_as_uint(pen_apply(z, theta, sizeof(Elem) == 2));
    if constexpr (sizeof(Elem) == 2) {
      const int sh = 16 * (e & 1);
      g.w[0][e >> 1] = (g.w[0][e >> 1] & ~(0xFFFFu << sh)) | ((v >> 16) << sh);
    } else {
      g.w[e >> 2][e & 3] = v;
    }
  }
}

// A token kept in a leading row, queued in LDS until the other row's logit at
// the same position is read.
struct alignas(8) QueuedTok {
  int32_t x;
  float z;   // the leading row's logit
};

// One logit of a row as float (a single-element read). Nontemporal: these
// gathers hit scattered cache lines that nothing reads again, and so they do
// not displace the lines of the rows being streamed.
template <typename Elem>
__device__ __forceinline__ float load_logit(const void* row, int x) {
  if constexpr (sizeof(Elem) == 2) return bf16_to_f32(__builtin_nontemporal_load((const uint16_t*)row + x));
  return __builtin_nontemporal_load((const float*)row + x);
}

// Orders a wave's LDS writes before its later LDS reads (and the reverse).
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace sv
