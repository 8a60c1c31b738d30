// Row statistics of the sampler-transformed target and draft rows.
//
// For every one of the B*(2*gamma+1) logit rows this kernel computes what the
// acceptance test and the final draw need to evaluate p(x) or q(x) of any token
// of the row: the largest kept logit m, the truncation threshold tau and the
// log-normaliser lse of the tempered kept logits (transforms: bans,
// temperature, top-k, top-p - "Speculative Decoding - Turn guesses into
// parallel work", section "Greedy, sampling and the real sampler").
//
// One workgroup owns one row and reads it from HBM exactly once.
//
// bf16 rows (count-histogram path). A bf16 logit has only 65536 possible
// values, and p(x) depends on x only through its logit. The workgroup
// therefore streams the row once and counts, in LDS, how often each logit
// value occurs (one LDS atomic and a few packed 16-bit integer ops per logit;
// no exp per logit). Counts cover every value with 2^-23 <= |z| < 2^9 (4096
// values per sign) plus exact zeros. From the counts the epilogue gets
//   m      = largest counted value,
//   Z      = sum_v count(v) * exp((v - m) / T) in fp64 (one exp per distinct value),
//   top-k  = the value where the running count from the top reaches k,
//   top-p  = the last value whose strictly-larger mass is < top_p * Z,
// all exact (integer counts, fp64 sums in a fixed order, so the result is also
// bitwise reproducible). Banned ids are subtracted from the counts afterwards;
// the raw ban list is first de-duplicated through a hash set in LDS (the space
// of the histogram, before it is cleared). Nonzero values below
// 2^-23 in magnitude are rare but do occur in large rows; they are counted with
// the zero bin and kept, up to TINY_MAX of them, in a small list whose exact
// contribution is added in a fixed (sorted) order. A row holding a value of
// magnitude >= 2^9, more tiny values than the list holds, or a truncation cut
// that falls among the tiny values is handed to the generic path.
//
// fp32 rows (generic path). A first streaming pass finds the maximum and the
// count. An untruncated row also sums, per lane, exp2(z*log2e/T - ref) against
// an integer reference ref that only ever increases, so rescaling is an exact
// power of two, and the per-lane sums are combined exactly at the end. A
// truncated row takes its cuts from a radix selection over the
// order-preserving integer keys of the values (8-bit digits: four passes for
// fp32 keys, two for the 16-bit keys of bf16 rows), whose per-digit counts and
// fixed-point mass sums are exact integers; the kept set's mass comes from
// the same sums. Bans are removed from those sums exactly, or looked up in
// the LDS hash set when a repetition penalty changes values. Exact in the
// same sense as the histogram path, only slower.
//
// Each row also evaluates the probability of its proposal token (target row
// i < gamma: p_i(x_i); draft row i: q_i(x_i)), which is all the acceptance walk
// needs from the row, and target row i draws the request's uniform of slot i
// (Philox, unless the caller passed the uniforms), so that the walk only loads
// them.

#include "sv_argmax.hpp"
#include "sv_bans.hpp"
#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

#ifndef SV_RS_THREADS
#define SV_RS_THREADS 512
#endif
#ifndef SV_RS_UNROLL
#define SV_RS_UNROLL 4
#endif
// One workgroup per row; each thread keeps four to eight 16-byte loads in
// flight (two buffers of RS_UNROLL chunks: one loading, one being counted).
constexpr int RS_THREADS = SV_RS_THREADS;
constexpr int RS_UNROLL = SV_RS_UNROLL;

// Count-histogram window for bf16 logits.
constexpr uint32_t HB_BASE = 104u << 7;       // bf16 |bits| of 2^-23
constexpr uint32_t HB_WIN = 32u * 128u;       // 32 binades x 128 mantissas per sign
constexpr uint32_t HB_NEG = HB_WIN + 4u;      // first bin of the negative half (16-byte aligned)
constexpr uint32_t HB_ZERO = HB_WIN;          // rank of zero; bin HB_WIN is a dump bin
constexpr uint32_t HB_BINS = HB_NEG + HB_WIN + 1u;
constexpr int HB_RANKS = 2 * HB_WIN + 1;      // value-ordered ranks: +window, zero, -window
constexpr uint32_t TINY_MAX = 64;             // tiny values tracked exactly per row

// The ban set and the penalty set each hold at most HT_MAX_IDS ids (the host
// bounds both lists), and both fit in the histogram storage before the stream.
static_assert(HT_MAX_IDS >= 2048 && 2 * HT_SLOTS <= HB_BINS, "hash set sizes");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Ranks order the counted values from the largest down: ranks 0..4095 are the
// positive window (bin 4095 - r), rank 4096 is zero, ranks 4097..8192 the
// negative window (bin HB_NEG + r - 4097).
__device__ __forceinline__ float hb_value_of_rank(int r) {
  if (r < (int)HB_WIN) return bf16_to_f32(HB_WIN - 1u - (uint32_t)r + HB_BASE);
  if (r == (int)HB_ZERO) return 0.0f;
  return bf16_to_f32(0x8000u | ((uint32_t)r - (HB_WIN + 1u) + HB_BASE));
}

struct alignas(16) WaveSlot {
  uint32_t n;     // admissible count of the wave  | exchange 2/3: selected rank
  int32_t top;    // top rank of the wave           | (unused)
  double z;       // mass of the wave (rel. to its top value) | prefix mass
};

struct RowShared {
  alignas(16) uint32_t hist[HB_BINS];
  uint32_t zero_cnt;   // exact zeros and tiny values
  uint32_t nonfinite;
  uint32_t special;
  uint32_t tiny_n;
  uint16_t tiny[TINY_MAX];
  double tiny_mass;
  float tiny_top;
  WaveSlot x1[RS_THREADS / WAVE], x2[RS_THREADS / WAVE], x3[RS_THREADS / WAVE];
  uint32_t xban;       // the row's proposal token is banned
  uint32_t xpen;       // the row's proposal token is penalized
  double dscr[RS_THREADS / WAVE];
  float fscr[RS_THREADS / WAVE];
  uint32_t uscr[RS_THREADS / WAVE];
  int32_t iscr[RS_THREADS / WAVE];
  // generic path: one 8-bit digit level of the radix selection
  uint32_t rcnt[256];
  unsigned long long rmh[256], rml[256];
  uint32_t rsel_d, rsel_c;
  unsigned long long rsel_h, rsel_l;
  double rsel_target;
};

// Exact classification of one bf16 logit that fell outside the counted window.
__device__ __forceinline__ void hb_classify_slow(uint32_t bits, RowShared& sh) {
  const uint32_t ae = bits & 0x7FFFu;
  if (ae - HB_BASE < HB_WIN) return;          // inside the window: already counted
  if (ae == 0u) {
    atomicAdd(&sh.zero_cnt, 1u);              // +0 and -0
  } else if ((ae & 0x7F80u) == 0x7F80u) {
    if (bits != 0xFF80u) sh.nonfinite = 1u;   // NaN or +inf; -inf is a masked token
  } else if (ae < HB_BASE) {
    atomicAdd(&sh.zero_cnt, 1u);              // tiny: counted with zero, listed exactly
    const uint32_t k = atomicAdd(&sh.tiny_n, 1u);
    if (k < TINY_MAX)
      sh.tiny[k] = (uint16_t)bits;
    else
      sh.special = 1u;
  } else {
    sh.special = 1u;                          // |z| >= 2^9
  }
}

// Count both bf16 halves of one dword; returns the out-of-window marker bits.
__device__ __forceinline__ uint32_t hb_count_pair(uint32_t d, uint32_t* hist) {
  const u16x2 x = __builtin_bit_cast(u16x2, d);
  u16x2 t = (x & (unsigned short)0x7FFF) - (unsigned short)HB_BASE;
  t = __builtin_elementwise_min(t, (u16x2)(unsigned short)HB_WIN);
  const u16x2 s = x >> (unsigned short)15;
  const u16x2 bin = s * (unsigned short)HB_NEG + t;
  const uint32_t b2 = __builtin_bit_cast(uint32_t, bin);
  atomicAdd(&hist[b2 & 0xFFFFu], 1u);
  atomicAdd(&hist[b2 >> 16], 1u);
  return __builtin_bit_cast(uint32_t, t) & 0x10001000u;
}

__device__ __forceinline__ void hb_count_one(uint32_t bits, RowShared& sh) {
  const uint32_t ae = bits & 0x7FFFu;
  const uint32_t t = ae - HB_BASE;
  if (t < HB_WIN)
    atomicAdd(&sh.hist[t + ((bits >> 15) ? HB_NEG : 0u)], 1u);
  else
    hb_classify_slow(bits, sh);
}

// ------------------------------------------------------------------ generic path

template <typename Elem>
__device__ __forceinline__ float elem_value(Elem e);
template <>
__device__ __forceinline__ float elem_value<uint16_t>(uint16_t e) {
  return bf16_to_f32(e);
}
template <>
__device__ __forceinline__ float elem_value<float>(float e) {
  return e;
}

// Calls f(z, id) for every element of the row: 16-byte vector loads in the
// body, software-pipelined (each thread's next GEN_U chunks are in flight
// while the current ones are processed).
constexpr int GEN_U = 2;
template <typename Elem, typename F>
__device__ __forceinline__ void for_each_elem(const Elem* rowp, int V, F&& f) {
  constexpr int PER = 16 / sizeof(Elem);
  constexpr int STEP = RS_THREADS * GEN_U;
  const int tid = threadIdx.x;
  const uintptr_t addr = (uintptr_t)rowp;
  int head = (int)(((16u - (addr & 15u)) & 15u) / sizeof(Elem));
  if (head > V) head = V;
  const int nchunk = (V - head) / PER;
  const int tail0 = head + nchunk * PER;
  if (tid < head) f(elem_value<Elem>(rowp[tid]), tid);
  if (tid < V - tail0) f(elem_value<Elem>(rowp[tail0 + tid]), tail0 + tid);
  const u32x4* body = (const u32x4*)(rowp + head);
  u32x4 va[GEN_U], vb[GEN_U];
  auto ld = [&](u32x4(&v)[GEN_U], int k0) {
#pragma unroll
    for (int u = 0; u < GEN_U; ++u) {
      const int k = k0 + u * RS_THREADS;
      if (k < nchunk) v[u] = __builtin_nontemporal_load(body + k);   // streamed: nontemporal
    }
  };
  auto run = [&](const u32x4(&v)[GEN_U], int k0) {
#pragma unroll
    for (int u = 0; u < GEN_U; ++u) {
      const int k = k0 + u * RS_THREADS;
      if (k >= nchunk) continue;
      const int id0 = head + k * PER;
      if constexpr (sizeof(Elem) == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = v[u][j];
          f(bf16_to_f32(w & 0xFFFFu), id0 + 2 * j);
          f(bf16_to_f32(w >> 16), id0 + 2 * j + 1);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = v[u][j];
          f(__uint_as_float(w), id0 + j);
        }
      }
    }
  };
  int k0 = tid;
  if (k0 < nchunk) ld(va, k0);
  while (k0 < nchunk) {
    if (k0 + STEP < nchunk) ld(vb, k0 + STEP);
    run(va, k0);
    k0 += STEP;
    if (k0 >= nchunk) break;
    if (k0 + STEP < nchunk) ld(va, k0 + STEP);
    run(vb, k0);
    k0 += STEP;
  }
}

// Admissibility test of the generic path: finite and not in the ban set.
struct GenericCtx {
  const uint32_t* tab;    // LDS hash set, or nullptr when the request bans nothing
  const uint32_t* ptab;   // LDS hash set of the penalized ids, or nullptr
  float theta;            // their repetition penalty
  bool bf16;              // penalized values are rounded to bf16
  // The banned values are listed in LDS behind the ban set (gen_banned_values)
  // for the radix cut to take out of its sums.
  bool sub_bans;
  __device__ __forceinline__ bool admissible(float z, int id) const {
    // finite and not banned; NaN fails both comparisons
    if (!(z > -INFINITY && z < INFINITY)) return false;
    return !tab || !ht_has(tab, id);
  }
  // the logit of an admissible token after the repetition penalty
  __device__ __forceinline__ float value(float z, int id) const {
    return (ptab && ht_has(ptab, id)) ? pen_apply(z, theta, bf16) : z;
  }
};

// Order-preserving keys for the radix selection and the bisection: 16 bits
// for bf16 rows, 32 for fp32.
template <typename Elem>
__device__ __forceinline__ uint32_t gkey(float v) {
  return sizeof(Elem) == 2 ? (f32_key(v) >> 16) : f32_key(v);
}
// The smallest float whose key is k (so z >= gval(k) <=> key(z) >= k for row values).
template <typename Elem>
__device__ __forceinline__ float gval(uint32_t k) {
  if (sizeof(Elem) == 2) {
    const uint32_t k32 = k << 16;
    return f32_from_key((k32 & 0x80000000u) ? k32 : (k32 | 0xFFFFu));
  }
  return f32_from_key(k);
}

// 2^x in fp64 for x <= about 0 (masses relative to the row's reference), to
// about an ulp: x = k + r with k = rint(x) and r exact (|r| <= 1/2); r ln 2 in
// double-double through an fma with ln 2 split into a head and a tail; e^t - 1
// from its degree-13 Taylor polynomial (|t| <= 0.35, remainder below 1e-17).
__device__ __forceinline__ double exp2_neg(double x) {
  x = fmax(x, -1100.0);                       // 2^-1100 is 0 in fp64
  const double k = rint(x);
  const double r = x - k;
  const double t = fma(r, 0x1.62e42fefa39efp-1, r * 0x1.abc9e3b39803fp-56);
  double q = fma(t, 1.0 / 6227020800.0, 1.0 / 479001600.0);
  q = fma(q, t, 1.0 / 39916800.0);
  q = fma(q, t, 1.0 / 3628800.0);
  q = fma(q, t, 1.0 / 362880.0);
  q = fma(q, t, 1.0 / 40320.0);
  q = fma(q, t, 1.0 / 5040.0);
  q = fma(q, t, 1.0 / 720.0);
  q = fma(q, t, 1.0 / 120.0);
  q = fma(q, t, 1.0 / 24.0);
  q = fma(q, t, 1.0 / 6.0);
  q = fma(q, t, 0.5);
  q = fma(q, t, 1.0);
  q *= t;                                     // e^t - 1
  return ldexp(1.0 + q, (int)k);
}

// The same 2^x through a 256-entry table of 2^(j/256) (P. T. P. Tang, "Table-
// driven implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989): x = m + j/256 + r with t = rint(256 x)
// and r = x - t/256 exact (|r| <= 1/512); 2^r = e^u with u = r ln 2 in
// double-double, e^u - 1 from its degree-4 Taylor polynomial (|u| < 0.0014,
// remainder below 4e-17 relative).
__device__ __forceinline__ double exp2_tab(double x, const double* tab) {
  x = fmax(x, -1100.0);
  const double t = rint(x * 256.0);
  const double r = fma(t, -1.0 / 256.0, x);
  const double u = fma(r, 0x1.62e42fefa39efp-1, r * 0x1.abc9e3b39803fp-56);
  double q = fma(u, 1.0 / 24.0, 1.0 / 6.0);
  q = fma(q, u, 0.5);
  q = fma(q, u, 1.0);
  q *= u;                                     // e^u - 1
  const int ti = (int)t;
  const double tj = tab[ti & 255];
  return ldexp(fma(tj, q, tj), ti >> 8);
}

// A mass m in [0, 1] in fixed point: m = (h + l * 2^-40) * 2^-40 up to 2^-80.
// Sums of h and of l are exact 64-bit integer sums (no carry between them is
// needed while fewer than 2^24 masses are added), so they do not depend on
// the order of the additions.
struct Fix {
  unsigned long long h, l;
};
__device__ __forceinline__ Fix fix_of(double m) {
  const double a = m * 0x1.0p40;
  const double hf = floor(a);
  Fix f;
  f.h = (unsigned long long)hf;
  f.l = (unsigned long long)((a - hf) * 0x1.0p40);
  return f;
}
__device__ __forceinline__ Fix fix_add(Fix a, Fix b) {
  a.h += b.h;
  a.l += b.l;
  return a;
}
__device__ __forceinline__ double fix_val(Fix f) {
  return (double)f.h * 0x1.0p-40 + (double)f.l * 0x1.0p-80;
}
// Rows with fewer elements than this take the radix selection (exact
// fixed-point sums); longer ones the bisection.
constexpr int RADIX_MAX_V = 1 << 24;

// The banned values a radix cut takes out of its sums: entry k of thread t
// (list index t + k * RS_THREADS) at k * RS_THREADS + t, NaN when that entry
// is not the one owner of a valid id. They sit behind the ban set, in the
// histogram storage that only a repetition penalty's set would use.
constexpr int GEN_BPT = (int)HT_MAX_IDS / RS_THREADS;   // list entries per thread
static_assert(GEN_BPT * RS_THREADS >= (int)HT_MAX_IDS, "ban entries per thread");
static_assert(GEN_BPT * RS_THREADS <= (int)HT_SLOTS, "banned values fit behind the set");
__device__ __forceinline__ float* gen_banned_values(uint32_t* hist) {
  return (float*)(hist + HT_SLOTS);
}

// Not inlined: its registers stay out of the count-histogram path's
// allocation (every bf16 row takes that path; only fp32 rows and rare bf16
// rows come here).
template <typename Elem>
__device__ __noinline__ RowStat row_generic(const Elem* rowp, int V, const SamplerDev s,
                                            const GenericCtx g, RowShared& sh, RowStat out) {
  const double c2 = 1.4426950408889634 / (double)s.temperature;  // log2(e) / T
  // A truncating sampler takes its cuts and the kept set's mass from the radix
  // selection below, so the first pass needs no exp.
  const bool radix_cut = V < RADIX_MAX_V && (s.top_k > 0 || s.top_p < 1.0f);
  // Bans of a radix cut without a repetition penalty: the passes take every
  // finite element and then remove the banned ones, each distinct id once by
  // its owner thread, from the integer counts and fixed-point masses (exact),
  // instead of a set lookup per element.
  const bool sub_bans = g.sub_bans;
  const float* zb = gen_banned_values(sh.hist) + threadIdx.x;   // this thread's entries, stride RS_THREADS
  // pass 1: max, min, count and (without a radix cut) the exp-sum against
  // per-lane integer references
  float mx = -INFINITY, mn = INFINITY;
  uint32_t cnt = 0, bad = 0;
  double ref = -INFINITY, acc = 0.0;
  for_each_elem<Elem>(rowp, V, [&](float z, int id) {
    if (z != z || z == INFINITY) bad = 1u;
    if (sub_bans ? !(z > -INFINITY && z < INFINITY) : !g.admissible(z, id)) return;
    z = g.value(z, id);
    ++cnt;
    mn = fminf(mn, z);
    if (z > mx) mx = z;
    if (radix_cut) return;
    const double e = (double)z * c2;
    if (e > ref) {
      const double nr = ceil(e);
      if (ref > -INFINITY) acc = ldexp(acc, (int)fmax(ref - nr, -2000.0));
      ref = nr;
    }
    acc += exp2_neg(e - ref);
  });
  mx = block_max<RS_THREADS>(mx, sh.fscr);
  mn = block_min<RS_THREADS>(mn, sh.fscr);
  cnt = block_sum<RS_THREADS>(cnt, sh.uscr);
  bad = block_max<RS_THREADS>(bad, sh.uscr);
  if (sub_bans) {
    uint32_t bc = 0u;
    float bm = -INFINITY;
#pragma unroll
    for (int k = 0; k < GEN_BPT; ++k) {
      const float z = zb[k * RS_THREADS];
      if (z > -INFINITY && z < INFINITY) {
        ++bc;
        bm = fmaxf(bm, z);
      }
    }
    cnt -= block_sum<RS_THREADS>(bc, sh.uscr);
    if (block_max<RS_THREADS>(bm, sh.fscr) >= mx) {
      // a banned token holds the maximum: one more pass, with lookups
      float m2 = -INFINITY;
      for_each_elem<Elem>(rowp, V, [&](float z, int id) {
        if (g.admissible(z, id) && z > m2) m2 = z;
      });
      mx = block_max<RS_THREADS>(m2, sh.fscr);
    }
  }
  // the reference exponent: ceil of the largest z / T in log2 units (what the
  // per-lane references give)
  const double rmax = radix_cut ? (mx > -INFINITY ? ceil((double)mx * c2) : -INFINITY)
                                : block_max<RS_THREADS>(ref, sh.dscr);
  out.flags |= bad ? FLAG_NONFINITE : 0u;
  if (cnt == 0u) {
    out.m = -INFINITY;
    out.tau = -INFINITY;
    out.lse = -INFINITY;
    out.flags |= FLAG_EMPTY;
    out.path = 1u;
    return out;
  }
  double Z = radix_cut ? 0.0
                       : block_sum<RS_THREADS>(
                             ref > -INFINITY ? ldexp(acc, (int)fmax(ref - rmax, -2000.0)) : 0.0,
                             sh.dscr);
  // mass (relative to 2^rmax) and count of the admissible values >= thr
  auto mass_ge = [&](float thr) -> double {
    double a = 0.0;
    for_each_elem<Elem>(rowp, V, [&](float z, int id) {
      if (!g.admissible(z, id)) return;
      z = g.value(z, id);
      if (z >= thr) a += exp2_neg((double)z * c2 - rmax);
    });
    return block_sum<RS_THREADS>(a, sh.dscr);
  };
  auto count_ge = [&](float thr) -> uint32_t {
    uint32_t a = 0;
    for_each_elem<Elem>(rowp, V, [&](float z, int id) {
      if (!g.admissible(z, id)) return;
      if (g.value(z, id) >= thr) ++a;
    });
    return block_sum<RS_THREADS>(a, sh.uscr);
  };
  float tau = -INFINITY;
  bool trunc = false;
  if (V < RADIX_MAX_V && ((s.top_k > 0 && (uint32_t)s.top_k < cnt) || s.top_p < 1.0f)) {
    // Radix selection over the order-preserving keys, most significant 8-bit
    // digit first: one pass over the row per digit (2 for bf16 keys, 4 for
    // fp32). Each pass counts, per digit value, the admissible elements whose
    // higher digits equal the part of the threshold fixed so far (and the
    // fixed-point sum of their masses exp(z/T) relative to 2^rmax); wave 0 then
    // picks the digit where the running total from the top reaches what is
    // needed. Top-k: the k-th largest key; top-p (after top-k, over keys at or
    // above its cut): the largest key whose mass at or above it reaches
    // top_p * Z. Counts and fixed-point sums are exact, so the result does not
    // depend on the order of the LDS additions.
    constexpr int KB = sizeof(Elem) == 2 ? 16 : 32;
    // Without a penalty set, the histogram storage around the banned values
    // is free during the levels (the ban set is not looked up there): it
    // holds MC copies of the count and mass bins, lane l adding to copy
    // l % MC, merged before each pick (a wave's lanes crowd into the few
    // digits that normal logits' exponents select, and LDS atomics to one
    // address serialise), the exp table, and a list of the values that share
    // the first two digits of an fp32 key (see `lmode` below).
    constexpr int MC = 4;
    constexpr uint32_t LOFF = HT_SLOTS + GEN_BPT * RS_THREADS + 2 * 256 + 256 * MC;
    constexpr uint32_t LCAP = HB_BINS - LOFF - 1u;
    static_assert(2 * 256 * MC * 2 <= (int)HT_SLOTS && LOFF + 1u + 256u <= HB_BINS,
                  "level storage");
    const bool spread = !g.ptab;
    unsigned long long* cmh = (unsigned long long*)sh.hist;   // [256][MC]
    unsigned long long* cml = cmh + 256 * MC;                  // [256][MC]
    double* etab = (double*)(sh.hist + HT_SLOTS + GEN_BPT * RS_THREADS);
    uint32_t* ccnt = sh.hist + HT_SLOTS + GEN_BPT * RS_THREADS + 2 * 256;   // [256][MC]
    uint32_t* lcnt = sh.hist + LOFF;
    float* lst = (float*)(sh.hist + LOFF + 1u);
    if (spread && threadIdx.x < 256) etab[threadIdx.x] = exp2((double)threadIdx.x * (1.0 / 256.0));
    // lmode 1: the pass also lists the values it counts (those whose key
    // matches the prefix), up to LCAP of them; lmode 2: the level runs over
    // that list instead of the row. The list holds every element the next
    // level can count, with the same values, so the counts and exact sums
    // are those a pass over the row would give.
    auto level = [&](int shift, uint32_t prefix, uint32_t floor_key, bool cnt_on, int lmode) {
      if (threadIdx.x < 256) {
        sh.rcnt[threadIdx.x] = 0u;
        sh.rmh[threadIdx.x] = 0ull;
        sh.rml[threadIdx.x] = 0ull;
      }
      if (spread)
        for (int k = threadIdx.x; k < 256 * MC; k += RS_THREADS) {
          cmh[k] = 0ull;
          cml[k] = 0ull;
          ccnt[k] = 0u;
        }
      if (lmode == 1 && threadIdx.x == 0) *lcnt = 0u;
      __syncthreads();
      auto body = [&](float z, int id) {
        // with a penalty the set lookups come first (they change values);
        // without one every finite element counts here and the banned ones
        // are taken back out after the loop
        if (g.ptab) {
          if (!g.admissible(z, id)) return;
          z = g.value(z, id);
        } else if (!(z > -INFINITY && z < INFINITY)) {
          return;
        }
        const uint32_t key = gkey<Elem>(z);
        if (key < floor_key) return;
        if (shift + 8 < KB && (key >> (shift + 8)) != prefix) return;
        const uint32_t d = (key >> shift) & 255u;
        if (spread) {
          const uint32_t c = d * MC + (threadIdx.x & (MC - 1));
          if (cnt_on) atomicAdd(&ccnt[c], 1u);
          const Fix f = fix_of(exp2_tab((double)z * c2 - rmax, etab));
          atomicAdd(&cmh[c], f.h);
          atomicAdd(&cml[c], f.l);
          if (lmode == 1) {
            const uint32_t k = atomicAdd(lcnt, 1u);
            if (k < LCAP) lst[k] = z;
          }
        } else {
          if (cnt_on) atomicAdd(&sh.rcnt[d], 1u);
          const Fix f = fix_of(exp2_neg((double)z * c2 - rmax));
          atomicAdd(&sh.rmh[d], f.h);
          atomicAdd(&sh.rml[d], f.l);
        }
      };
      if (lmode == 2) {
        const uint32_t n = *lcnt;
        for (uint32_t k = threadIdx.x; k < n; k += RS_THREADS) body(lst[k], 0);
      } else {
        for_each_elem<Elem>(rowp, V, body);
      }
      if (sub_bans) {
        // the banned elements this level counted, taken back out (the bins
        // wrap through zero at worst, and end exact)
#pragma unroll
        for (int k = 0; k < GEN_BPT; ++k) {
          const float z = zb[k * RS_THREADS];
          if (!(z > -INFINITY && z < INFINITY)) continue;
          const uint32_t key = gkey<Elem>(z);
          if (key < floor_key) continue;
          if (shift + 8 < KB && (key >> (shift + 8)) != prefix) continue;
          const uint32_t d = (key >> shift) & 255u;
          if (cnt_on) atomicSub(&sh.rcnt[d], 1u);
          const Fix f = fix_of(exp2_tab((double)z * c2 - rmax, etab));
          atomicAdd(&sh.rmh[d], 0ull - f.h);
          atomicAdd(&sh.rml[d], 0ull - f.l);
        }
      }
      __syncthreads();
      if (spread) {
        if (threadIdx.x < 256) {
          unsigned long long h = sh.rmh[threadIdx.x], l = sh.rml[threadIdx.x];
          uint32_t n = sh.rcnt[threadIdx.x];
#pragma unroll
          for (int c = 0; c < MC; ++c) {
            h += cmh[threadIdx.x * MC + c];
            l += cml[threadIdx.x * MC + c];
            n += ccnt[threadIdx.x * MC + c];
          }
          sh.rmh[threadIdx.x] = h;
          sh.rml[threadIdx.x] = l;
          sh.rcnt[threadIdx.x] = n;
        }
        __syncthreads();
      }
    };
    // Wave 0 scans the digits from the top (lane l takes 255 - 4l - j,
    // j = 0..3) for the first one where the running count reaches `need`
    // (count mode) or above + the running mass reaches `target` (mass mode;
    // a negative target, given at the first level only, means top_p times that
    // level's total mass, i.e. the whole set's); if rounding leaves every digit
    // short, the lowest digit with elements. It writes the digit, the count and
    // mass of the level's elements above it, and the target it used.
    auto pick = [&](bool mass_mode, uint32_t need, Fix above, double target, float top_p) {
      if (threadIdx.x < WAVE) {
        const int l = threadIdx.x;
        uint32_t c[4];
        Fix m[4];
        uint32_t lc = 0u;
        Fix lm = {0ull, 0ull};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 255 - 4 * l - j;
          c[j] = sh.rcnt[d];
          m[j].h = sh.rmh[d];
          m[j].l = sh.rml[d];
          lc += c[j];
          lm = fix_add(lm, m[j]);
        }
        const uint32_t ic = wave_incl_scan(lc);
        const unsigned long long ih = wave_incl_scan(lm.h), il = wave_incl_scan(lm.l);
        if (target < 0.0) {
          Fix tot;
          tot.h = (unsigned long long)__shfl(ih, WAVE - 1, WAVE);
          tot.l = (unsigned long long)__shfl(il, WAVE - 1, WAVE);
          target = (double)top_p * fix_val(fix_add(above, tot));
        }
        uint32_t rc = ic - lc;
        Fix rm;
        rm.h = ih - lm.h;
        rm.l = il - lm.l;
        int sel = -1, last = -1;
        uint32_t selc = 0u, lastc = 0u;
        Fix selm = {0ull, 0ull}, lastm = {0ull, 0ull};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool nz = c[j] != 0u || (m[j].h | m[j].l) != 0ull;
          if (nz) {
            const bool reached = mass_mode ? fix_val(fix_add(fix_add(above, rm), m[j])) >= target
                                           : rc + c[j] >= need;
            if (reached && sel < 0) {
              sel = 255 - 4 * l - j;
              selc = rc;
              selm = rm;
            }
            last = 255 - 4 * l - j;
            lastc = rc;
            lastm = rm;
          }
          rc += c[j];
          rm = fix_add(rm, m[j]);
        }
        const uint64_t bs = __ballot(sel >= 0), bl = __ballot(last >= 0);
        const int who = bs ? __ffsll((unsigned long long)bs) - 1 : (bl ? 63 - __clzll((long long)bl) : 0);
        if (l == 0) sh.rsel_target = target;
        if (l == who) {
          const bool found = sel >= 0;
          sh.rsel_d = (uint32_t)(found ? sel : (last >= 0 ? last : 0));
          sh.rsel_c = found ? selc : lastc;
          sh.rsel_h = found ? selm.h : lastm.h;
          sh.rsel_l = found ? selm.l : lastm.l;
        }
      }
      __syncthreads();
    };
    // fp32 keys without a penalty set: the third pass lists the values that
    // share its 16-bit prefix (at a cut among normal logits, about a hundred
    // of c5's 151,936), and the last level reads that list instead of the row
    // when it held them all. The list is read after the barriers that end the
    // third level and its pick, so every thread sees the same count.
    auto lmode_of = [&](int shift) -> int {
      if (KB != 32 || !spread) return 0;
      if (shift == 8) return 1;
      return (shift == 0 && *lcnt <= LCAP) ? 2 : 0;
    };
    uint32_t floor_key = 0u;
    if (s.top_k > 0 && (uint32_t)s.top_k < cnt) {
      uint32_t need = (uint32_t)s.top_k, prefix = 0u;
      Fix above = {0ull, 0ull}, zk = {0ull, 0ull};
      for (int shift = KB - 8; shift >= 0; shift -= 8) {
        level(shift, prefix, 0u, true, lmode_of(shift));
        pick(false, need, above, 0.0, 1.0f);
        const uint32_t d = sh.rsel_d;
        need -= sh.rsel_c;
        above = fix_add(above, Fix{sh.rsel_h, sh.rsel_l});
        if (shift == 0) zk = fix_add(above, Fix{sh.rmh[d], sh.rml[d]});
        prefix = (prefix << 8) | d;
        __syncthreads();   // the digit's bins are read before the next level clears them
      }
      floor_key = prefix;
      tau = gval<Elem>(prefix);
      trunc = true;
      Z = fix_val(zk);
    }
    if (s.top_p < 1.0f) {
      uint32_t prefix = 0u;
      Fix above = {0ull, 0ull}, zp = {0ull, 0ull};
      // top_p times the kept set's mass after top-k; otherwise times the
      // first level's total, which the first pick computes
      double target = trunc ? (double)s.top_p * Z : -1.0;
      for (int shift = KB - 8; shift >= 0; shift -= 8) {
        level(shift, prefix, floor_key, false, lmode_of(shift));
        pick(true, 0u, above, target, s.top_p);
        target = sh.rsel_target;
        const uint32_t d = sh.rsel_d;
        above = fix_add(above, Fix{sh.rsel_h, sh.rsel_l});
        if (shift == 0) zp = fix_add(above, Fix{sh.rmh[d], sh.rml[d]});
        prefix = (prefix << 8) | d;
        __syncthreads();
      }
      tau = gval<Elem>(prefix);
      trunc = true;
      Z = fix_val(zp);
    }
  } else if (s.top_k > 0 && (uint32_t)s.top_k < cnt) {
    // largest key t with count(z >= value(t)) >= k
    uint32_t lo = gkey<Elem>(mn), hi = gkey<Elem>(mx) + 1u;
    while (hi - lo > 1u) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      if (count_ge(gval<Elem>(mid)) >= (uint32_t)s.top_k)
        lo = mid;
      else
        hi = mid;
    }
    tau = gval<Elem>(lo);
    trunc = true;
    Z = mass_ge(tau);
  }
  if (V >= RADIX_MAX_V && s.top_p < 1.0f) {
    // largest key t with mass(z >= value(t)) >= top_p * Z (within the top-k set)
    const double target = (double)s.top_p * Z;
    uint32_t lo = gkey<Elem>(trunc ? fmaxf(tau, mn) : mn), hi = gkey<Elem>(mx) + 1u;
    double zlo = Z;
    while (hi - lo > 1u) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      const double mm = mass_ge(gval<Elem>(mid));
      if (mm >= target) {
        lo = mid;
        zlo = mm;
      } else {
        hi = mid;
      }
    }
    tau = gval<Elem>(lo);
    trunc = true;
    Z = zlo;
  }
  // a radix-cut sampler that keeps everything (top-k at least the count,
  // top-p 1): the first pass skipped the exp-sum
  if (radix_cut && !trunc) Z = mass_ge(-INFINITY);
  out.m = mx;
  out.tau = trunc ? tau : -INFINITY;
  out.lse = rmax * 0.6931471805599453 + log(Z);
  out.path = 1u;
  return out;
}

// ------------------------------------------------------------------ histogram epilogue
//
// While one workgroup derives its statistics, the other workgroups of the CU
// keep the LDS saturated with histogram atomics, so every LDS round trip of the
// epilogue waits in that queue. The epilogue is therefore built around few
// dependent LDS round trips: each thread loads its HB_TPR counts in one batch
// and keeps them in registers, wave-level scans use DPP lane moves, and the
// waves meet in one exchange (two to four with truncation).
//
// Thread t < NT/2 owns ranks HB_TPR*t .. (positive values, descending), thread
// NT/2 + t owns ranks 4097 + HB_TPR*t .. (negative values), and thread NT/2
// also owns the zero rank, which precedes its ranks. Ranks are thus contiguous
// in thread order. A thread's ranks lie in one binade, where bf16 values are
// equally spaced by delta = 2^(e - 134): the mass per unit count
// exp((v - ref) / T) of consecutive ranks differs by the factor exp(-delta / T),
// so each thread needs two exps. Masses are taken relative to the largest value
// of the thread's wave and rescaled exactly once the row maximum is known.

constexpr int HB_TPR = 2 * (int)HB_WIN / RS_THREADS;   // ranks per thread
static_assert(HB_TPR % 4 == 0 && 128 % HB_TPR == 0, "epilogue rank tiling");

// A slot read from LDS is the same for every lane: keep it in scalar registers.
__device__ __forceinline__ WaveSlot slot_uniform(const WaveSlot& src) {
  const u32x4 v = *(const u32x4*)&src;
  WaveSlot r;
  r.n = (uint32_t)__builtin_amdgcn_readfirstlane((int)v[0]);
  r.top = __builtin_amdgcn_readfirstlane((int)v[1]);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)v[2]);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)v[3]);
  r.z = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  return r;
}

// The counts of ranks r0 .. r0 + HB_TPR - 1 in rank order.
__device__ __forceinline__ void hb_load_counts(const uint32_t* hist, int r0, bool pos,
                                               uint32_t (&c)[HB_TPR]) {
#pragma unroll
  for (int i = 0; i < HB_TPR / 4; ++i) {
    if (pos) {
      const u32x4 v = *(const u32x4*)(hist + (HB_WIN - 4) - r0 - 4 * i);
      c[4 * i] = v[3];
      c[4 * i + 1] = v[2];
      c[4 * i + 2] = v[1];
      c[4 * i + 3] = v[0];
    } else {
      const u32x4 v = *(const u32x4*)(hist + HB_NEG + (r0 - (int)HB_WIN - 1) + 4 * i);
      c[4 * i] = v[0];
      c[4 * i + 1] = v[1];
      c[4 * i + 2] = v[2];
      c[4 * i + 3] = v[3];
    }
  }
}

__device__ __forceinline__ int hb_thread_rank0(int t) {
  return t < RS_THREADS / 2 ? HB_TPR * t : (int)HB_WIN + 1 + HB_TPR * (t - RS_THREADS / 2);
}

// Exact statistics from the counts, computed by the whole block; false when the
// row must go to the generic path (a truncation cut among the tiny values).
__device__ __forceinline__ bool hb_epilogue(const SamplerDev s, RowShared& sh, RowStat& out) {
  constexpr int NW = RS_THREADS / WAVE;
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int r0 = hb_thread_rank0(tid);
  const bool pos = tid < RS_THREADS / 2;
  const bool zown = tid == RS_THREADS / 2;

  // counts of the thread's ranks, in rank order, in one batch of LDS loads
  uint32_t c[HB_TPR];
  hb_load_counts(sh.hist, r0, pos, c);
  const uint32_t zc = zown ? sh.zero_cnt : 0u;
  const uint32_t tn = min(sh.tiny_n, TINY_MAX);
  uint32_t cl = zc, nz = 0u;
#pragma unroll
  for (int j = 0; j < HB_TPR; ++j) {
    cl += c[j];
    nz |= (c[j] != 0u ? 1u : 0u) << j;
  }
  const int top = zc ? (int)HB_ZERO : (nz ? r0 + __ffs(nz) - 1 : HB_RANKS);
  const uint32_t cnt_incl = wave_scan_dpp(cl, 0u, [](uint32_t x, uint32_t y) { return x + y; });
  const int top_w = lane63(wave_scan_dpp(top, (int32_t)HB_RANKS,
                                         [](int32_t x, int32_t y) { return x < y ? x : y; }));
  const double invT = 1.0 / (double)s.temperature;
  const double mw = top_w < HB_RANKS ? (double)hb_value_of_rank(top_w) : 0.0;
  // masses relative to the wave's top value, anchored at the thread's first
  // nonzero rank (its value is <= the wave's top, so no exp overflows)
  const uint32_t bits0 = pos ? (HB_WIN - 1u - (uint32_t)r0 + HB_BASE)
                             : ((uint32_t)r0 - (HB_WIN + 1u) + HB_BASE);
  const double ratio = exp_neg(-ldexp(1.0, (int)(bits0 >> 7) - 134) * invT);
  const int jtop = nz ? __ffs(nz) - 1 : HB_TPR;
  const double e0 = nz ? exp_neg(((double)hb_value_of_rank(r0 + jtop) - mw) * invT) : 0.0;
  double zmass = 0.0;                 // zero rank and the tiny values listed with it
  if (zc) {
    zmass = (double)(zc - tn) * exp_neg(-mw * invT);
    for (uint32_t k = 0; k < tn; ++k)   // sorted beforehand: a fixed order
      zmass += exp_neg(((double)bf16_to_f32(sh.tiny[k]) - mw) * invT);
  }
  // the thread's mass: sum over j >= jtop of c[j] * e0 * ratio^(j - jtop), in
  // Horner form from the smallest value up (one fp64 accumulator)
  double hm = 0.0;
#pragma unroll
  for (int j = HB_TPR - 1; j >= 0; --j)
    if (j >= jtop) hm = hm * ratio + (double)c[j];
  const double ml = zmass + e0 * hm;
  const double mass_incl = wave_scan_dpp(ml, 0.0, [](double x, double y) { return x + y; });

  // exchange 1: per-wave count, top rank and mass
  if (lane == WAVE - 1) {
    WaveSlot ws;
    ws.n = cnt_incl;
    ws.top = top_w;
    ws.z = mass_incl;
    sh.x1[w] = ws;
  }
  __syncthreads();
  WaveSlot x[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) x[k] = slot_uniform(sh.x1[k]);
  uint32_t N = 0u;
  int rtop = HB_RANKS;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    N += x[k].n;
    rtop = min(rtop, x[k].top);
  }
  if (N == 0u) {
    out.flags |= FLAG_EMPTY;
    return true;
  }
  const float m = hb_value_of_rank(rtop);
  const double md = (double)m;
  // rescale every wave to the row maximum; prefixes before this thread. Lane
  // k evaluates wave k's factor once; the wave reads it back from that lane.
  static_assert(NW <= WAVE, "one lane per wave's factor");
  int tk = x[0].top;
#pragma unroll
  for (int k = 1; k < NW; ++k)
    if (lane == k) tk = x[k].top;
  const double sc_lane =
      tk < HB_RANKS ? exp_neg(((double)hb_value_of_rank(tk) - md) * invT) : 0.0;
  double Z0 = 0.0, mass_before = 0.0, scale_w = 0.0;
  uint32_t cnt_before = cnt_incl - cl;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const double sc = readlane_f64(sc_lane, k);
    const double zk = x[k].z * sc;
    Z0 += zk;
    if (k < w) {
      mass_before += zk;
      cnt_before += x[k].n;
    }
    if (k == w) scale_w = sc;
  }
  mass_before += (mass_incl - ml) * scale_w;

  // visit the thread's nonzero ranks <= rlim in order: fn(rank, count, mass rel.
  // to md). Only threads at a truncation cut walk; they reload their counts.
  auto walk = [&](int rlim, auto&& fn) {
    if (zc && rlim >= (int)HB_ZERO) fn((int)HB_ZERO, zc, zmass * scale_w);
    uint32_t cc[HB_TPR];
    hb_load_counts(sh.hist, r0, pos, cc);
    const int jlim = rlim - r0;
    double e = e0;
#pragma unroll
    for (int j = 0; j < HB_TPR; ++j) {
      if (j > jtop) e *= ratio;
      if (j <= jlim && cc[j]) fn(r0 + j, cc[j], (double)cc[j] * e * scale_w);
    }
  };

  int rk = HB_RANKS - 1;
  double Z = Z0;
  bool trunc = false;
  if (s.top_k > 0 && (uint32_t)s.top_k < N) {
    // exchange 2: the thread holding the k-th largest count reports its rank
    // and the mass up to it (integer prefixes: exactly one such thread)
    const uint32_t kk = (uint32_t)s.top_k;
    const bool mine = cnt_before < kk && cnt_before + cl >= kk;
    int rsel = -1;
    double zsel = 0.0;
    if (mine) {
      uint32_t cum = cnt_before;
      double zz = mass_before;
      walk(HB_RANKS - 1, [&](int r, uint32_t cc, double mass) {
        if (cum < kk) {
          rsel = r;
          zz += mass;
        }
        cum += cc;
      });
      zsel = zz;
    }
    const uint64_t bal = __ballot(mine);
    if (lane == (bal ? __ffsll((unsigned long long)bal) - 1 : 0)) {
      WaveSlot ws;
      ws.n = (uint32_t)rsel;
      ws.top = 0;
      ws.z = zsel;
      sh.x2[w] = ws;
    }
    __syncthreads();
#pragma unroll
    for (int k = NW - 1; k >= 0; --k) {
      const WaveSlot ws = slot_uniform(sh.x2[k]);
      if ((int32_t)ws.n >= 0) {
        rk = (int)ws.n;
        Z = ws.z;
      }
    }
    trunc = true;
    if (rk == (int)HB_ZERO && tn > 0u) return false;
  }
  int rp_last = rk;
  if (s.top_p < 1.0f) {
    // exchange 3: keep rank r while the mass strictly above it is < top_p * Z;
    // the first thread whose ranks reach the target reports the last kept rank
    // and the kept mass
    const double target = (double)s.top_p * Z;
    int last = -1;
    double above = mass_before;
    const bool cand = mass_before < target && r0 <= rk + (zown ? 1 : 0) &&
                      (mass_before + ml * scale_w >= target || r0 + HB_TPR - 1 > rk);
    if (cand) {
      walk(rk, [&](int r, uint32_t, double mass) {
        if (above < target) {
          last = r;
          above += mass;
        }
      });
    }
    const bool crosses = cand && last >= 0 && above >= target;
    const uint64_t bal = __ballot(crosses);
    if (lane == (bal ? __ffsll((unsigned long long)bal) - 1 : 0)) {
      WaveSlot ws;
      ws.n = crosses ? (uint32_t)last : 0xFFFFFFFFu;
      ws.top = 0;
      ws.z = above;
      sh.x3[w] = ws;
    }
    __syncthreads();
    // the first wave with a crossing; none (rounding at the very end): keep rk
#pragma unroll
    for (int k = NW - 1; k >= 0; --k) {
      const WaveSlot ws = slot_uniform(sh.x3[k]);
      if ((int32_t)ws.n >= 0) {
        rp_last = (int)ws.n;
        Z = ws.z;
      }
    }
    trunc = true;
    if (rp_last == (int)HB_ZERO && tn > 0u) return false;
  }
  // the largest kept logit (a tiny positive can top the zero bin)
  if (rtop == (int)HB_ZERO && tn > 0u) {
    float tt = -INFINITY;
    for (uint32_t k = 0; k < tn; ++k) tt = fmaxf(tt, bf16_to_f32(sh.tiny[k]));
    out.m = sh.zero_cnt > tn ? fmaxf(0.0f, tt) : tt;
  } else {
    out.m = m;
  }
  out.tau = trunc ? hb_value_of_rank(rp_last) : -INFINITY;
  // only thread 0 reports the row: the other waves skip the fp64 log
  out.lse = threadIdx.x < WAVE ? md * invT + log(Z) : -INFINITY;
  return true;
}

// ------------------------------------------------------------------ the kernel

// Three 512-thread workgroups per CU (6 waves per SIMD, up to 80 VGPRs). The
// streaming loop is bound by the CU's LDS atomic rate, which the resident
// workgroups share, so a fourth one would not stream faster; it would only
// force register spills in the epilogue and make the last round of rows
// coarser (rows / (3 * CUs) is closer to a whole number for large batches).
// The ids a row penalizes: entry j < H of the request's history `hist`, then
// the proposals props[0 .. npen-H-1] that precede the row's position.
__device__ __forceinline__ int32_t pen_id(const int32_t* hist, int H, const int32_t* props, int j) {
  return j < H ? hist[j] : props[j - H];
}

// Inserts the row's penalized ids (valid, not banned) into the LDS hash set
// `ptab` (all slots HT_EMPTY beforehand). Bit k of the result is set when this
// thread's k-th entry (j = threadIdx.x + k * RS_THREADS) entered the set, so
// every distinct id has one owner. Sets *xpen when the row's proposal x is one.
// `first` is entry threadIdx.x, loaded by the caller.
__device__ __forceinline__ uint32_t pen_build(uint32_t* ptab, const uint32_t* bantab,
                                              const int32_t* hist, int H, const int32_t* props,
                                              int npen, int V, int32_t first, int32_t x,
                                              uint32_t* xpen) {
  uint32_t own = 0u;
  int k = 0;
  for (int j = threadIdx.x; j < npen; j += RS_THREADS, ++k) {
    const int32_t id = j == (int)threadIdx.x ? first : pen_id(hist, H, props, j);
    if (id < 0 || id >= V) continue;
    if (bantab && ht_has(bantab, id)) continue;   // banned wins
    if (id == x) *xpen = 1u;
    if (ht_insert(ptab, id)) own |= 1u << k;
  }
  return own;
}

// The target row of a greedy request in a mixed batch: its argmax (the
// request's target bans and NaN excluded) as the row's RowStat: path = the
// argmax, px = 1 iff the row's proposal is the argmax (the sampling walk's
// test u * q <= p with q = 1 then accepts exactly on a match). Not inlined:
// its registers stay out of the statistics path's allocation. Returns
// (path, flags) by value, so that the caller's RowStat stays in registers.
template <typename Elem>
__device__ __attribute__((noinline)) uint2 greedy_row_stat(const Elem* rowp, int V,
                                                           const int32_t* bl, int nb, int32_t first,
                                                           const int32_t* hist, int H,
                                                           const int32_t* props, int npen,
                                                           float theta, RowShared& sh) {
  const uint32_t* tab = nullptr;
  const uint32_t* ptab = nullptr;
  if (nb > 0 || npen > 0) {
    for (uint32_t k = threadIdx.x; k < 2 * HT_SLOTS; k += RS_THREADS) sh.hist[k] = HT_EMPTY;
    __syncthreads();
  }
  if (nb > 0) {
    (void)ht_build(sh.hist, bl, nb, V, first, -1, &sh.xban);
    __syncthreads();
    tab = sh.hist;
  }
  if (npen > 0) {
    const int32_t p0 = threadIdx.x < (unsigned)npen ? pen_id(hist, H, props, threadIdx.x) : -1;
    (void)pen_build(sh.hist + HT_SLOTS, tab, hist, H, props, npen, V, p0, -1, &sh.xpen);
    __syncthreads();
    ptab = sh.hist + HT_SLOTS;
  }
  // one instantiation with run-time tests of both sets keeps this call small
  const ArgResult r = row_argmax<Elem, RS_THREADS, 2, true, true>(rowp, V, tab, sh.fscr, sh.iscr,
                                                                  sh.uscr, ptab, theta);
  return make_uint2((uint32_t)r.arg,
                    (r.nonfinite ? FLAG_NONFINITE : 0u) | (r.arg < 0 ? FLAG_EMPTY : 0u));
}

// Thread 0 of a row: its RowStat, the optional lse outputs, and the counters
// the later kernels expect at zero.
__device__ __forceinline__ void row_finish(const RowStatsArgs& a, int row, const RowStat& out) {
  const int G1 = a.gamma + 1, RPR = 2 * a.gamma + 1;
  const int b = row / RPR, i = row % RPR;
  a.stats[row] = out;
  if (i == 0 && a.tickets) a.tickets[b] = 0;
  if (i < a.gamma && a.ov_tickets) a.ov_tickets[(int64_t)b * a.gamma + i] = 0;
  if (row == 0 && a.accept_hist)
    for (int k = 0; k <= a.gamma; ++k) a.accept_hist[k] = 0u;
  if (i < G1) {
    if (a.out_tlse) a.out_tlse[(int64_t)b * G1 + i] = (float)out.lse;
  } else {
    if (a.out_dlse) a.out_dlse[(int64_t)b * a.gamma + (i - G1)] = (float)out.lse;
  }
}

// MIXED: per-request draft lengths, samplers (greedy requests included) and
// draft ban lists; the plain variant carries none of that logic.
template <typename Elem, bool MIXED>
__global__ __launch_bounds__(RS_THREADS) __attribute__((amdgpu_waves_per_eu(sizeof(Elem) == 2 ? 6 : 4)))
void row_stats_kernel(RowStatsArgs a) {
  __shared__ RowShared sh;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int G1 = a.gamma + 1, RPR = 2 * a.gamma + 1;
  const int b = row / RPR, i = row % RPR;
  const bool is_target = i < G1;
  const Elem* rowp = is_target
                         ? (const Elem*)a.target + ((int64_t)b * G1 + i) * (int64_t)a.V
                         : (const Elem*)a.draft + ((int64_t)b * a.gamma + (i - G1)) * (int64_t)a.V;
  const int V = a.V;
  const int pi = is_target ? i : i - G1;
  // draft rows take the draft ban list when there is one
  const bool dbans = MIXED && !is_target && a.req.banned_d;
  const int nb_all = dbans ? a.req.n_banned_d : (a.banned ? a.n_banned : 0);
  const int32_t* bl_all = nb_all == 0 ? nullptr
                          : dbans ? a.req.banned_d + (int64_t)b * a.req.n_banned_d
                                  : a.banned + (int64_t)b * a.n_banned;
  // repetition penalty of the row: its history and the proposals before it
  const int H = (MIXED && a.req.history) ? a.req.n_history : 0;
  const int32_t* hist = H ? a.req.history + (int64_t)b * a.req.n_history : nullptr;
  const int32_t* props = a.draft_tokens + (int64_t)b * a.gamma;
  // The row's first ban and penalty entries and its proposal token are loaded
  // before the request's settings are known (every index here is in range),
  // so that in a mixed batch these loads do not wait for the settings.
  const int32_t ban0_all = tid < nb_all ? bl_all[tid] : -1;
  const int32_t pen0_all = (MIXED && tid < H + pi) ? pen_id(hist, H, props, tid) : -1;
  const int32_t xprop_all = pi < a.gamma ? props[pi] : -1;
  ReqInfo rq;
  if constexpr (MIXED) {
    rq = request_info(a.req, b, a.gamma, a.st, a.sd);
  } else {
    rq.g = a.gamma;
    rq.st = a.st;
    rq.sd = a.sd;
    rq.greedy = false;
    rq.bad = false;
  }
  const SamplerDev s = is_target ? rq.st : rq.sd;
  // rows the request does not use: beyond its draft length, the draft rows of
  // a greedy request, every row of a request with settings out of range
  const bool used = !MIXED || (!rq.bad && pi <= rq.g && (is_target ? true : !rq.greedy && pi < rq.g));
  const bool greedy_row = MIXED && used && rq.greedy;   // a target row: its argmax
  const int nb = used ? nb_all : 0;
  const int32_t* bl = nb == 0 ? nullptr : bl_all;
  const int32_t ban0 = used ? ban0_all : -1;
  // the proposal this row scores (none for the bonus row) and its logit
  const int32_t xprop = (used && pi < (MIXED ? rq.g : a.gamma)) ? xprop_all : -1;
  const bool xvalid = xprop >= 0 && xprop < V;
  const float zx = (tid == 0 && xvalid) ? elem_value<Elem>(rowp[xprop]) : 0.0f;
  if (tid == 0) {
    sh.xban = 0u;
    sh.xpen = 0u;
  }
  const float theta = is_target ? rq.pt : rq.pd;
  const int npen = (MIXED && used && theta != 1.0f) ? H + pi : 0;
  const int32_t pen0 = tid < npen ? pen0_all : -1;
  // Target row i also draws uniform slot i of its request for the acceptance
  // walk (slot gamma: the final draw). Lane 0 of the last wave computes it,
  // in the bf16 stream while its first loads are in flight.
  bool u_pending = a.ustore && is_target && tid == RS_THREADS - WAVE;
  auto emit_u = [&]() {
    a.ustore[(int64_t)b * G1 + i] = philox_uniform(a.seed, a.offset, (uint32_t)b, (uint32_t)i);
    u_pending = false;
  };

  RowStat out;
  out.m = -INFINITY;
  out.tau = -INFINITY;
  out.lse = -INFINITY;
  out.flags = 0u;
  out.path = 0u;
  out.px = 0.0;

  if constexpr (MIXED) {
    if (!used || greedy_row) {
      // no statistics: an unused row, or the argmax of a greedy request's
      // target row (its proposal survives, p = 1, iff it is the argmax)
      out.lse = __builtin_nan("");
      if (!used) out.flags = rq.bad ? FLAG_BAD_PARAM : 0u;
      if (greedy_row) {
        const uint2 gr = greedy_row_stat<Elem>(rowp, V, bl, nb, ban0, hist, H, props, npen, theta, sh);
        out.path = gr.x;
        out.flags = gr.y;
        out.px = (xvalid && (int32_t)gr.x == xprop) ? 1.0 : 0.0;
      }
      if (u_pending) emit_u();
      if (tid == 0) row_finish(a, row, out);
      return;
    }
  }

  bool generic = (sizeof(Elem) == 4) || a.force_generic;
  if (!generic) {
    // The logits of the thread's first ban and penalty entries are gathered
    // first, so that their latency hides behind the fill and the set builds.
    const uint16_t* rp = (const uint16_t*)rowp;
    const uint32_t ban_bits = (ban0 >= 0 && ban0 < V) ? (uint32_t)rp[ban0] : 0u;
    const uint32_t pen_bits = (MIXED && pen0 >= 0 && pen0 < V) ? (uint32_t)rp[pen0] : 0u;
    const uintptr_t addr = (uintptr_t)rp;
    int head = (int)(((16u - (addr & 15u)) & 15u) >> 1);
    if (head > V) head = V;
    const int nchunk = (V - head) >> 3;
    const int tail0 = head + nchunk * 8;
    const u32x4* body = (const u32x4*)(rp + head);
    constexpr int STEP = RS_THREADS * RS_UNROLL;
    u32x4 va[RS_UNROLL], vb[RS_UNROLL];
    auto ld = [&](u32x4 (&v)[RS_UNROLL], int k0) {
#pragma unroll
      for (int u = 0; u < RS_UNROLL; ++u) {
        const int k = k0 + u * RS_THREADS;
        if (k < nchunk) v[u] = __builtin_nontemporal_load(body + k);
      }
    };
    // A ban list of at most one wave's length, in a row without a penalty
    // set, needs no hash set: during the stream, the first wave finds each
    // distinct id's first copy with lane shuffles and takes its logit
    // (gathered above) out of the counts.
    const bool wave_bans = nb > 0 && nb <= WAVE && npen == 0;
    // A row with no set to build issues its first buffer of stream loads now,
    // so that it arrives during the histogram fill. (With sets to build,
    // measured slower: their gathers would queue behind it.)
    const bool early = (nb == 0 || wave_bans) && npen == 0;
    if (early && tid < nchunk) ld(va, tid);
    // the first HT_SLOTS bins hold the ban hash set until the stream starts
    const uint32_t fill = (nb > 0 && !wave_bans) ? HT_EMPTY : 0u;
    const uint32_t pfill = npen > 0 ? HT_EMPTY : 0u;
    // 16-byte stores: the two set regions end on 16-byte boundaries
    static_assert(HT_SLOTS % 4 == 0 && 2 * HT_SLOTS <= HB_BINS &&
                  HB_BINS - 2 * HT_SLOTS <= RS_THREADS, "fill tiling");
    for (uint32_t k = tid; k < HB_BINS; k += RS_THREADS)
      sh.hist[k] = k < HT_SLOTS ? fill : (k < 2 * HT_SLOTS ? pfill : 0u);
    if (tid == 0) {
      sh.zero_cnt = 0u;
      sh.nonfinite = 0u;
      sh.special = 0u;
      sh.tiny_n = 0u;
    }
    __syncthreads();

    uint32_t own = 0u, own_p = 0u;
    if (nb > 0 && !wave_bans) {
      own = ht_build(sh.hist, bl, nb, V, ban0, xprop, &sh.xban);
      __syncthreads();
    }
    if (MIXED && npen > 0) {
      // penalized ids (the set sits behind the ban set, in the same storage)
      own_p = pen_build(sh.hist + HT_SLOTS, nb > 0 ? sh.hist : nullptr, hist, H, props, npen, V,
                        pen0, xprop, &sh.xpen);
      __syncthreads();
    }
    // subtracts the counts of a banned bf16 logit (each distinct id once)
    auto unban = [&](uint32_t bits) {
      const uint32_t ae = bits & 0x7FFFu;
      const uint32_t t = ae - HB_BASE;
      if (t < HB_WIN)
        atomicSub(&sh.hist[t + ((bits >> 15) ? HB_NEG : 0u)], 1u);
      else if (ae == 0u)
        atomicSub(&sh.zero_cnt, 1u);
      else if (ae < HB_BASE)
        sh.special = 1u;   // a banned tiny value: the generic path sorts it out
    };
    if ((nb > 0 && !wave_bans) || (MIXED && npen > 0)) {
      for (uint32_t k = tid; k < 2 * HT_SLOTS; k += RS_THREADS) sh.hist[k] = 0u;
      __syncthreads();
      // Each distinct banned id leaves the counts once (its owner subtracts
      // it), and each distinct penalized id moves one count from its logit to
      // the penalized logit (a bf16 value). This happens before the stream
      // adds the row's counts: the counts are unsigned and wrap, so a bin
      // that dips below zero here is exact again once the stream has added
      // the logit it removed.
      int kb = 0;
      for (int j = tid; j < nb; j += RS_THREADS, ++kb) {
        if (!((own >> kb) & 1u)) continue;
        unban(kb == 0 ? ban_bits : (uint32_t)rp[bl[j]]);
      }
      if constexpr (MIXED) {
        // values outside the counted window on either side of a move send
        // the row to the generic path
        int kp = 0;
        for (int j = tid; j < npen; j += RS_THREADS, ++kp) {
          if (!((own_p >> kp) & 1u)) continue;
          const uint32_t bits = kp == 0 ? pen_bits : (uint32_t)rp[pen_id(hist, H, props, j)];
          const float z = bf16_to_f32(bits);
          if (!(z > -INFINITY && z < INFINITY)) continue;   // not admissible: nothing to move
          const uint32_t nbits = __float_as_uint(pen_apply(z, theta, true)) >> 16;
          const uint32_t t0 = (bits & 0x7FFFu) - HB_BASE, t1 = (nbits & 0x7FFFu) - HB_BASE;
          if (t0 < HB_WIN && t1 < HB_WIN) {
            atomicSub(&sh.hist[t0 + ((bits >> 15) ? HB_NEG : 0u)], 1u);
            atomicAdd(&sh.hist[t1 + ((nbits >> 15) ? HB_NEG : 0u)], 1u);
          } else {
            sh.special = 1u;
          }
        }
      }
    }
    if (tid < head) hb_count_one(rp[tid], sh);
    if (tid < V - tail0) hb_count_one(rp[tail0 + tid], sh);

    // Software-pipelined stream: the loads of the next RS_UNROLL chunks are in
    // flight while the current ones are counted.
    auto proc = [&](const u32x4 (&v)[RS_UNROLL], int k0) {
#pragma unroll
      for (int u = 0; u < RS_UNROLL; ++u) {
        const int k = k0 + u * RS_THREADS;
        if (k < nchunk) {
          uint32_t oow = hb_count_pair(v[u][0], sh.hist);
          oow |= hb_count_pair(v[u][1], sh.hist);
          oow |= hb_count_pair(v[u][2], sh.hist);
          oow |= hb_count_pair(v[u][3], sh.hist);
          if (oow) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              hb_classify_slow(v[u][j] & 0xFFFFu, sh);
              hb_classify_slow(v[u][j] >> 16, sh);
            }
          }
        }
      }
    };
    // The first wave's short ban list, taken out once its first stream
    // buffer is counted: the gathered logits have long arrived by then, and
    // the wave waits for them while its next buffer is in flight (used only
    // after the stream, the gather would be issued there, a round trip at the
    // end of the row).
    bool bans_due = wave_bans && tid < WAVE;
    auto take_bans = [&]() {
      // lane l holds list entry l (-1 past the list); it owns its id when no
      // lower lane holds the same valid id
      const bool valid = ban0 >= 0 && ban0 < V;
      bool dup = false;
      for (int i = 0; i < WAVE; ++i) {
        const int32_t o = __shfl(ban0, i, WAVE);
        dup |= i < tid && o == ban0;
      }
      if (__ballot(valid && ban0 == xprop) && tid == 0) sh.xban = 1u;
      if (valid && !dup) unban(ban_bits);
      bans_due = false;
    };
    int k0 = tid;
    if (!early && k0 < nchunk) ld(va, k0);
    if (u_pending) emit_u();
    while (k0 < nchunk) {
      if (k0 + STEP < nchunk) ld(vb, k0 + STEP);
      proc(va, k0);
      if (bans_due) take_bans();
      k0 += STEP;
      if (k0 >= nchunk) break;
      if (k0 + STEP < nchunk) ld(va, k0 + STEP);
      proc(vb, k0);
      k0 += STEP;
    }
    if (bans_due) take_bans();
    __syncthreads();

    if (tid == 0) {
      // tiny values in ascending order: the epilogue sums them in this order
      const int n = (int)min(sh.tiny_n, TINY_MAX);
      for (int k = 1; k < n; ++k) {
        const uint16_t v = sh.tiny[k];
        const float fv = bf16_to_f32(v);
        int j = k - 1;
        while (j >= 0 && bf16_to_f32(sh.tiny[j]) > fv) {
          sh.tiny[j + 1] = sh.tiny[j];
          --j;
        }
        sh.tiny[j + 1] = v;
      }
    }
    __syncthreads();
    if (sh.nonfinite) out.flags |= FLAG_NONFINITE;
    if (sh.special || !hb_epilogue(s, sh, out)) generic = true;
  }

  if (generic) {
    __syncthreads();
    // the ban set moves into the (now free) histogram storage
    GenericCtx g{nullptr, nullptr, theta, sizeof(Elem) == 2, false};
    if (nb > 0 || (MIXED && npen > 0)) {
      for (uint32_t k = tid; k < 2 * HT_SLOTS; k += RS_THREADS) sh.hist[k] = HT_EMPTY;
      __syncthreads();
    }
    if (nb > 0) {
      const uint32_t own = ht_build(sh.hist, bl, nb, V, ban0, xprop, &sh.xban);
      __syncthreads();
      g.tab = sh.hist;
      // A radix cut without a repetition penalty takes the banned values out
      // of its exact sums: each owner lists its values (a thread reads only
      // its own entries later, so no barrier is needed).
      if (!(MIXED && npen > 0) && V < RADIX_MAX_V && (s.top_k > 0 || s.top_p < 1.0f)) {
        float* zl = gen_banned_values(sh.hist);
#pragma unroll
        for (int k = 0; k < GEN_BPT; ++k) {
          float z = __builtin_nanf("");
          if ((own >> k) & 1u) z = elem_value<Elem>(rowp[k == 0 ? ban0 : bl[tid + k * RS_THREADS]]);
          zl[k * RS_THREADS + tid] = z;
        }
        g.sub_bans = true;
      }
    }
    if (MIXED && npen > 0) {
      (void)pen_build(sh.hist + HT_SLOTS, g.tab, hist, H, props, npen, V, pen0, xprop, &sh.xpen);
      __syncthreads();
      g.ptab = sh.hist + HT_SLOTS;
    }
    out.flags &= ~FLAG_EMPTY;
    out = row_generic<Elem>(rowp, V, s, g, sh, out);
  }

  if (u_pending) emit_u();
  if (tid == 0) {
    // probability of the row's proposal under the row's distribution
    const float zp = (MIXED && sh.xpen && zx > -INFINITY && zx < INFINITY)
                         ? pen_apply(zx, theta, sizeof(Elem) == 2) : zx;
    const bool kept = xvalid && !sh.xban && !(out.flags & FLAG_EMPTY) && zp > -INFINITY &&
                      zp < INFINITY && zp >= out.tau;
    out.px = kept ? exp((double)zp / (double)s.temperature - out.lse) : 0.0;
    row_finish(a, row, out);
  }
}

int launch_row_stats(const RowStatsArgs& a, int dtype_bf16, int rows, hipStream_t stream) {
  const bool mixed = a.req.gammas || a.req.ts || a.req.ds || a.req.banned_d || a.req.pen_t ||
                     a.req.pen_d || a.req.history;
  const dim3 grid(rows), block(RS_THREADS);
  if (dtype_bf16) {
    if (mixed)
      hipLaunchKernelGGL((row_stats_kernel<uint16_t, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((row_stats_kernel<uint16_t, false>), grid, block, 0, stream, a);
  } else {
    if (mixed)
      hipLaunchKernelGGL((row_stats_kernel<float, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((row_stats_kernel<float, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
