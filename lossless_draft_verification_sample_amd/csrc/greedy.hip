// Greedy verification ("Drafters and Speculative Decoding: Useful Tokens,
// Correct State", section "Greedy verification"; "Speculative Decoding - Turn
// guesses into parallel work", section "Greedy, sampling and the real sampler"):
// a proposal survives while it equals the argmax of its target row; the first
// mismatch emits that row's argmax; if all gamma match, the argmax of row gamma
// is appended. Ties go to the lowest token id (-0 and +0 tie); banned ids and
// NaN logits are not candidates.
//
// greedy_argmax: one workgroup per target row (row_argmax). The argmax is
// parked in out_tokens as (argmax + 1) in bits 0..30 (0: no admissible token)
// with bit 31 marking NaN or +inf in the row; greedy_scan then rewrites
// out_tokens into the emitted block.

#include "sv_argmax.hpp"
#include "sv_launch.hpp"

namespace sv {

constexpr int GA_THREADS = 512;
constexpr int GA_UNROLL = 4;

template <typename Elem>
__global__ __launch_bounds__(GA_THREADS) void greedy_argmax_kernel(GreedyArgs a) {
  __shared__ uint32_t tab[HT_SLOTS];
  __shared__ float sv_[GA_THREADS / WAVE];
  __shared__ int32_t si_[GA_THREADS / WAVE];
  __shared__ uint32_t su_[GA_THREADS / WAVE];
  __shared__ uint32_t xban;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int V = a.V;
  const Elem* rowp = (const Elem*)a.target + (int64_t)row * V;
  const int b = row / (a.gamma + 1);
  const int nb = a.banned ? a.n_banned : 0;
  const uint32_t* bans = nullptr;
  if (nb > 0) {
    const int32_t* bl = a.banned + (int64_t)b * a.n_banned;
    const int32_t first = tid < nb ? bl[tid] : -1;
    for (uint32_t k = tid; k < HT_SLOTS; k += GA_THREADS) tab[k] = HT_EMPTY;
    __syncthreads();
    (void)ht_build(tab, bl, nb, V, first, -1, &xban);
    __syncthreads();
    bans = tab;
  }
  const ArgResult r =
      bans ? row_argmax<Elem, GA_THREADS, GA_UNROLL, true>(rowp, V, bans, sv_, si_, su_)
           : row_argmax<Elem, GA_THREADS, GA_UNROLL, false>(rowp, V, nullptr, sv_, si_, su_);
  if (tid == 0) a.out_tokens[row] = (r.arg + 1) | (int32_t)((r.nonfinite ? 1u : 0u) << 31);
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
    const bool range = x < 0 || x >= a.V;
    if (range) flags |= FLAG_TOKEN_RANGE;
    // a proposal outside the vocabulary never matches, not even the -1 of a
    // row without an admissible id
    if (n == g && (range || x != (out[i] & 0x7FFFFFFF) - 1)) n = i;
  }
  for (int i = 0; i < G1; ++i) {
    const int32_t e = out[i];
    if (e < 0) flags |= FLAG_NONFINITE;
    const int32_t am = (e & 0x7FFFFFFF) - 1;
    if (i == n && am < 0) flags |= FLAG_EMPTY;
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
