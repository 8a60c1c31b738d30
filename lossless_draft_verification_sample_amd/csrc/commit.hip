// Chain KV-commit metadata after one verification round ("Speculative
// Decoding - Turn guesses into parallel work", section "Committed tokens versus
// cached states"; "Drafters and Speculative Decoding: Useful Tokens, Correct
// State", section "Committing state after rejection").
//
// Convention: before the round request b has kv_len[b] = K materialised target
// KV rows and its last committed token (the anchor) is pending. The target pass
// ran the anchor and the gamma proposals at positions K .. K+gamma, writing
// scratch rows there (slots[b][j] = physical slot of position K + j). After the
// round the anchor's row and the n accepted rows are history (new_kv_len =
// K + 1 + n), the emitted correction or bonus token becomes the pending anchor,
// and the rows of the gamma - n rejected proposals are freed in position order.
// Every output is written from the verifier's outputs alone, so the kernel can
// follow either verification entry point.

#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

constexpr int CM_THREADS = 256;
constexpr int CM_NW = CM_THREADS / WAVE;   // requests per workgroup

// One wave per request: lane j loads position j of the token and slot rows
// (gamma + 1 <= 64), so every load is issued at once and coalesced; the
// entries that depend on n are then picked with lane shuffles.
__global__ __launch_bounds__(CM_THREADS) void commit_kernel(CommitArgs a) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int b = blockIdx.x * CM_NW + (int)threadIdx.x / WAVE;
  if (b >= a.B) return;
  const int G1 = a.gamma + 1;
  const int g = a.gammas ? a.gammas[b] : a.gamma;   // the request's proposals
  const int n = a.num_accepted[b];
  const int32_t k = a.kv_len[b];
  const int32_t tok = lane < G1 ? a.tokens[(int64_t)b * G1 + lane] : -1;
  const int32_t slot = (a.free_slots && lane < G1) ? a.slots[(int64_t)b * G1 + lane] : -1;
  // an accepted count outside [0, g] (or a g outside [0, gamma]) is not a
  // verifier output: the request is left as it was (nothing committed,
  // nothing freed, no anchor)
  const bool ok = g >= 0 && g <= a.gamma && n >= 0 && n <= g;
  const int nn = ok ? n : 0;
  const int32_t anchor = __shfl(tok, nn, WAVE);
  if (a.free_slots) {
    const int nf = ok ? g - n : 0;
    const int32_t moved = __shfl(slot, min(nn + 1 + lane, WAVE - 1), WAVE);
    if (lane < a.gamma) a.free_slots[(int64_t)b * a.gamma + lane] = lane < nf ? moved : -1;
  }
  if (lane == 0) {
    a.new_kv_len[b] = ok ? k + 1 + n : k;
    a.anchor[b] = ok ? anchor : -1;
    if (a.n_free) a.n_free[b] = ok ? g - n : 0;
  }
}

int launch_commit(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3((a.B + CM_NW - 1) / CM_NW), dim3(CM_THREADS), 0, st, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
