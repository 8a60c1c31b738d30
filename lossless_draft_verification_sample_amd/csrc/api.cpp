// Host side of the C interface declared in include/spec_verify.h: argument
// validation (before anything touches the device), workspace carving and the
// kernel launch sequence on the caller's stream.
//
// Built twice: as the product library, and with SV_BENCH_TIMING as the
// benchmark library, which also records HIP event pairs around every launch
// (sv_bench_timing.h).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/spec_verify.h"
#include "sv_bans.hpp"
#include "sv_bench_timing.h"
#include "sv_launch.hpp"

// The penalized ids of a row (history plus up to 63 proposals) and a ban list
// must each fit the on-chip hash sets at most half full.
static_assert(SV_MAX_HISTORY + 63 <= (int)sv::HT_MAX_IDS, "penalty set bound");
static_assert(SV_MAX_BANNED <= (int)sv::HT_MAX_IDS, "ban set bound");

namespace {

constexpr size_t WS_ALIGN = 256;

size_t align_up(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

struct Layout {
  size_t stats, unif, sums, tickets, ov_partial, ov_tickets;
  size_t base;                // bytes up to here: everything but the draw's lists
  size_t lcount, lx, lw;      // the draw's kept-token lists (optional)
  size_t total;
  int nsub;
  int ov_spp, ov_parts;
};

// Draw workgroups per request (nwg), each over spw consecutive sub-chunks.
// A draw that may weigh every token of its row (a target sampler that keeps
// everything, or per-request target samplers, which only the device sees) is
// fp64 work on every token: one sub-chunk per wave, so that every wave takes
// part.
// Otherwise (a plain batch whose target sampler truncates) a draw weighs a few
// thousand tokens at most and extra workgroups only add their setup: about
// DRAW_TARGET_WGS in total, each over at most DRAW_SPW_MAX sub-chunks.
void draw_split(int64_t nsub, int64_t B, bool dense, int64_t* spw, int64_t* nwg) {
  if (dense) {
    *spw = nsub < sv::DRAW_WAVES ? nsub : sv::DRAW_WAVES;
  } else {
    int64_t n = (sv::DRAW_TARGET_WGS + B - 1) / B;
    if (n > nsub) n = nsub;
    *spw = (nsub + n - 1) / n;
    if (*spw > sv::DRAW_SPW_MAX) *spw = sv::DRAW_SPW_MAX;
  }
  *nwg = (nsub + *spw - 1) / *spw;
}

bool layout(int32_t B, int32_t gamma, int32_t V, Layout* L) {
  if (B < 1 || gamma < 1 || gamma > 63 || V < 1) return false;
  const int64_t rows = (int64_t)B * (2 * (int64_t)gamma + 1);
  if (rows >= INT32_MAX) return false;
  const int64_t nsub = ((int64_t)V + sv::DRAW_SUB - 1) / sv::DRAW_SUB;
  // the draw grid of either split must fit
  for (const bool dense : {false, true}) {
    int64_t spw, nwg;
    draw_split(nsub, B, dense, &spw, &nwg);
    if ((int64_t)B * nwg >= INT32_MAX) return false;
  }
  // overlap workgroups: about OV_TARGET_WGS in total, each over at most
  // OV_SPW_MAX sub-chunks of one (request, position) pair
  const int64_t pairs = (int64_t)B * gamma;
  int64_t parts = (sv::OV_TARGET_WGS + pairs - 1) / pairs;
  const int64_t min_parts = (nsub + sv::OV_SPW_MAX - 1) / sv::OV_SPW_MAX;
  if (parts < min_parts) parts = min_parts;
  if (parts > nsub) parts = nsub;
  const int64_t spp = (nsub + parts - 1) / parts;
  parts = (nsub + spp - 1) / spp;
  if (pairs * parts >= INT32_MAX) return false;
  L->nsub = (int)nsub;
  L->ov_spp = (int)spp;
  L->ov_parts = (int)parts;
  size_t off = 0;
  L->stats = off;
  off = align_up(off + (size_t)rows * sizeof(sv::RowStat));
  L->unif = off;
  off = align_up(off + (size_t)B * (size_t)(gamma + 1) * sizeof(double));
  L->sums = off;
  off = align_up(off + (size_t)B * (size_t)nsub * sizeof(sv::ChunkSums));
  L->tickets = off;
  off = align_up(off + (size_t)B * sizeof(int32_t));
  L->ov_partial = off;
  off = align_up(off + (size_t)pairs * (size_t)parts * sizeof(double));
  L->ov_tickets = off;
  off = align_up(off + (size_t)pairs * sizeof(int32_t));
  L->base = off;
  L->lcount = off;
  off = align_up(off + (size_t)B * (size_t)nsub * sizeof(int32_t));
  L->lx = off;
  off = align_up(off + (size_t)B * (size_t)nsub * sv::DRAW_LIST * sizeof(int32_t));
  L->lw = off;
  off = align_up(off + (size_t)B * (size_t)nsub * sv::DRAW_LIST * sizeof(double));
  L->total = off;
  return true;
}

bool sampler_ok(const sv_sampler& s) {
  if (!(s.temperature > 0.0f) || !isfinite(s.temperature)) return false;
  if (s.top_k < 0) return false;
  if (!(s.top_p > 0.0f && s.top_p <= 1.0f)) return false;
  return true;
}

sv::SamplerDev to_dev(const sv_sampler& s) {
  sv::SamplerDev d;
  d.temperature = s.temperature;
  d.top_k = s.top_k;
  d.top_p = s.top_p;
  d.pad = 0.0f;
  return d;
}

// ---------------------------------------------------------------- profiling

#ifdef SV_BENCH_TIMING
struct Prof {
  bool on = false;
  int cap = 0;
  std::vector<hipEvent_t> ev[SV_NUM_KERNELS];  // 2 per launch
  int used[SV_NUM_KERNELS] = {0};
};
Prof g_prof;

// Records an event pair around one launch while a profile is active.
struct ProfScope {
  int k;
  hipStream_t s;
  bool active;
  ProfScope(int kernel, hipStream_t stream) : k(kernel), s(stream), active(false) {
    if (g_prof.on && g_prof.used[k] < g_prof.cap) {
      active = hipEventRecord(g_prof.ev[k][2 * g_prof.used[k]], s) == hipSuccess;
    }
  }
  ~ProfScope() {
    if (active) {
      (void)hipEventRecord(g_prof.ev[k][2 * g_prof.used[k] + 1], s);
      ++g_prof.used[k];
    }
  }
};
#else
// The product library records nothing.
struct ProfScope {
  ProfScope(int, hipStream_t) {}
};
#endif

// ---------------------------------------------------------------- static scratch

// Workspace of spec_verify_sample_noalloc, for callers that cannot allocate
// device memory. Each device holds its own copy until the process ends. In
// host code this name is only a stand-in for the symbol: the device address
// comes from hipGetSymbolAddress, once per device, and only that address is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[MAX_DEVICES] = {nullptr};

// Device address of the current device's scratch array (resolved on the first
// call on that device, with that device current).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SV_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_EHIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SV_OK;
}

// The sampling call. With use_scratch the workspace is this device's static
// scratch array (spec_verify_sample_noalloc) instead of the caller's.
int sample_impl(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                const int32_t* draft_tokens, const int32_t* banned_ids, int32_t n_banned,
                int32_t B, int32_t gamma, int32_t V, sv_sampler target, sv_sampler draft,
                const sv_requests* requests, uint64_t seed, uint64_t offset,
                const double* uniforms, int32_t* out_tokens, int32_t* out_num_accepted,
                uint32_t* out_flags, float* out_target_lse, float* out_draft_lse,
                double* out_overlap, uint32_t* out_accept_hist, void* workspace,
                size_t workspace_bytes, bool use_scratch, void* stream) {
  if (!target_logits || !draft_logits || !draft_tokens || !out_tokens || !out_num_accepted)
    return SV_EINVAL;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_EDTYPE;
  if (B < 1 || gamma < 1 || gamma > 63 || V < 1) return SV_EINVAL;
  if (n_banned < 0 || n_banned > SV_MAX_BANNED || (n_banned > 0 && !banned_ids)) return SV_EINVAL;
  if (!sampler_ok(target) || !sampler_ok(draft)) return SV_EINVAL;
  sv::ReqArgs req{};
  if (requests) {
    if (requests->n_banned_draft < 0 || requests->n_banned_draft > SV_MAX_BANNED ||
        (requests->n_banned_draft > 0 && !requests->banned_draft))
      return SV_EINVAL;
    req.gammas = requests->gamma;
    req.ts = (const sv::SamplerReq*)requests->target;
    req.ds = (const sv::SamplerReq*)requests->draft;
    // a draft list (even an empty one) replaces banned_ids for the draft rows
    req.banned_d = requests->banned_draft;
    req.n_banned_d = requests->banned_draft ? requests->n_banned_draft : 0;
    if (requests->n_history < 0 || requests->n_history > SV_MAX_HISTORY ||
        (requests->n_history > 0 && !requests->history))
      return SV_EINVAL;
    req.history = requests->n_history > 0 ? requests->history : nullptr;
    req.n_history = req.history ? requests->n_history : 0;
    req.pen_t = requests->penalty;
    req.pen_d = requests->penalty_draft;
  }
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (((uintptr_t)target_logits % es) || ((uintptr_t)draft_logits % es)) return SV_EINVAL;
  Layout L;
  if (!layout(B, gamma, V, &L)) return SV_ESIZE;
  // The static scratch holds the draw's lists when they fit; larger sizes run
  // without them (the selection then rereads its sub-chunk: same results).
  bool lists = true;
  if (use_scratch) {
    if (L.total > (size_t)SV_NOALLOC_SCRATCH_BYTES) {
      if (L.base > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ESCRATCH;
      lists = false;
    }
    const int rc = scratch_ptr(&workspace);
    if (rc != SV_OK) return rc;
    workspace_bytes = SV_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || ((uintptr_t)workspace % WS_ALIGN) ||
      workspace_bytes < (lists ? L.total : L.base))
    return SV_EWORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  sv::RowStat* stats = (sv::RowStat*)(ws + L.stats);
  double* unif = (double*)(ws + L.unif);
  sv::ChunkSums* sums = (sv::ChunkSums*)(ws + L.sums);
  int32_t* tickets = (int32_t*)(ws + L.tickets);
  double* ov_partial = (double*)(ws + L.ov_partial);
  int32_t* ov_tickets = (int32_t*)(ws + L.ov_tickets);
  const int bf16 = dtype == SV_BF16;
  const int rows = B * (2 * gamma + 1);
  const int32_t* bans = n_banned ? banned_ids : nullptr;

  {
    sv::RowStatsArgs a{};
    a.target = target_logits;
    a.draft = draft_logits;
    a.gamma = gamma;
    a.V = V;
    a.st = to_dev(target);
    a.sd = to_dev(draft);
    a.draft_tokens = draft_tokens;
    a.banned = bans;
    a.n_banned = n_banned;
    a.stats = stats;
    a.tickets = tickets;
    a.ov_tickets = out_overlap ? ov_tickets : nullptr;
    a.accept_hist = out_accept_hist;
    a.req = req;
    a.out_tlse = out_target_lse;
    a.out_dlse = out_draft_lse;
    a.force_generic = 0;
    a.ustore = uniforms ? nullptr : unif;
    a.seed = seed;
    a.offset = offset;
    ProfScope p(SV_K_ROW_STATS, st);
    if (sv::launch_row_stats(a, bf16, rows, st)) return SV_EHIP;
  }
  {
    sv::DrawArgs a{};
    a.target = target_logits;
    a.draft = draft_logits;
    a.bf16 = bf16;
    a.vec = ((uintptr_t)target_logits % 16 == 0) && ((uintptr_t)draft_logits % 16 == 0) &&
            ((size_t)V * es) % 16 == 0;
    a.gamma = gamma;
    a.V = V;
    a.nsub = L.nsub;
    // per-request target samplers are only visible on the device; otherwise
    // every request uses the call's own
    const bool dense = req.ts || (target.top_k == 0 && target.top_p >= 1.0f);
    int64_t spw, nwg;
    draw_split(L.nsub, B, dense, &spw, &nwg);
    a.spw = (int)spw;
    a.nwg = (int)nwg;
    a.st = to_dev(target);
    a.sd = to_dev(draft);
    a.req = req;
    a.draft_tokens = draft_tokens;
    a.banned = bans;
    a.n_banned = n_banned;
    a.stats = stats;
    a.uniforms = uniforms ? uniforms : unif;
    a.sums = sums;
    a.lcount = lists ? (int32_t*)(ws + L.lcount) : nullptr;
    a.lx = lists ? (int32_t*)(ws + L.lx) : nullptr;
    a.lw = lists ? (double*)(ws + L.lw) : nullptr;
    a.tickets = tickets;
    a.out_tokens = out_tokens;
    a.out_num_accepted = out_num_accepted;
    a.out_flags = out_flags;
    a.accept_hist = out_accept_hist;
    ProfScope p(SV_K_DRAW, st);
    if (sv::launch_draw(a, B, st)) return SV_EHIP;
  }
  if (out_overlap) {
    sv::OverlapArgs a{};
    a.target = target_logits;
    a.draft = draft_logits;
    a.vec = ((uintptr_t)target_logits % 16 == 0) && ((uintptr_t)draft_logits % 16 == 0) &&
            ((size_t)V * es) % 16 == 0;
    a.gamma = gamma;
    a.V = V;
    a.nsub = L.nsub;
    a.spp = L.ov_spp;
    a.parts = L.ov_parts;
    a.st = to_dev(target);
    a.sd = to_dev(draft);
    a.req = req;
    a.banned = bans;
    a.n_banned = n_banned;
    a.stats = stats;
    a.draft_tokens = draft_tokens;
    a.partial = ov_partial;
    a.tickets = ov_tickets;
    a.out_overlap = out_overlap;
    ProfScope p(SV_K_OVERLAP, st);
    if (sv::launch_overlap(a, bf16, B * gamma, st)) return SV_EHIP;
  }
  return SV_OK;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t V) {
  Layout L;
  if (!layout(B, gamma, V, &L)) return 0;
  return L.total;
}

const char* spec_verify_strerror(int status) {
  switch (status) {
    case SV_OK: return "success";
    case SV_EINVAL: return "invalid argument (null pointer, size or sampler setting)";
    case SV_EDTYPE: return "unsupported dtype (expected SV_F32 or SV_BF16)";
    case SV_EWORKSPACE: return "workspace missing or smaller than spec_verify_workspace_bytes()";
    case SV_ESIZE: return "sizes exceed the supported index ranges";
    case SV_EHIP: return "HIP launch or runtime error";
    case SV_ESCRATCH:
      return "sizes need more workspace than spec_verify_sample_noalloc's static scratch holds";
    default: return "unknown status";
  }
}

int spec_verify_sample(const void* target_logits, const void* draft_logits, sv_dtype dtype,
                       const int32_t* draft_tokens, const int32_t* banned_ids,
                       int32_t n_banned, int32_t B, int32_t gamma, int32_t V,
                       sv_sampler target, sv_sampler draft, const sv_requests* requests,
                       uint64_t seed, uint64_t offset,
                       const double* uniforms, int32_t* out_tokens, int32_t* out_num_accepted,
                       uint32_t* out_flags, float* out_target_lse, float* out_draft_lse,
                       double* out_overlap, uint32_t* out_accept_hist,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return sample_impl(target_logits, draft_logits, dtype, draft_tokens, banned_ids, n_banned, B,
                     gamma, V, target, draft, requests, seed, offset, uniforms, out_tokens,
                     out_num_accepted, out_flags, out_target_lse, out_draft_lse, out_overlap,
                     out_accept_hist, workspace, workspace_bytes, false, stream);
}

int spec_verify_sample_noalloc(const void* target_logits, const void* draft_logits,
                               sv_dtype dtype, const int32_t* draft_tokens,
                               const int32_t* banned_ids, int32_t n_banned, int32_t B,
                               int32_t gamma, int32_t V, sv_sampler target, sv_sampler draft,
                               const sv_requests* requests, uint64_t seed, uint64_t offset,
                               const double* uniforms, int32_t* out_tokens,
                               int32_t* out_num_accepted, uint32_t* out_flags,
                               float* out_target_lse, float* out_draft_lse, double* out_overlap,
                               uint32_t* out_accept_hist, void* stream) {
  return sample_impl(target_logits, draft_logits, dtype, draft_tokens, banned_ids, n_banned, B,
                     gamma, V, target, draft, requests, seed, offset, uniforms, out_tokens,
                     out_num_accepted, out_flags, out_target_lse, out_draft_lse, out_overlap,
                     out_accept_hist, nullptr, 0, true, stream);
}

int spec_verify_greedy(const void* target_logits, sv_dtype dtype, const int32_t* draft_tokens,
                       const int32_t* banned_ids, int32_t n_banned,
                       int32_t B, int32_t gamma, int32_t V, int32_t* out_tokens,
                       int32_t* out_num_accepted, uint32_t* out_flags,
                       uint32_t* out_accept_hist, void* stream) {
  if (!target_logits || !draft_tokens || !out_tokens || !out_num_accepted) return SV_EINVAL;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_EDTYPE;
  if (B < 1 || gamma < 1 || gamma > 63 || V < 1) return SV_EINVAL;
  if (n_banned < 0 || n_banned > SV_MAX_BANNED || (n_banned > 0 && !banned_ids)) return SV_EINVAL;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if ((uintptr_t)target_logits % es) return SV_EINVAL;
  if ((int64_t)B * (gamma + 1) >= INT32_MAX) return SV_ESIZE;
  hipStream_t st = (hipStream_t)stream;
  sv::GreedyArgs a{target_logits, dtype == SV_BF16, gamma, V, B, draft_tokens,
                   n_banned ? banned_ids : nullptr, n_banned,
                   out_tokens, out_num_accepted, out_flags, out_accept_hist};
  {
    ProfScope p(SV_K_GREEDY_ARGMAX, st);
    if (sv::launch_greedy_argmax(a, st)) return SV_EHIP;
  }
  {
    ProfScope p(SV_K_GREEDY_SCAN, st);
    if (sv::launch_greedy_scan(a, st)) return SV_EHIP;
  }
  return SV_OK;
}

int spec_verify_commit(const int32_t* out_tokens, const int32_t* out_num_accepted,
                       const int32_t* kv_len, const int32_t* slots, const int32_t* gamma_b,
                       int32_t B, int32_t gamma,
                       int32_t* new_kv_len, int32_t* anchor, int32_t* n_free,
                       int32_t* free_slots, void* stream) {
  if (!out_tokens || !out_num_accepted || !kv_len || !new_kv_len || !anchor) return SV_EINVAL;
  if (free_slots && !slots) return SV_EINVAL;
  if (B < 1 || gamma < 1 || gamma > 63) return SV_EINVAL;
  if ((int64_t)B * (gamma + 1) >= INT32_MAX) return SV_ESIZE;
  hipStream_t st = (hipStream_t)stream;
  sv::CommitArgs a{out_tokens, out_num_accepted, kv_len, slots, B, gamma,
                   new_kv_len, anchor, n_free, free_slots, gamma_b};
  ProfScope p(SV_K_COMMIT, st);
  if (sv::launch_commit(a, st)) return SV_EHIP;
  return SV_OK;
}

#ifdef SV_BENCH_TIMING
int sv_bench_profile_start(int32_t max_launches_per_kernel) {
  if (g_prof.on || max_launches_per_kernel < 1) return SV_EINVAL;
  for (int k = 0; k < SV_NUM_KERNELS; ++k) {
    g_prof.ev[k].assign(2 * (size_t)max_launches_per_kernel, nullptr);
    for (auto& e : g_prof.ev[k])
      if (hipEventCreate(&e) != hipSuccess) return SV_EHIP;
    g_prof.used[k] = 0;
  }
  g_prof.cap = max_launches_per_kernel;
  g_prof.on = true;
  return SV_OK;
}

int sv_bench_profile_stop(double* total_ms, int32_t* launches) {
  if (!g_prof.on) return SV_EINVAL;
  int rc = SV_OK;
  for (int k = 0; k < SV_NUM_KERNELS; ++k) {
    double tot = 0.0;
    for (int j = 0; j < g_prof.used[k]; ++j) {
      float ms = 0.0f;
      if (hipEventSynchronize(g_prof.ev[k][2 * j + 1]) != hipSuccess ||
          hipEventElapsedTime(&ms, g_prof.ev[k][2 * j], g_prof.ev[k][2 * j + 1]) != hipSuccess)
        rc = SV_EHIP;
      tot += ms;
    }
    if (total_ms) total_ms[k] = tot;
    if (launches) launches[k] = g_prof.used[k];
    for (auto& e : g_prof.ev[k]) (void)hipEventDestroy(e);
    g_prof.ev[k].clear();
    g_prof.used[k] = 0;
  }
  g_prof.on = false;
  return rc;
}

#endif  // SV_BENCH_TIMING

}  // extern "C"
