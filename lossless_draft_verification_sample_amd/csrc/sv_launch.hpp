// Kernel argument blocks and host-side launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_common.hpp"

namespace sv {

// Final draw: the vocabulary is cut into sub-chunks of DRAW_SUB tokens; each
// draw workgroup sums the weights of up to DRAW_SPW_MAX consecutive sub-chunks,
// and the selection rescans a single sub-chunk.
constexpr int DRAW_SUB = 2048;
constexpr int DRAW_SPW_MAX = 16;
// about 3.5 draw workgroups per CU: below the four per CU that can be resident,
// so that a launch runs in one round with room to spare (1,024 for c5, 8 per
// request, was 0.9 µs slower; B = 96 at 1,024 needed 1,056 and a second round)
constexpr int DRAW_TARGET_WGS = 896;
constexpr int DRAW_WAVES = 4;           // waves per draw workgroup
// kept tokens a draw workgroup lists per sub-chunk of a truncated row (more:
// the selection rescans the sub-chunk)
constexpr int DRAW_LIST = 32;

// Per-position overlap: every (request, position) pair is split into `parts`
// workgroups of at most OV_SPW_MAX sub-chunks, about OV_TARGET_WGS in total.
constexpr int OV_SPW_MAX = 32;
constexpr int OV_TARGET_WGS = 2048;

struct RowStatsArgs {
  const void* target;
  const void* draft;
  int gamma, V;
  SamplerDev st, sd;
  const int32_t* draft_tokens;  // [B][gamma]
  const int32_t* banned;        // [B][n_banned] raw ban lists, or nullptr
  int n_banned;
  RowStat* stats;               // [B][2*gamma+1]: target rows 0..gamma, then draft rows
  int32_t* tickets;             // [B] draw-kernel arrival counters, zeroed here
  int32_t* ov_tickets;          // [B][gamma] overlap arrival counters, zeroed here, or nullptr
  uint32_t* accept_hist;        // [gamma+1] zeroed here, or nullptr
  ReqArgs req;
  float* out_tlse;
  float* out_dlse;
  int force_generic;
  // Philox uniforms of the acceptance walk and the final draw, [B][gamma+1]:
  // target row i writes slot i. nullptr when the caller supplies the uniforms.
  double* ustore;
  uint64_t seed, offset;
};

struct DrawArgs {
  const void* target;
  const void* draft;
  int bf16;
  int vec;                    // rows 16-byte aligned and V*size a multiple of 16
  int gamma, V, nsub;
  int spw, nwg;               // sub-chunks per workgroup, workgroups per request
  const int32_t* draft_tokens;
  const int32_t* banned;      // raw ban lists or nullptr
  int n_banned;
  const RowStat* stats;
  const double* uniforms;     // [B][gamma+1]: the caller's, or those of the row pass
  ChunkSums* sums;            // [B][nsub]
  int32_t* lcount;            // [B][nsub]: tokens listed, DRAW_LIST + 1 when not listed;
                              // nullptr: no lists (every selection rereads its sub-chunk)
  int32_t* lx;                // [B][nsub][DRAW_LIST]: their ids
  double* lw;                 // [B][nsub][DRAW_LIST]: their draw weights
  int32_t* tickets;           // [B], zero on entry
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  uint32_t* out_flags;
  uint32_t* accept_hist;      // [gamma+1], zero on entry, or nullptr
  SamplerDev st, sd;          // call-wide samplers
  ReqArgs req;
};

struct OverlapArgs {
  const void* target;
  const void* draft;
  int vec;                    // rows 16-byte aligned and V*size a multiple of 16
  int gamma, V, nsub;
  int spp, parts;             // sub-chunks per workgroup, workgroups per pair
  const int32_t* banned;      // raw ban lists or nullptr
  int n_banned;
  const int32_t* draft_tokens;  // [B][gamma]
  const RowStat* stats;
  double* partial;            // [B*gamma][parts] when parts > 1
  int32_t* tickets;           // [B*gamma], zero on entry, when parts > 1
  double* out_overlap;        // [B][gamma]
  SamplerDev st, sd;          // call-wide samplers
  ReqArgs req;
};

struct GreedyArgs {
  const void* target;
  int bf16;
  int gamma, V, B;
  const int32_t* draft_tokens;
  const int32_t* banned;        // [B][n_banned] raw ban lists, or nullptr
  int n_banned;
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  uint32_t* out_flags;
  uint32_t* accept_hist;        // [gamma+1] or nullptr
};

struct CommitArgs {
  const int32_t* tokens;        // [B][gamma+1] verifier output
  const int32_t* num_accepted;  // [B]
  const int32_t* kv_len;        // [B] materialised rows before the round
  const int32_t* slots;         // [B][gamma+1] or nullptr (only with free_slots)
  int B, gamma;
  int32_t* new_kv_len;          // [B]
  int32_t* anchor;              // [B]
  int32_t* n_free;              // [B] or nullptr
  int32_t* free_slots;          // [B][gamma] or nullptr
  const int32_t* gammas;        // [B] proposals of each request, or nullptr (all gamma)
};

int launch_row_stats(const RowStatsArgs& a, int dtype_bf16, int rows, hipStream_t s);
int launch_draw(const DrawArgs& a, int B, hipStream_t s);
int launch_overlap(const OverlapArgs& a, int bf16, int pairs, hipStream_t s);
int launch_greedy_argmax(const GreedyArgs& a, hipStream_t s);
int launch_greedy_scan(const GreedyArgs& a, hipStream_t s);
int launch_commit(const CommitArgs& a, hipStream_t s);

}  // namespace sv
