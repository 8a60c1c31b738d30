// Kernel argument blocks and host-side launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_common.hpp"

namespace sv {

// Final draw: one workgroup sums the weights of DRAW_CHUNK tokens, reported per
// DRAW_SUB tokens; the selection then rescans a single sub-chunk.
constexpr int DRAW_CHUNK = 8192;
constexpr int DRAW_SUB = 2048;
constexpr int SUB_PER_CHUNK = DRAW_CHUNK / DRAW_SUB;

struct BanPrepArgs {
  const int32_t* banned;  // [B][n_banned]
  int n_banned;
  int V;
  int32_t* ban_sorted;    // [B][n_banned] sorted unique ids in [0, V)
  int32_t* ban_count;     // [B]
};

struct RowStatsArgs {
  const void* target;
  const void* draft;
  int gamma, V;
  SamplerDev st, sd;
  const int32_t* ban_sorted;  // or nullptr
  const int32_t* ban_count;   // or nullptr
  int ban_stride;
  RowStat* stats;             // [B][2*gamma+1]: target rows 0..gamma, then draft rows
  float* out_tlse;
  float* out_dlse;
  int force_generic;
};

struct AcceptArgs {
  const void* target;
  const void* draft;
  int bf16;
  int gamma, V;
  float t_temp, d_temp;
  const int32_t* draft_tokens;
  const int32_t* ban_sorted;
  const int32_t* ban_count;
  int ban_stride;
  const RowStat* stats;
  const double* uniforms;
  uint64_t seed, offset;
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  ReqState* req;
};

struct DrawArgs {
  const void* target;
  const void* draft;
  int bf16;
  int vec;                    // rows 16-byte aligned and V*size a multiple of 16
  int gamma, V, nchunk, nsub;
  float t_temp, d_temp;
  const int32_t* ban_sorted;
  const int32_t* ban_count;
  int ban_stride;
  const RowStat* stats;
  const ReqState* req;
  ChunkSums* sums;            // [B][nsub]
  int32_t* out_tokens;
  uint32_t* out_flags;
};

struct GreedyArgs {
  const void* target;
  int bf16;
  int gamma, V, B;
  const int32_t* draft_tokens;
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  uint32_t* out_flags;
};

int launch_ban_prep(const BanPrepArgs& a, int B, hipStream_t s);
int launch_row_stats(const RowStatsArgs& a, int dtype_bf16, int rows, hipStream_t s);
int launch_accept(const AcceptArgs& a, int B, hipStream_t s);
int launch_residual_partial(const DrawArgs& a, int B, hipStream_t s);
int launch_residual_select(const DrawArgs& a, int B, hipStream_t s);
int launch_greedy_argmax(const GreedyArgs& a, hipStream_t s);
int launch_greedy_scan(const GreedyArgs& a, hipStream_t s);

}  // namespace sv
