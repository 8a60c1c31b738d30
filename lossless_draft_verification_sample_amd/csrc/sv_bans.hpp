// LDS hash set of token ids (linear probing), shared by the kernels that test
// single ids against a raw ban list or a row's repetition-penalized ids.
//
// Every set holds at most HT_MAX_IDS distinct ids, half of its slots: the host
// bounds the ban lists (SV_MAX_BANNED) and the penalized ids of a row (the
// history, SV_MAX_HISTORY, plus at most 63 earlier proposals) accordingly, so
// a probe sequence always meets an empty slot. The probe loops are also capped
// at HT_SLOTS steps, so no input can keep them spinning.
#pragma once

#include "sv_common.hpp"

namespace sv {

constexpr uint32_t HT_SLOTS = 4096;
constexpr uint32_t HT_EMPTY = 0xFFFFFFFFu;
constexpr uint32_t HT_MAX_IDS = HT_SLOTS / 2;

__device__ __forceinline__ uint32_t ht_slot(int32_t id) {
  return ((uint32_t)id * 0x9E3779B1u) >> 20;   // multiplicative hash, 12 bits
}

// Inserts `id` into the set; true when this call added it (false when it was
// already there).
__device__ __forceinline__ bool ht_insert(uint32_t* tab, int32_t id) {
  uint32_t slot = ht_slot(id);
  for (uint32_t probe = 0; probe < HT_SLOTS; ++probe) {
    const uint32_t old = atomicCAS(&tab[slot], HT_EMPTY, (uint32_t)id);
    if (old == HT_EMPTY) return true;
    if (old == (uint32_t)id) return false;
    slot = (slot + 1u) & (HT_SLOTS - 1u);
  }
  return false;   // a full set: unreachable within HT_MAX_IDS ids
}

// Inserts the valid ids of a raw ban list into the LDS hash set `tab` (all
// slots HT_EMPTY beforehand). Bit k of the result is set when this thread's
// k-th id (list index threadIdx.x + k * blockDim.x) was the copy that entered
// the set, so every distinct id has exactly one owner. `first` is list element
// threadIdx.x, loaded by the caller. Sets *xban when the list holds `x`.
__device__ __forceinline__ uint32_t ht_build(uint32_t* tab, const int32_t* bl, int nb, int V,
                                             int32_t first, int32_t x, uint32_t* xban) {
  uint32_t own = 0u;
  int k = 0;
  for (int j = threadIdx.x; j < nb; j += blockDim.x, ++k) {
    const int32_t id = j == (int)threadIdx.x ? first : bl[j];
    if (id < 0 || id >= V) continue;
    if (id == x) *xban = 1u;
    if (ht_insert(tab, id)) own |= 1u << k;
  }
  return own;
}

__device__ __forceinline__ bool ht_has(const uint32_t* tab, int32_t id) {
  uint32_t slot = ht_slot(id);
  for (uint32_t probe = 0; probe < HT_SLOTS; ++probe) {
    const uint32_t v = tab[slot];
    if (v == (uint32_t)id) return true;
    if (v == HT_EMPTY) return false;
    slot = (slot + 1u) & (HT_SLOTS - 1u);
  }
  return false;
}

}  // namespace sv
