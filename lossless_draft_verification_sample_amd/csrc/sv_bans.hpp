// LDS hash set of a request's banned ids (linear probing, at most half full),
// shared by the kernels that test single ids against a raw ban list.
#pragma once

#include "sv_common.hpp"

namespace sv {

constexpr uint32_t HT_SLOTS = 4096;
constexpr uint32_t HT_EMPTY = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t ht_slot(int32_t id) {
  return ((uint32_t)id * 0x9E3779B1u) >> 20;   // multiplicative hash, 12 bits
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
    uint32_t slot = ht_slot(id);
    while (true) {
      const uint32_t old = atomicCAS(&tab[slot], HT_EMPTY, (uint32_t)id);
      if (old == HT_EMPTY) {
        own |= 1u << k;
        break;
      }
      if (old == (uint32_t)id) break;
      slot = (slot + 1u) & (HT_SLOTS - 1u);
    }
  }
  return own;
}

__device__ __forceinline__ bool ht_has(const uint32_t* tab, int32_t id) {
  uint32_t slot = ht_slot(id);
  while (true) {
    const uint32_t v = tab[slot];
    if (v == (uint32_t)id) return true;
    if (v == HT_EMPTY) return false;
    slot = (slot + 1u) & (HT_SLOTS - 1u);
  }
}

}  // namespace sv
