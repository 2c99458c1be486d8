// fm_sched.hpp -- persistent tile scheduling and chunk-flag waits.
//
// Tile scheduling (the FLUX review's "瓦片坐标 Swizzling": a naive tile
// mapping makes concurrent tiles contend for memory, so tile coordinates are
// rearranged):
//  * The grid is persistent: G workgroups (G <= number of CUs), workgroup w
//    takes schedule positions L = slot(w), slot(w) + G, ...
//  * Workgroups are dispatched round-robin over the 8 XCDs (w -> XCD w % 8).
//    slot() makes the 32 workgroups of one XCD take 32 consecutive schedule
//    positions, so the tiles in flight on an XCD share A rows and B columns
//    in that XCD's L2.
//  * Schedule positions walk bands of `group_m` M-tiles column by column, so
//    32 consecutive positions form a compact group_m x (32/group_m) block.
//  * An optional M-tile order (morder) decides which rows come first: chunk
//    arrival order for AllGather, destination rank order starting at rank+1
//    for ReduceScatter.
#pragma once

#include "fm_common.hpp"

namespace fm {

constexpr int kMaxMOrder = 256;

struct TileOrder {
  int tiles_m, tiles_n, total, group_m;
  int has_morder;
  uint16_t morder[kMaxMOrder];
};

__device__ __forceinline__ int xcd_slot(int wg, int G) {
  return (G & 7) == 0 ? ((wg & 7) * (G >> 3) + (wg >> 3)) : wg;
}

__device__ __forceinline__ void band_coords(int L, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn) {
  const int band_tiles = group_m * tiles_n;
  const int band = L / band_tiles;
  const int idx = L - band * band_tiles;
  const int rows_left = tiles_m - band * group_m;
  const int gm = rows_left < group_m ? rows_left : group_m;
  tm = band * group_m + idx % gm;
  tn = idx / gm;
}

// Chunk readiness: flags[c] has reached `epoch` (wrap-safe comparison).
__device__ __forceinline__ bool flag_reached(uint32_t v, uint32_t epoch) {
  return (int32_t)(v - epoch) >= 0;
}

// Called by one thread: wait until every chunk in [c_lo, c_hi] is published.
// `ready` caches chunks this workgroup has already acquired.  Polls use
// relaxed device-scope loads with s_sleep backoff; one acquire fence follows
// the last new observation, so the chunk data is read only after its flag.
// Returns false (after writing FM_ERR_TIMEOUT to err) once `limit` polls pass.
__device__ __forceinline__ bool wait_chunks(const uint32_t* flags, uint32_t epoch, int c_lo,
                                            int c_hi, uint64_t& ready, int64_t limit,
                                            int32_t* err) {
  bool fresh = false;
  for (int c = c_lo; c <= c_hi; ++c) {
    if ((ready >> c) & 1ull) continue;
    int64_t polls = 0;
    while (!flag_reached(__hip_atomic_load(flags + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                         epoch)) {
      __builtin_amdgcn_s_sleep(2);
      if (++polls > limit) {
        if (err) __hip_atomic_store(err, (int32_t)FM_ERR_TIMEOUT, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
    }
    ready |= 1ull << c;
    fresh = true;
  }
  if (fresh) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// Store 16 bytes written through every cache level (system-scope store):
// once the wave's vmcnt drains, the data is visible device-wide without an
// L2 write-back.  Used for data that a counted tile hands to a tile that may
// run on another XCD (each XCD has its own, non-coherent L2).
__device__ __forceinline__ void store_through(float* p, const f32x4& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}

}  // namespace fm
