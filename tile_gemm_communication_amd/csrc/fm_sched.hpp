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

// Producer workgroups of an AllGather launch (COMET-style split of
// workgroups into communication and computation roles): chunk c's source
// src[c] (null: already in X) is copied into rows of X by the first n_prod
// workgroups, chunks taken in `order`.
struct ProducerArgs {
  int n_prod, n_chunks;
  int64_t chunk_bytes;
  char* X;
  uint32_t* flags;
  uint32_t* counters;   // zero before and after every launch
  uint32_t epoch;
  uint8_t order[64];
  const char* src[64];
};

// Producer workgroup p of P: for each chunk in arrival order, copy its p-th
// share into X with write-through stores, wait until they have completed,
// then check in on the chunk's counter; the last of the P workgroups resets
// the counter and publishes the chunk's flag.
// All producers work on the same chunk at a time, so chunks complete in
// arrival order.  Chunks without a source are published by workgroup 0.
template <int NT>
__device__ __forceinline__ void produce_chunks(const ProducerArgs& pa) {
  const int p = blockIdx.x, P = pa.n_prod, t = threadIdx.x;
  const int64_t n16 = pa.chunk_bytes / 16;
  const int64_t per = cdiv(cdiv(n16, P), NT) * NT;
  const int64_t b0 = min((int64_t)p * per, n16), b1 = min(b0 + per, n16);
  if (p == 0 && t == 0)
    for (int c = 0; c < pa.n_chunks; ++c)
      if (!pa.src[c])
        __hip_atomic_store(pa.flags + c, pa.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  for (int a = 0; a < pa.n_chunks; ++a) {
    const int c = pa.order[a];
    if (!pa.src[c]) continue;
    const u32x4* __restrict__ src = reinterpret_cast<const u32x4*>(pa.src[c]);
    u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(pa.X + c * pa.chunk_bytes);
    int64_t i = b0 + t;
    for (; i + 3 * NT < b1; i += 4 * NT) {
      const u32x4 x0 = src[i], x1 = src[i + NT], x2 = src[i + 2 * NT], x3 = src[i + 3 * NT];
      store_through(dst + i, x0);
      store_through(dst + i + NT, x1);
      store_through(dst + i + 2 * NT, x2);
      store_through(dst + i + 3 * NT, x3);
    }
    for (; i < b1; i += NT) store_through(dst + i, src[i]);
    // this wave's write-through stores are in memory: no release needed
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (t == 0) {
      const uint32_t prev =
          __hip_atomic_fetch_add(pa.counters + c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == (uint32_t)P - 1) {
        __hip_atomic_store(pa.counters + c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pa.flags + c, pa.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Host: fill a ProducerArgs (order == null: index order).
inline void fill_producers(ProducerArgs& pa, int P, int n_chunks, int64_t chunk_bytes,
                           const void* const* src, const int32_t* order, void* X,
                           uint32_t* flags, uint32_t* counters, uint32_t epoch) {
  pa.n_prod = P;
  pa.n_chunks = n_chunks;
  pa.chunk_bytes = chunk_bytes;
  pa.X = (char*)X;
  pa.flags = flags;
  pa.counters = counters;
  pa.epoch = epoch;
  for (int c = 0; c < n_chunks; ++c) pa.src[c] = (const char*)src[c];
  for (int a = 0; a < n_chunks; ++a) pa.order[a] = (uint8_t)(order ? order[a] : a);
}


}  // namespace fm
