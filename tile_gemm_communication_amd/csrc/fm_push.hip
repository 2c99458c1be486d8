// fm_push.hip -- producer side of the chunk-arrival protocol.
//
// A chunk is copied with coalesced 16-byte loads and write-through stores by a
// small grid; every workgroup waits until its stores have reached memory
// (visible to every XCD) and checks in on a counter; the last one to check in
// resets the counter and publishes the chunk's flag.  This is the signalled one-sided put of
// the FlagCX guide ("flagcxPutSignal": write the data, then bump the remote
// signal) and the push mode of the FLUX review ("拉取 vs 推送数据传输"), with
// the peer's buffer being local HBM on one GPU.
#include <algorithm>
#include <cstring>

#include "fm_common.hpp"

namespace fm {

__global__ __launch_bounds__(256) void push_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16,
                                                   uint32_t* flag, uint32_t* counter,
                                                   uint32_t epoch) {
  const int64_t per = cdiv(n16, (int64_t)gridDim.x);
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = min(begin + per, n16);
  int64_t i = begin + threadIdx.x;
  for (; i + 3 * 256 < end; i += 4 * 256) {
    const u32x4 a = src[i], b = src[i + 256], c = src[i + 512], d = src[i + 768];
    store_through(dst + i, a);
    store_through(dst + i + 256, b);
    store_through(dst + i + 512, c);
    store_through(dst + i + 768, d);
  }
  for (; i < end; i += 256) store_through(dst + i, src[i]);
  // Every wave waits until its write-through stores have completed; after the
  // barrier the workgroup's part of the chunk is in memory, so the count and
  // the flag need no release (which would write back this XCD's whole L2,
  // once per workgroup, under the GEMM that runs beside the copy).
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Paced arrival: the a-th flag of the schedule is published once the
// device's constant-rate wall clock has advanced by `at[a]` ticks since the
// kernel started.  One lane does the work; the wait is bounded by the last
// arrival time, which the host limits.
struct PacedArgs {
  uint32_t* flags;
  uint32_t epoch;
  int32_t n;
  int32_t chunk[64];
  uint64_t at[64];
};

__global__ __launch_bounds__(64) void paced_kernel(const PacedArgs p) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = wall_clock64();
  for (int a = 0; a < p.n; ++a) {
    while (wall_clock64() - t0 < p.at[a]) __builtin_amdgcn_s_sleep(4);
    __hip_atomic_store(p.flags + p.chunk[a], p.epoch, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace fm

using namespace fm;

extern "C" fm_status_t fm_chunk_signal_paced(uint32_t* flags, int32_t n_chunks,
                                             const int32_t* order, const int64_t* arrive_ns,
                                             uint32_t epoch, hipStream_t stream) {
  if (!flags || (reinterpret_cast<uintptr_t>(flags) & 3u) || !arrive_ns) return FM_ERR_INVALID_ARG;
  if (n_chunks < 1 || n_chunks > 64) return FM_ERR_INVALID_ARG;
  PacedArgs p;
  std::memset(&p, 0, sizeof(p));
  p.flags = flags;
  p.epoch = epoch;
  p.n = n_chunks;
  bool seen[64] = {};
  for (int a = 0; a < n_chunks; ++a) {
    const int c = order ? order[a] : a;
    if (c < 0 || c >= n_chunks || seen[c]) return FM_ERR_INVALID_ARG;
    seen[c] = true;
    // arrival times: non-decreasing, at most one second
    if (arrive_ns[a] < 0 || arrive_ns[a] > 1000000000ll || (a > 0 && arrive_ns[a] < arrive_ns[a - 1]))
      return FM_ERR_INVALID_ARG;
    p.chunk[a] = c;
  }
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    return FM_ERR_HIP;
  for (int a = 0; a < n_chunks; ++a)   // round up: a signal is never early
    p.at[a] = (uint64_t)((arrive_ns[a] * (int64_t)khz + 999999) / 1000000);
  hipLaunchKernelGGL(paced_kernel, dim3(1), dim3(64), 0, stream, p);
  return launch_status();
}

extern "C" fm_status_t fm_chunk_push(const void* src, void* dst, int64_t bytes, uint32_t* flag,
                                     uint32_t* counter, uint32_t epoch, int32_t n_workgroups,
                                     hipStream_t stream) {
  if (!flag || !counter || bytes < 0 || bytes % 16 || n_workgroups < 0) return FM_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(flag) & 3u) || (reinterpret_cast<uintptr_t>(counter) & 3u))
    return FM_ERR_INVALID_ARG;
  if (bytes > 0 && (!src || !dst || !aligned16(src) || !aligned16(dst))) return FM_ERR_INVALID_ARG;
  if (bytes > 0) {
    const char* s = (const char*)src;
    const char* d = (const char*)dst;
    if (s < d + bytes && d < s + bytes) return FM_ERR_INVALID_ARG;   // overlap
  }
  const int64_t n16 = bytes / 16;
  // Default: one workgroup per 96 KiB, at most two per CU.  Each thread
  // keeps four 16-byte loads in flight (16 KiB per workgroup).  A 12.6 MB
  // chunk gets 128 workgroups.  Beside the TP=8 AllGather-GEMM
  // (4096x6144x12288, 7 chunks on 3 streams) 16/32/64/128/256 workgroups
  // per chunk gave 0.660/0.622/0.597/0.584/0.585 ms for the fused call.
  int wg = n_workgroups > 0
               ? n_workgroups
               : (int)std::min<int64_t>(std::max<int64_t>(cdiv(bytes, 98304), 1),
                                        2 * (int64_t)device_cu_count());
  if (n16 == 0) wg = 1;
  else if (wg > cdiv(n16, 256)) wg = (int)cdiv(n16, 256);
  hipLaunchKernelGGL(push_kernel, dim3(wg), dim3(256), 0, stream, (const u32x4*)src, (u32x4*)dst,
                     n16, flag, counter, epoch);
  return launch_status();
}

extern "C" fm_status_t fm_chunk_push_dma(const void* src, void* dst, int64_t bytes,
                                         uint32_t* flag, uint32_t epoch, hipStream_t stream) {
  if (!flag || bytes < 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(flag) & 3u))
    return FM_ERR_INVALID_ARG;
  if (bytes > 0 && (!src || !dst || !aligned16(src) || !aligned16(dst))) return FM_ERR_INVALID_ARG;
  if (bytes > 0) {
    const char* s = (const char*)src;
    const char* d = (const char*)dst;
    if (s < d + bytes && d < s + bytes) return FM_ERR_INVALID_ARG;   // overlap
    if (hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDeviceToDeviceNoCU, stream) !=
        hipSuccess)
      return FM_ERR_HIP;
  }
  if (hipStreamWriteValue32(stream, flag, epoch, 0) != hipSuccess) return FM_ERR_HIP;
  return FM_OK;
}
