// fm_moe.hip -- the MoE path of one expert-parallel rank:
//   route   expert-sorted row index (counting sort, stable, deterministic)
//   layer 0 token gather fused into a grouped (per-expert, ragged-M) GEMM
//   layer 1 grouped GEMM with the top-k weighted scatter-reduce fused into
//           its epilogue (fp32 atomic adds into the token rows)
//
// COMET article, "COMET 的技术原理": the tensor shared by the MoE layers is
// decomposed along the token dimension so that the smallest communication and
// computation units line up; local data blocks are computed first.  Here the
// unit is a row tile of one expert's gathered tokens.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fm_sched.hpp"
#include "fm_tile.hpp"

namespace fm {

constexpr int kMaxLocalExperts = 64;
constexpr int kRouteThreads = 256;
constexpr int kRouteSeg = 16;                         // pairs per thread per chunk
constexpr int kRouteChunk = kRouteThreads * kRouteSeg;

// ---------------------------------------------------------------------------
// Route: one workgroup.  Pass 1 counts local pairs per expert; the exclusive
// scan of the counts gives expert_offsets.  Pass 2 walks the pairs in chunks
// of kRouteChunk; inside a chunk thread t owns the contiguous pairs
// [t*kRouteSeg, (t+1)*kRouteSeg), so ordering slots by (expert, chunk, thread,
// position) is ordering by (expert, pair id): a stable sort.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t* __restrict__ ids,
                                                               int64_t P, int e0, int n_local,
                                                               int32_t* __restrict__ sorted_pairs,
                                                               int32_t* __restrict__ offsets) {
  __shared__ int s_cnt[kMaxLocalExperts * kRouteThreads];   // [expert][thread]
  __shared__ int s_base[kMaxLocalExperts];
  __shared__ int s_tot[kMaxLocalExperts];
  __shared__ signed char s_e[kRouteChunk];
  const int t = threadIdx.x;

  // Pass 1: totals per expert.
  if (t < n_local) s_tot[t] = 0;
  __syncthreads();
  for (int64_t p = t; p < P; p += kRouteThreads) {
    const int e = ids[p] - e0;
    if (e >= 0 && e < n_local) atomicAdd(&s_tot[e], 1);
  }
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int e = 0; e < n_local; ++e) {
      s_base[e] = acc;
      offsets[e] = acc;
      acc += s_tot[e];
    }
    offsets[n_local] = acc;
  }
  __syncthreads();

  // Pass 2: stable placement, chunk by chunk.
  for (int64_t c0 = 0; c0 < P; c0 += kRouteChunk) {
    for (int i = t; i < kRouteChunk; i += kRouteThreads) {
      const int64_t p = c0 + i;
      int e = -1;
      if (p < P) {
        e = ids[p] - e0;
        if (e < 0 || e >= n_local) e = -1;
      }
      s_e[i] = (signed char)e;
    }
    for (int e = 0; e < n_local; ++e) s_cnt[e * kRouteThreads + t] = 0;
    __syncthreads();
    for (int i = 0; i < kRouteSeg; ++i) {
      const int e = s_e[t * kRouteSeg + i];
      if (e >= 0) s_cnt[e * kRouteThreads + t] += 1;
    }
    __syncthreads();
    if (t < n_local) {   // exclusive scan over threads for expert t
      int acc = 0;
      for (int u = 0; u < kRouteThreads; ++u) {
        const int v = s_cnt[t * kRouteThreads + u];
        s_cnt[t * kRouteThreads + u] = acc;
        acc += v;
      }
      s_tot[t] = acc;
    }
    __syncthreads();
    for (int i = 0; i < kRouteSeg; ++i) {
      const int e = s_e[t * kRouteSeg + i];
      if (e >= 0) {
        const int slot = s_base[e] + s_cnt[e * kRouteThreads + t];
        s_cnt[e * kRouteThreads + t] += 1;
        sorted_pairs[slot] = (int32_t)(c0 + t * kRouteSeg + i);
      }
    }
    __syncthreads();
    if (t < n_local) s_base[t] += s_tot[t];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM over the local experts.  The ragged tile list (per expert:
// ceil(rows_e / BM) x tiles_n tiles, expert by expert) is built on the device
// from expert_offsets, so no host round trip is needed.
// ---------------------------------------------------------------------------
struct MoeArgs {
  const char* A;              // layer 0: X [T, K]; layer 1: H [rows, K]
  const char* W;              // [n_local, K, N]
  char* out;                  // layer 0: H [rows, N] (16-bit); layer 1: out [T, N] fp32
  const int32_t* sorted_pairs;
  const int32_t* offsets;
  const float* weights;       // [T * topk] (layer 1)
  uint32_t* col_done;         // layer 1: finished tiles per N-tile column (self-resetting)
  int64_t K, N;
  int64_t spin_limit;
  int topk, n_local, tiles_n, group_m;
};

template <class E, int BM, int BN, int NW, bool SCATTER, bool KTAIL>
__global__ __launch_bounds__(64 * NW, 1) void moe_kernel(const MoeArgs a) {
  using Eng = Engine<E, BM, BN, KTAIL, NW>;
  __shared__ __attribute__((aligned(16))) char smem[Eng::LDS_BYTES];
  __shared__ int s_off[kMaxLocalExperts + 1];
  __shared__ int s_tile0[kMaxLocalExperts + 1];

  const int t = threadIdx.x;
  if (t <= a.n_local) s_off[t] = a.offsets[t];
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int e = 0; e < a.n_local; ++e) {
      s_tile0[e] = acc;
      acc += (int)cdiv(s_off[e + 1] - s_off[e], BM) * a.tiles_n;
    }
    s_tile0[a.n_local] = acc;
  }
  __syncthreads();

  Eng eng(smem, a.K);
  const int64_t N = a.N, K = a.K;
  const int total = s_tile0[a.n_local];
  const int G = gridDim.x;
  const int slot = xcd_slot(blockIdx.x, G);

  for (int L = slot; L < total; L += G) {
    int e = 0;
    while (e + 1 < a.n_local && s_tile0[e + 1] <= L) ++e;
    const int row_base = s_off[e];
    const int rows_e = s_off[e + 1] - row_base;
    const int tiles_me = (int)cdiv(rows_e, BM);
    int tm, tn;
    band_coords(L - s_tile0[e], tiles_me, a.tiles_n, min(a.group_m, tiles_me), tm, tn);
    const int m0 = tm * BM;
    const int64_t n0 = (int64_t)tn * BN;

    eng.set_a_base(a.A);
#pragma unroll
    for (int i = 0; i < Eng::A_DMA; ++i) {
      const int lr = min(m0 + eng.a_dma_row(i), rows_e - 1);
      int64_t src_row;
      if constexpr (SCATTER) {
        src_row = row_base + lr;                              // H rows are expert-sorted
      } else {
        src_row = a.sorted_pairs[row_base + lr] / a.topk;     // gather: token of the pair
      }
      eng.set_a(i, (uint32_t)(src_row * K * 2));
    }
    eng.set_b(a.W + (int64_t)e * K * N * 2, N * 2, n0, N);
    eng.run();

    // Epilogue through the LDS staging regions (whole-line global accesses).
    eng.ep_begin();
    if constexpr (SCATTER) {
      // out[token] += weight * row.  A token's top-k pairs sit in different
      // experts, never twice in one; the tiles of one N column therefore only
      // collide across experts, and expert e's tiles of column tn apply their
      // read-modify-write after every earlier expert's tiles of that column
      // (count per column, in expert order).  The adds are plain fp32 loads
      // and stores, in a fixed order: the combine is deterministic.
      if (e > 0 && t == 0)
        wait_count(a.col_done + tn, (uint32_t)(s_tile0[e] / a.tiles_n), a.spin_limit);
      __syncthreads();
      const int col = eng.ep_col();
      const bool col_ok = n0 + col < N;
#pragma unroll
      for (int i = 0; i < Eng::FM; ++i) {
        eng.ep_stage(i);
        float* dst[Eng::EP_READS];
        float wt[Eng::EP_READS];
#pragma unroll
        for (int q = 0; q < Eng::EP_READS; ++q) {
          const int lr = m0 + eng.ep_row(i, q);
          dst[q] = nullptr;
          wt[q] = 0.f;
          if (lr < rows_e && col_ok) {
            const int p = a.sorted_pairs[row_base + lr];
            wt[q] = a.weights[p];
            dst[q] = reinterpret_cast<float*>(a.out) + (int64_t)(p / a.topk) * N + n0 + col;
          }
        }
        f32x4 old[Eng::EP_READS];
#pragma unroll
        for (int q = 0; q < Eng::EP_READS; ++q)
          if (dst[q]) old[q] = *reinterpret_cast<const f32x4*>(dst[q]);
#pragma unroll
        for (int q = 0; q < Eng::EP_READS; ++q) {
          const f32x4 v = eng.ep_read(q);
          if (dst[q]) {
            f32x4 o = old[q];
            o[0] += wt[q] * v[0];
            o[1] += wt[q] * v[1];
            o[2] += wt[q] * v[2];
            o[3] += wt[q] * v[3];
            *reinterpret_cast<f32x4*>(dst[q]) = o;
          }
        }
      }
      wait_vmcnt<0>();   // this wave's stores are complete
      __syncthreads();
      if (t == 0) signal_count(a.col_done + tn, (uint32_t)(total / a.tiles_n));
    } else {
      // H rows in expert-sorted order, 16-bit.
      const int col = eng.ep_col();
      const bool col_ok = n0 + col < N;
#pragma unroll
      for (int i = 0; i < Eng::FM; ++i) {
        eng.ep_stage(i);
#pragma unroll
        for (int q = 0; q < Eng::EP_READS; ++q) {
          const int lr = m0 + eng.ep_row(i, q);
          const f32x4 v = eng.ep_read(q);
          if (lr < rows_e && col_ok) {
            const u32x2 pk = {E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
            *reinterpret_cast<u32x2*>(a.out + ((int64_t)(row_base + lr) * N + n0 + col) * 2) = pk;
          }
        }
      }
    }
    eng.ep_end();
  }
}

namespace {

struct MoeTile {
  int bm, bn, nw;
};

MoeTile moe_tile() {
  if (const char* env = std::getenv("FM_MOE_TILE")) {
    int bm = 0, bn = 0, nw = 0;
    const int got = std::sscanf(env, "%dx%dw%d", &bm, &bn, &nw);
    if (got >= 2 && (bm == 128 || bm == 256) && (bn == 128 || bn == 256)) {
      if (got < 3 || (nw != 4 && nw != 8)) nw = (bm == 256 && bn == 256) ? 8 : 4;
      if (!(bm == 128 && bn == 128 && nw == 8)) return {bm, bn, nw};
    }
  }
  return {256, 256, 8};
}

template <bool SCATTER>
fm_status_t launch_moe(fm_dtype_t dt, MoeTile cfg, MoeArgs& a, hipStream_t stream) {
  a.tiles_n = (int)cdiv(a.N, cfg.bn);
  a.group_m = 8;
  a.spin_limit = 1ll << 26;
  if (SCATTER) {
    if (a.tiles_n > kTileCounters) return FM_ERR_UNSUPPORTED;
    a.col_done = device_tile_counters();
    if (!a.col_done) return FM_ERR_HIP;
  }
  const dim3 grid(device_cu_count());
#define FM_LAUNCH(E, BM, BN, NW)                                                             \
  do {                                                                                       \
    if (a.K % kBK) /* ragged K: the 4-wave form keeps the tail path spill-free */            \
      hipLaunchKernelGGL((moe_kernel<E, BM, BN, 4, SCATTER, true>), grid, dim3(256), 0,       \
                         stream, a);                                                         \
    else                                                                                     \
      hipLaunchKernelGGL((moe_kernel<E, BM, BN, NW, SCATTER, false>), grid, dim3(64 * NW), 0, \
                         stream, a);                                                         \
  } while (0)
#define FM_LAUNCH_E(E)                                                                       \
  do {                                                                                       \
    if (cfg.bm == 256 && cfg.bn == 256) {                                                    \
      if (cfg.nw == 8) FM_LAUNCH(E, 256, 256, 8); else FM_LAUNCH(E, 256, 256, 4);            \
    } else if (cfg.bm == 256) {                                                              \
      if (cfg.nw == 8) FM_LAUNCH(E, 256, 128, 8); else FM_LAUNCH(E, 256, 128, 4);            \
    } else {                                                                                 \
      FM_LAUNCH(E, 128, 128, 4);                                                             \
    }                                                                                        \
  } while (0)
  if (dt == FM_F16) FM_LAUNCH_E(F16); else FM_LAUNCH_E(BF16);
#undef FM_LAUNCH_E
#undef FM_LAUNCH
  return launch_status();
}

fm_status_t check_route_args(int64_t T, int32_t topk, int32_t n_local, const int32_t* topk_ids,
                             const int32_t* sorted_pairs, const int32_t* expert_offsets) {
  if (T < 0 || topk < 1 || n_local < 1 || n_local > kMaxLocalExperts) return FM_ERR_INVALID_ARG;
  if (T * topk >= (1ll << 31)) return FM_ERR_UNSUPPORTED;
  if (!expert_offsets || (T > 0 && (!topk_ids || !sorted_pairs))) return FM_ERR_INVALID_ARG;
  return FM_OK;
}

}  // namespace
}  // namespace fm

using namespace fm;

extern "C" fm_status_t fm_moe_route(int64_t T, int32_t topk, int32_t expert_begin,
                                    int32_t n_local, const int32_t* topk_ids,
                                    int32_t* sorted_pairs, int32_t* expert_offsets,
                                    hipStream_t stream) {
  const fm_status_t st =
      check_route_args(T, topk, n_local, topk_ids, sorted_pairs, expert_offsets);
  if (st != FM_OK) return st;
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, stream, topk_ids, T * topk,
                     (int)expert_begin, (int)n_local, sorted_pairs, expert_offsets);
  return launch_status();
}

extern "C" fm_status_t fm_moe_gather_gemm(fm_dtype_t dt, int64_t T, int64_t hidden,
                                          int64_t ffn, int32_t topk, int32_t expert_begin,
                                          int32_t n_local, const void* X,
                                          const int32_t* topk_ids, const void* W1, void* H,
                                          int32_t* sorted_pairs, int32_t* expert_offsets,
                                          hipStream_t stream) {
  if (dt != FM_F16 && dt != FM_BF16) return FM_ERR_UNSUPPORTED;
  fm_status_t st = check_route_args(T, topk, n_local, topk_ids, sorted_pairs, expert_offsets);
  if (st != FM_OK) return st;
  if (hidden < 0 || ffn < 0 || hidden % 8 || ffn % 8) return FM_ERR_INVALID_ARG;
  if (T > 0 && ffn > 0 &&
      (!X || !W1 || !H || !aligned16(X) || !aligned16(W1) || !aligned16(H)))
    return FM_ERR_INVALID_ARG;
  // gathered-row byte offsets are 32-bit
  if (hidden >= (1ll << 22) || ffn >= (1ll << 22) || T * hidden >= (1ll << 31))
    return FM_ERR_UNSUPPORTED;
  st = fm_moe_route(T, topk, expert_begin, n_local, topk_ids, sorted_pairs, expert_offsets,
                    stream);
  if (st != FM_OK || T == 0 || ffn == 0) return st;
  MoeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = (const char*)X;
  a.W = (const char*)W1;
  a.out = (char*)H;
  a.sorted_pairs = sorted_pairs;
  a.offsets = expert_offsets;
  a.K = hidden;
  a.N = ffn;
  a.topk = topk;
  a.n_local = n_local;
  return launch_moe<false>(dt, moe_tile(), a, stream);
}

extern "C" fm_status_t fm_moe_gemm_scatter(fm_dtype_t dt, int64_t T, int64_t hidden,
                                           int64_t ffn, int32_t topk, int32_t n_local,
                                           const void* H, const void* W2,
                                           const int32_t* sorted_pairs,
                                           const int32_t* expert_offsets,
                                           const float* topk_weights, float* out,
                                           hipStream_t stream) {
  if (dt != FM_F16 && dt != FM_BF16) return FM_ERR_UNSUPPORTED;
  if (T < 0 || topk < 1 || n_local < 1 || n_local > kMaxLocalExperts) return FM_ERR_INVALID_ARG;
  if (hidden < 0 || ffn < 0 || hidden % 8 || ffn % 8) return FM_ERR_INVALID_ARG;
  if (!expert_offsets) return FM_ERR_INVALID_ARG;
  if (T == 0 || hidden == 0) return FM_OK;
  if (!H || !W2 || !sorted_pairs || !topk_weights || !out || !aligned16(H) || !aligned16(W2) ||
      !aligned16(out))
    return FM_ERR_INVALID_ARG;
  if (hidden >= (1ll << 22) || ffn >= (1ll << 22) || T * topk * ffn >= (1ll << 31))
    return FM_ERR_UNSUPPORTED;
  MoeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = (const char*)H;
  a.W = (const char*)W2;
  a.out = (char*)out;
  a.sorted_pairs = sorted_pairs;
  a.offsets = expert_offsets;
  a.weights = topk_weights;
  a.K = ffn;
  a.N = hidden;
  a.topk = topk;
  a.n_local = n_local;
  return launch_moe<true>(dt, moe_tile(), a, stream);
}
