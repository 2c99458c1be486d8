// fm_moe.hip -- the MoE path of one expert-parallel rank:
//   route   expert-sorted row index (chunked counting sort, stable, deterministic)
//   layer 0 token gather fused into a grouped (per-expert, ragged-M) GEMM
//   layer 1 grouped GEMM with the top-k weighted scatter-reduce fused into
//           its epilogue (ordered fp32 read-modify-write into the token rows)
//
// COMET article, "COMET 的技术原理": the tensor shared by the MoE layers is
// decomposed along the token dimension so that the smallest communication and
// computation units line up; local data blocks are computed first.  Here the
// unit is a row tile of one expert's gathered tokens.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "fm_sched.hpp"
#include "fm_tile.hpp"

namespace fm {

constexpr int kMaxLocalExperts = 64;
constexpr int kMaxMTiles = 1024;                      // token ranges cached in LDS
constexpr int kMaxBands = 256;                        // bands ordered by arrival in LDS
constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / 64;

// ---------------------------------------------------------------------------
// Workspace of the MoE operators: caller-owned device memory, zero-filled once
// before its first use; every call leaves it ready for the next.  Layout, in
// uint32 words (every region at a fixed offset, so a workspace may serve
// calls of different shapes one after another):
//   [0, 64)       control words of the combine (below)
//   [64, 320)     1 KiB the combine's epilogue reads and writes in place of
//                 rows it does not own (lanes past the last row or column),
//                 so that every wave issues the same number of memory
//                 instructions per block; its contents are meaningless
//   [320, +16384) route: per-chunk expert histograms of the counting sort
//   [16704, ...)  combine: one completion epoch per (M-tile, N-tile)
// The route region and the combine regions are disjoint: a route (or MoE
// layer 0) and a combine may use one workspace at the same time; two routes,
// or two combines, may not.
// ---------------------------------------------------------------------------
constexpr int kCtlEpoch = 0;     // the last combine launch's epoch
constexpr int kCtlDone = 1;      // workgroups of the running combine that finished
constexpr int kCtlAbort = 3;     // = epoch once a wait of that launch gave up
constexpr int kCtlQueue = 8;     // [8, 12): next ticket of each combine tile queue
constexpr int kMaxQueues = 4;    // combine tile queues (XCDs x and x + 4 share one)
// The combine's register-fetch epilogue addresses out (at most
// kVepMaxRecords bytes) by 32-bit offsets, each the sum of a row part and a
// column part.  A missing row adds kVepNoRow, a missing column kVepNoCol: any
// sum with a missing part lies in [kVepMaxRecords, 2^32), past the end of out,
// where a buffer load returns 0 and a store is dropped.
constexpr uint32_t kVepMaxRecords = 0x7FFFFFF0u;
constexpr uint32_t kVepNoRow = 0x80000000u;
constexpr uint32_t kVepNoCol = 0x7FFFFFF0u;
constexpr int64_t kWsSink = 64;
constexpr int64_t kWsRoute = kWsSink + 256;
constexpr int64_t kRouteWords = 16384;
constexpr int64_t kWsFlags = kWsRoute + kRouteWords;
constexpr int kMinTileEdge = 128;   // the smallest BM and BN of any combine tile
static_assert((kWsSink * 4) % 16 == 0, "the sink must be 16-byte aligned");

// Pairs per route workgroup: one round of kRouteThreads, doubled until the
// per-chunk histograms fit the route region.
inline int64_t route_chunk_pairs(int64_t P, int n_local) {
  int64_t ch = kRouteThreads;
  while (std::max<int64_t>(1, cdiv(P, ch)) * n_local > kRouteWords) ch *= 2;
  return ch;
}

// Completion flags the combine needs: one per (M-tile, N-tile) for the
// smallest tile, with M-tiles <= pairs / BM + one partial tile per expert.
inline int64_t combine_flag_words(int64_t pairs, int64_t hidden, int n_local) {
  return (cdiv(pairs, kMinTileEdge) + n_local) * cdiv(hidden, kMinTileEdge);
}

inline size_t moe_ws_bytes(int64_t pairs, int64_t hidden, int n_local) {
  const int64_t words = kWsFlags + combine_flag_words(pairs, hidden, n_local);
  return (size_t)cdiv(words * 4, 256) * 256;
}

// ---------------------------------------------------------------------------
// Route: a counting sort over chunks of `ch` consecutive pairs (256 unless
// the histograms need larger chunks), one workgroup per chunk.
//   count: per-chunk histogram of local experts.
//   place: every workgroup derives its chunk's first slot per expert from
//          the histograms (totals -> expert_offsets, plus the counts of the
//          earlier chunks), then walks its chunk in rounds of 256 pairs in
//          pair order.  Within a round a pair's rank among same-expert pairs
//          of its wave comes from a ballot, and earlier waves' counts come
//          from LDS, so slots follow pair order: the sort is stable.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(
    const int32_t* __restrict__ ids, int64_t P, int e0, int n_local, int64_t ch,
    uint32_t* __restrict__ counts) {
  __shared__ int s_cnt[kMaxLocalExperts];
  const int t = threadIdx.x;
  if (t < n_local) s_cnt[t] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * ch, p1 = min(p0 + ch, P);
  for (int64_t p = p0 + t; p < p1; p += kRouteThreads) {
    const int e = ids[p] - e0;
    if (e >= 0 && e < n_local) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  if (t < n_local) counts[(int64_t)blockIdx.x * n_local + t] = (uint32_t)s_cnt[t];
}

__global__ __launch_bounds__(kRouteThreads) void route_place_kernel(
    const int32_t* __restrict__ ids, int64_t P, int e0, int n_local, int64_t ch, int n_chunks,
    const uint32_t* __restrict__ counts, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ offsets) {
  __shared__ int s_base[kMaxLocalExperts];            // next slot per expert
  __shared__ int s_tot[kMaxLocalExperts];
  __shared__ int s_wcnt[kRouteWaves][kMaxLocalExperts];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c = blockIdx.x;
  if (t < n_local) {
    s_tot[t] = 0;
    s_base[t] = 0;
  }
  __syncthreads();
  {
    // Every thread sums part of the histograms: thread t takes expert
    // t % n_local of every (S / n_local)-th chunk from t / n_local on, and
    // adds its totals (all chunks, and the chunks before this one) into LDS.
    const int S = (kRouteThreads / n_local) * n_local;
    if (t < S) {
      const int e = t % n_local;
      int tot = 0, pre = 0;
      for (int cc = t / n_local; cc < n_chunks; cc += S / n_local) {
        const int v = (int)counts[(int64_t)cc * n_local + e];
        pre += cc < c ? v : 0;
        tot += v;
      }
      if (tot) atomicAdd(&s_tot[e], tot);
      if (pre) atomicAdd(&s_base[e], pre);
    }
  }
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int e = 0; e < n_local; ++e) {
      s_base[e] += acc;
      if (c == 0) offsets[e] = acc;
      acc += s_tot[e];
    }
    if (c == 0) offsets[n_local] = acc;
  }
  const int64_t p0 = (int64_t)c * ch, p1 = min(p0 + ch, P);
  for (int64_t r0 = p0; r0 < p1; r0 += kRouteThreads) {
    if (t < kRouteWaves * kMaxLocalExperts) (&s_wcnt[0][0])[t] = 0;
    __syncthreads();
    const int64_t p = r0 + t;
    int e = -1;
    if (p < p1) {
      e = ids[p] - e0;
      if (e < 0 || e >= n_local) e = -1;
    }
    // rank among the earlier lanes of this wave with the same expert
    int rank = 0;
    uint64_t todo = __ballot(e >= 0);
    while (todo) {
      const int le = __shfl(e, __ffsll((unsigned long long)todo) - 1);
      const uint64_t m = __ballot(e == le);
      if (e == le) rank = __popcll(m & ((1ull << lane) - 1));
      if (lane == 0) s_wcnt[w][le] = __popcll(m);
      todo &= ~m;
    }
    __syncthreads();
    if (e >= 0) {
      int slot = s_base[e] + rank;
      for (int v = 0; v < w; ++v) slot += s_wcnt[v][e];
      sorted_pairs[slot] = (int32_t)p;
    }
    __syncthreads();
    if (t < n_local) {
      int add = 0;
      for (int v = 0; v < kRouteWaves; ++v) add += s_wcnt[v][t];
      s_base[t] += add;
    }
    __syncthreads();   // s_wcnt is cleared for the next round
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
  uint32_t* tile_done;        // layer 1: per (M-tile, N-tile) completion epoch
  uint32_t* ws;               // layer 1: the workspace (control words, sink)
  int64_t K, N;
  int64_t spin_limit;
  int topk, n_local, tiles_n, group_m;
  int act;                    // layer 0: activation of the fp32 result (fm_act_t)
  // Tail split (layer 0): when the last wave of 256x256 tiles would fill at
  // most half of g_ref CUs, part 0 runs the full waves and part 1 the
  // remaining tiles as 256x128 halves.  tiles_n always counts 256-wide tiles.
  int split, part, g_ref;
  int64_t rows_cap;           // T * topk: an upper bound on the local rows
  // Combine: bytes of out (T x N fp32) when at most kVepMaxRecords, which
  // selects the register-fetch epilogue over a buffer resource; 0 selects the
  // LDS-DMA one.
  uint32_t out_records;
  // Layer 0 behind a token AllGather (flags != null): chunk c holds tokens
  // [c*chunk_tokens, (c+1)*chunk_tokens) and is read after flags[c] >= epoch.
  const uint32_t* flags;
  uint32_t chunk_epoch;
  int64_t chunk_tokens;
  int32_t* err_word;
  int64_t chunk_spin;
  // Bands of ag_group M-tiles of one expert run in the order of the last
  // chunk they need to arrive (chunk_pos[c] = arrival position of chunk c).
  int ag_group;
  uint8_t chunk_pos[64];
  // Token chunks copied by the first prod.n_prod workgroups of layer 0's own
  // launch (prod.n_prod == 0: the chunks arrive from elsewhere).
  ProducerArgs prod;
  // Pull mode (layer 0): token chunk c is read in place from pull_src[c].
  const char* pull_src[64];
};


// Activation of layer 0's fp32 result (fm_act_t), from the definitions:
// ReLU max(x, 0); GELU in its tanh form x/2 (1 + tanh(u)) with u =
// sqrt(2/pi) (x + 0.044715 x^3); SiLU x / (1 + exp(-x)).  The exponentials
// use the hardware exp (__expf) and tanh(u) = 1 - 2 / (exp(2u) + 1), so the
// epilogue makes no library calls (which would spill the accumulators around
// them); both stay exact in the limits (exp overflowing to inf gives tanh 1
// and SiLU -0).  Their fp32 error is far below the 16-bit rounding of H.
__device__ __forceinline__ float apply_act(int act, float x) {
  switch (act) {
    case FM_ACT_RELU:
      return fmaxf(x, 0.f);
    case FM_ACT_GELU_TANH: {
      const float u = 0.7978845608028654f * (x + 0.044715f * x * x * x);
      const float th = 1.f - 2.f / (__expf(2.f * u) + 1.f);
      return 0.5f * x * (1.f + th);
    }
    case FM_ACT_SILU:
      return x / (1.f + __expf(-x));
    default:
      return x;
  }
}

// Called by the 64 lanes of one wave: wait until every tile of an expert
// before e in column tn whose token range overlaps that of global M-tile gm
// has published this call's epoch, then acquire.  The tiles to wait for are
// a range of global M-tiles per earlier expert: lane ep finds expert ep's
// range, a scan over the wave lays the ranges end to end in s_wr ([0, 64):
// first tile, [64, 128): first position), and lane l polls positions l,
// l + 64, ..., so the polls are in flight together (one lane polling them
// in turn paid a round trip per flag).  Beyond kMaxMTiles tiles the ranges
// are not cached and every earlier tile of the column is waited for.
// Returns false (on every lane) if the wait gave up: after spin_limit polls
// of one flag (that lane then writes FM_ERR_TIMEOUT to err_word and marks
// the launch aborted in the workspace), or once another workgroup has
// marked it aborted.
__device__ __forceinline__ bool wait_token_range(const MoeArgs& a, const int* s_tile0,
                                                 const int* s_ftok, const int* s_ltok,
                                                 int* s_wr, int total_m, int e, int gm, int tn,
                                                 uint32_t epoch, int lane) {
  const bool cached = total_m <= kMaxMTiles;
  const int lo_tok = cached ? s_ftok[gm] : 0;
  const int hi_tok = cached ? s_ltok[gm] : 0x7FFFFFFF;
  uint32_t* const abort_word = a.ws + kCtlAbort;
  // this lane's expert (e <= 63 < 64): its tiles [m_lo, m_hi) overlap
  int m_lo = 0, cnt = 0;
  if (lane < e) {
    const int g0 = s_tile0[lane] / a.tiles_n, g1 = s_tile0[lane + 1] / a.tiles_n;
    int lo = g0, hi = g1;
    if (cached) {
      while (lo < hi) {   // first tile whose last token is >= lo_tok
        const int mid = (lo + hi) >> 1;
        if (s_ltok[mid] < lo_tok) lo = mid + 1; else hi = mid;
      }
      m_lo = lo;
      hi = g1;
      while (lo < hi) {   // first tile whose first token is > hi_tok
        const int mid = (lo + hi) >> 1;
        if (s_ftok[mid] <= hi_tok) lo = mid + 1; else hi = mid;
      }
      cnt = lo - m_lo;
    } else {
      m_lo = g0;
      cnt = g1 - g0;
    }
  }
  int incl = cnt;   // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  const int total = __shfl(incl, 63);
  s_wr[lane] = m_lo;
  s_wr[64 + lane] = incl - cnt;
  bool ok = true;
  for (int j = lane; ok && j < total; j += 64) {
    int lo = 0, hi = e - 1;   // the last expert whose first position is <= j
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_wr[64 + mid] <= j) lo = mid; else hi = mid - 1;
    }
    const int m = s_wr[lo] + (j - s_wr[64 + lo]);
    const uint32_t* f = a.tile_done + (int64_t)m * a.tiles_n + tn;
    int64_t polls = 0;
    while (!flag_reached(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                         epoch)) {
      __builtin_amdgcn_s_sleep(2);
      ++polls;
      if ((polls & 63) == 0 &&
          __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) {
        ok = false;
        break;
      }
      if (polls > a.spin_limit) {
        if (a.err_word)
          __hip_atomic_store(a.err_word, (int32_t)FM_ERR_TIMEOUT, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(abort_word, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = false;
        break;
      }
    }
  }
  ok = __all(ok);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok;
}

// Combine tile queues.  The N columns are dealt to Q = min(4, tiles_n)
// queues, column tn to queue tn % Q, and a workgroup takes its tiles from
// the queue of its XCD (XCDs x and x + 4 share one): the tiles in flight on
// one L2 then share their B columns and, four columns to an M-tile, their A
// rows.  A queue's tickets walk the global M-tiles in order (all of expert
// 0's, then expert 1's, ...), each M-tile's columns of the queue in turn.  A
// tile only waits for tiles of earlier experts in its own column: tiles of
// the same queue with smaller tickets.  (EP=8 combine: L2 misses 29% fewer
// than with one queue for all tiles, time equal within 1%; eight queues, one
// per XCD, were 1.7% slower: each queue's last, small experts then wait on
// each other among fewer workgroups.)
struct CombineQueues {
  int Q, total_m, tiles_n;
  __device__ __forceinline__ int cols(int q) const { return (tiles_n - q + Q - 1) / Q; }
  __device__ __forceinline__ int size(int q) const { return total_m * cols(q); }
  // ticket t of queue q: global M-tile gm, column tn
  __device__ __forceinline__ void tile(int q, int t, int& gm, int& tn) const {
    const int c = cols(q);
    gm = t / c;
    tn = q + (t - gm * c) * Q;
  }
};

// The XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ int xcc_id() {
  return (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & 15u);
}

template <class E, int BM, int BN, int NW, bool SCATTER, bool KTAIL, bool PULL = false,
          bool ACT = false, bool VEP = false>
__global__ __launch_bounds__(64 * NW, 1) void moe_kernel(const MoeArgs a) {
  // One wave per SIMD has the register room for a two-sub-step read-ahead.
  // PULL: the token rows are gathered from the owners' chunk buffers, one
  // 64-bit address per row.
  static_assert(!(SCATTER && PULL), "pull mode is a layer-0 form");
  // ACT: layer 0 with an activation (a.act); a separate instantiation, so
  // the plain form carries none of its code.
  static_assert(!(ACT && (SCATTER || PULL)), "the activation is a plain layer-0 form");
  // VEP: the combine's register-fetch epilogue (out below 2 GiB, a.out_records).
  static_assert(!VEP || SCATTER, "the register-fetch epilogue is the combine's");
  using Eng = Engine<E, BM, BN, KTAIL, NW, 4, NW == 4 ? 2 : 1, false, PULL, BN == 128 ? 3 : 2>;
  // the combine's epilogue also keeps its destination rows in LDS
  constexpr int kSmem =
      (SCATTER && Eng::EP_RMW_LDS > Eng::LDS_BYTES) ? Eng::EP_RMW_LDS : Eng::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ int s_off[kMaxLocalExperts + 1];
  __shared__ int s_tile0[kMaxLocalExperts + 1];
  __shared__ int s_tok[SCATTER ? BM : 1];      // combine: token and gate weight per tile row
  __shared__ float s_wt[SCATTER ? BM : 1];
  // combine: first and last token of every M-tile (all experts, in order)
  __shared__ int s_ftok[SCATTER ? kMaxMTiles : 1];
  __shared__ int s_ltok[SCATTER ? kMaxMTiles : 1];
  __shared__ int s_wr[SCATTER ? 128 : 1];   // combine: wave 0's table of tiles to wait for
  __shared__ int s_abort;
  // combine: this tile has a row whose token also has the previous row (two
  // pairs of one token in one expert), and the next ticket (by tile parity)
  __shared__ int s_dup;
  __shared__ int s_next_q[2], s_next_t[2];
  // token AllGather: bands of M-tiles sorted by the arrival of their chunks
  __shared__ int s_band0[SCATTER ? 1 : kMaxLocalExperts + 1];
  __shared__ uint8_t s_blvl[SCATTER ? 1 : kMaxBands];
  __shared__ uint16_t s_bord[SCATTER ? 1 : kMaxBands];   // expert << 8 | band of the expert
  __shared__ int s_btile0[SCATTER ? 1 : kMaxBands + 1];
  uint64_t ready = 0;   // token chunks this workgroup has already acquired

  int wg = blockIdx.x, G = gridDim.x;
  if constexpr (!SCATTER) {
    // Producers take the lowest workgroup ids: they are dispatched before any
    // consumer that may wait on their chunks.
    if (wg < a.prod.n_prod) {
      produce_chunks<64 * NW>(a.prod);
      return;
    }
    wg -= a.prod.n_prod;
    G -= a.prod.n_prod;
  }
  const int t = threadIdx.x;
  const int gmb = SCATTER ? 1 : a.ag_group;
  // Combine: this launch's epoch (never 0, the flags' initial value).
  uint32_t epoch = 0;
  if constexpr (SCATTER) {
    epoch = __hip_atomic_load(a.ws + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
    if (epoch == 0) epoch = 1;
    if (t == 0) s_dup = 0;
  }
  if (t <= a.n_local) s_off[t] = a.offsets[t];
  __syncthreads();
  if (t == 0) {
    int acc = 0, nb = 0;
    for (int e = 0; e < a.n_local; ++e) {
      const int tiles_me = (int)cdiv(s_off[e + 1] - s_off[e], BM);
      s_tile0[e] = acc;
      acc += tiles_me * a.tiles_n;
      if constexpr (!SCATTER) {
        s_band0[e] = nb;
        nb += (tiles_me + gmb - 1) / gmb;
      }
    }
    s_tile0[a.n_local] = acc;
    if constexpr (!SCATTER) s_band0[a.n_local] = nb;
  }
  __syncthreads();

  // Token AllGather: a band of up to ag_group M-tiles of one expert covers an
  // increasing token range; bands run in the order in which the last chunk
  // they need arrives (stable, so expert-major within one arrival position).
  // This only orders the tiles: every tile still waits for its own chunks.
  bool by_arrival = false;
  int n_bands = 0;
  if constexpr (!SCATTER) {
    n_bands = s_band0[a.n_local];
    by_arrival = a.flags != nullptr && n_bands <= kMaxBands;
    if (by_arrival) {
      for (int g = t; g < n_bands; g += 64 * NW) {
        int e = 0;
        while (e + 1 < a.n_local && s_band0[e + 1] <= g) ++e;
        const int b = g - s_band0[e];
        const int rows_e = s_off[e + 1] - s_off[e];
        const int r0 = s_off[e] + b * gmb * BM;
        const int r1 = s_off[e] + min((b + 1) * gmb * BM, rows_e) - 1;
        const int c_lo = (int)(a.sorted_pairs[r0] / a.topk / a.chunk_tokens);
        const int c_hi = (int)(a.sorted_pairs[r1] / a.topk / a.chunk_tokens);
        int lvl = 0;
        for (int c = c_lo; c <= c_hi; ++c) lvl = max(lvl, (int)a.chunk_pos[c]);
        s_blvl[g] = (uint8_t)lvl;
      }
      __syncthreads();
      for (int g = t; g < n_bands; g += 64 * NW) {
        const int lvl = s_blvl[g];
        int rank = 0;
        for (int g2 = 0; g2 < n_bands; ++g2) {
          const int l2 = s_blvl[g2];
          rank += (l2 < lvl) | ((l2 == lvl) & (g2 < g));
        }
        int e = 0;
        while (e + 1 < a.n_local && s_band0[e + 1] <= g) ++e;
        s_bord[rank] = (uint16_t)((e << 8) | (g - s_band0[e]));
      }
      __syncthreads();
      if (t == 0) {
        int acc = 0;
        for (int k = 0; k < n_bands; ++k) {
          const int e = s_bord[k] >> 8, b = s_bord[k] & 255;
          const int tiles_me = (int)cdiv(s_off[e + 1] - s_off[e], BM);
          s_btile0[k] = acc;
          acc += min(gmb, tiles_me - b * gmb) * a.tiles_n;
        }
        s_btile0[n_bands] = acc;
      }
      __syncthreads();
    }
  }

  // Combine: token range of every M-tile.  Rows of an expert are sorted by
  // pair id, hence by token, and hold each token at most once, so the tiles
  // of one expert cover disjoint, increasing token ranges.
  const int total_m = s_tile0[a.n_local] / a.tiles_n;
  if constexpr (SCATTER) {
    for (int m = t; m < total_m && m < kMaxMTiles; m += 64 * NW) {
      int e = 0;
      while (e + 1 < a.n_local && s_tile0[e + 1] / a.tiles_n <= m) ++e;
      const int tm = m - s_tile0[e] / a.tiles_n;
      const int rows_e = s_off[e + 1] - s_off[e];
      const int r0 = s_off[e] + tm * BM, r1 = s_off[e] + min((tm + 1) * BM, rows_e) - 1;
      s_ftok[m] = a.sorted_pairs[r0] / a.topk;
      s_ltok[m] = a.sorted_pairs[r1] / a.topk;
    }
    __syncthreads();
  }

  Eng eng(smem, a.K);
  const int64_t N = a.N, K = a.K;
  const int total = s_tile0[a.n_local];
  const int slot = xcd_slot(wg, G);
  int full = total;
  if (a.split) {
    const int rem = total % a.g_ref;
    if (rem > 0 && 2 * rem <= a.g_ref) full = total - rem;
  }
  const int sub_n = a.part ? 2 : 1;                  // BN = 256 / sub_n
  const int pos0 = a.part ? full : 0;
  const int n_items = a.part ? 2 * (total - full) : full;

  // Combine: flag index of the last tile whose stores are not yet known to
  // be complete (-1: none).  publish() is called by every thread after a
  // wait for this wave's stores and a barrier.
  int pending = -1;
  auto publish = [&] {
    if (pending >= 0 && t == 0)
      __hip_atomic_store(a.tile_done + pending, epoch, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    pending = -1;
  };

  // Layer 0: static positions slot, slot + G, ...
  // Combine: tickets of the tile queues.  A workgroup takes its tiles from
  // its home queue (its XCD's), each ticket taken ahead during the previous
  // tile's K loop; once the home queue is exhausted it takes tickets of the
  // other queues one at a time, with nothing taken ahead.  A ticket taken
  // ahead is never one the current tile waits for (a later ticket of the
  // same queue), and a ticket taken from another queue is never held while
  // waiting, so every ticket taken is held by a running workgroup that can
  // finish it, whatever share of the CUs the launch gets.  Thread 0 takes
  // the tickets; `dead` holds the queues it found exhausted.
  CombineQueues cqs{1, 0, 1};
  int home = 0, cq = 0, ct = -1;
  uint32_t dead = 0;
  auto take = [&](int q) -> int {
    const uint32_t v = __hip_atomic_fetch_add(a.ws + kCtlQueue + q, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (v < (uint32_t)cqs.size(q)) return (int)v;
    dead |= 1u << q;
    return -1;
  };
  auto steal = [&](int& q) -> int {   // the home queue last
    for (int k = 1; k <= cqs.Q; ++k) {
      const int r = (home + k) % cqs.Q;
      if (dead & (1u << r)) continue;
      const int v = take(r);
      if (v >= 0) {
        q = r;
        return v;
      }
    }
    return -1;
  };
  if constexpr (SCATTER) {
    cqs = CombineQueues{min(kMaxQueues, a.tiles_n), total_m, a.tiles_n};
    home = xcc_id() % cqs.Q;
    if (t == 0) {
      int q = home;
      int v = take(home);
      if (v < 0) v = steal(q);
      s_next_q[1] = q;
      s_next_t[1] = v;
    }
    __syncthreads();
    cq = s_next_q[1];
    ct = s_next_t[1];
  }
  int L2 = SCATTER ? 0 : slot;
  for (int it = 0; SCATTER ? (ct >= 0) : (L2 < n_items); ++it) {
    const int L = pos0 + L2 / sub_n, sub = L2 % sub_n;
    int e = 0, tm, tn;
    if constexpr (SCATTER) {
      int gm;
      cqs.tile(cq, ct, gm, tn);
      while (e + 1 < a.n_local && s_tile0[e + 1] / a.tiles_n <= gm) ++e;
      tm = gm - s_tile0[e] / a.tiles_n;
    } else if (by_arrival) {
      int lo = 0, hi = n_bands - 1;   // last band starting at or before L
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_btile0[mid] <= L) lo = mid; else hi = mid - 1;
      }
      e = s_bord[lo] >> 8;
      const int b = s_bord[lo] & 255;
      const int tiles_e = (int)cdiv(s_off[e + 1] - s_off[e], BM);
      const int rows_b = min(gmb, tiles_e - b * gmb);
      const int li = L - s_btile0[lo];
      tm = b * gmb + li % rows_b;
      tn = li / rows_b;
    } else {
      while (e + 1 < a.n_local && s_tile0[e + 1] <= L) ++e;
      const int tiles_e = (int)cdiv(s_off[e + 1] - s_off[e], BM);
      band_coords(L - s_tile0[e], tiles_e, a.tiles_n, min(a.group_m, tiles_e), tm, tn);
    }
    const int row_base = s_off[e];
    const int rows_e = s_off[e + 1] - row_base;
    const int m0 = tm * BM;
    const int64_t n0 = ((int64_t)tn * sub_n + sub) * BN;
    if (!SCATTER && n0 >= N) {   // the right half of an edge tile that lies past N
      L2 += G;
      continue;
    }

    if constexpr (!SCATTER) {
      if (a.flags) {
        // Token AllGather: rows of an expert are sorted by token, so the tile
        // needs the chunks from its first row's token to its last row's.
        if (t == 0) {
          const int r_last = row_base + min(m0 + BM, rows_e) - 1;
          const int64_t tok_lo = a.sorted_pairs[row_base + m0] / a.topk;
          const int64_t tok_hi = a.sorted_pairs[r_last] / a.topk;
          const bool ok = wait_chunks(a.flags, a.chunk_epoch, (int)(tok_lo / a.chunk_tokens),
                                      (int)(tok_hi / a.chunk_tokens), ready, a.chunk_spin,
                                      a.err_word);
          s_abort = ok ? 0 : 1;
        }
        __syncthreads();
        const int abort_now = s_abort;
        __syncthreads();
        if (abort_now) return;   // timed out: err_word is set, H is undefined
      }
    }

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
      if constexpr (PULL) {
        const int c = (int)(src_row / a.chunk_tokens);       // the token's owner
        eng.set_a64(i, a.pull_src[c] + (src_row - (int64_t)c * a.chunk_tokens) * K * 2);
      } else {
        eng.set_a(i, (uint32_t)(src_row * K * 2));
      }
    }
    eng.set_b(a.W + (int64_t)e * K * N * 2, N * 2, n0, N);
    // Combine: fetch each tile row's pair id now, so that the load overlaps
    // the K loop (the K loop's first wait drains it with the stage-0 DMA).
    int my_p = -1, prev_p = -1;
    int next_q = 0, next_t = -1;
    if constexpr (SCATTER) {
      if (t < BM && m0 + t < rows_e) {
        my_p = a.sorted_pairs[row_base + m0 + t];
        if (m0 + t > 0) prev_p = a.sorted_pairs[row_base + m0 + t - 1];
      }
    }
    eng.run([&] {
      if constexpr (SCATTER) {
        publish();
        // the next ticket of the home queue, taken now and kept in a
        // register until the epilogue (its return drains with the K loop's
        // first wait); -2: take one of another queue after this tile
        if (t == 0) {
          next_q = home;
          next_t = -2;
          if (cq == home && !(dead & (1u << home))) {
            const int v = take(home);
            if (v >= 0) next_t = v;
          }
        }
      }
    });

    // Epilogue through the LDS staging regions (whole-line global accesses).
    eng.ep_begin();
    if constexpr (SCATTER) {
      // out[token] += weight * row.  A token's top-k pairs sit in different
      // experts, never twice in one; the tiles of one N column therefore only
      // collide across experts, and expert e's tiles of column tn apply their
      // read-modify-write after every earlier expert's tiles of that column
      // (count per column, in expert order).  The adds are plain fp32 loads
      // and stores, in a fixed order: the combine is deterministic.
      // Row metadata into LDS: the token (the register-fetch form: its row's
      // byte offset in out) and the gate weight, with a no-row mark past the
      // expert's rows.
      // Rows of an expert are sorted by pair id, so two pairs of one token in
      // one expert (an input the combine does not accept) are neighbours.
      if (t == 0) {
        s_next_q[it & 1] = next_q;
        s_next_t[it & 1] = next_t;
      }
      if (t < BM) {
        if constexpr (VEP)   // the row's byte offset in out (or the no-row mark)
          s_tok[t] = (int)(my_p >= 0 ? (uint32_t)(my_p / a.topk) * ((uint32_t)a.N * 4u)
                                     : kVepNoRow);
        else
          s_tok[t] = my_p >= 0 ? my_p / a.topk : -1;
        s_wt[t] = my_p >= 0 ? a.weights[my_p] : 0.f;
        if (my_p >= 0 && prev_p >= 0 && my_p / a.topk == prev_p / a.topk) s_dup = 1;
      }
      // Wait for the tiles of earlier experts in this N column whose token
      // ranges overlap this tile's: they hold every earlier contribution to
      // this tile's tokens, and are usually long finished (each expert walks
      // its tokens in order, about one expert's worth of tiles earlier).
      const int gm = s_tile0[e] / a.tiles_n + tm;   // this tile's global M-tile
      if (t < 64) {   // wave 0
        const bool ok =
            e == 0 ||
            wait_token_range(a, s_tile0, s_ftok, s_ltok, s_wr, total_m, e, gm, tn, epoch, t);
        if (t == 0) s_abort = ok ? 0 : 1;
      }
      __syncthreads();
      // A wait that gave up ends this workgroup's work (err_word is set, out
      // is undefined); a duplicated token skips the tile's adds and is
      // reported, and its flag still goes out.
      const bool skip = s_abort != 0 || s_dup != 0;
      if (t == 0 && s_dup && a.err_word)
        __hip_atomic_store(a.err_word, (int32_t)FM_ERR_INVALID_ARG, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      if constexpr (VEP) {
        // Register-fetch form.  Per wave and 32-row block i: the accumulators
        // are staged through LDS into whole rows, weight * row is added to
        // the destination values and the sums are stored through.  The
        // destination rows of AHEAD blocks are in flight at a time, in
        // registers (the K loop's fragment registers are free here): block
        // i+AHEAD's are requested right after block i's stores.  Loads and
        // stores go through a buffer resource over out, so the compiler counts
        // them in its waits; a lane with nothing to add (a row past the
        // expert's rows, a column past N, a skipped tile) uses an offset past
        // the end of out, which loads 0 and drops the store.
        constexpr int R = Eng::EP_READS;
        constexpr int H = R / 2;
        // blocks in flight per wave: two with one wave per SIMD; one with
        // two (the SIMD's other wave covers the wait, and the registers are
        // half as many)
        constexpr int AHEAD = NW == 4 ? 2 : 1;
        static_assert(Eng::FM >= AHEAD, "blocks in flight");
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(a.out, 0, (int)a.out_records, kBufRsrcWord3);
        // Offset = the row's part (s_tok, kVepNoRow for no row) + the
        // lane's column part (kVepNoCol past N or for a skipped tile): one
        // add per access, no branch (a branch per row would make each row's
        // read wait on its own).
        const int col = eng.ep_col();
        const uint32_t col_bytes =
            (!skip && n0 + col < N) ? (uint32_t)(n0 + col) * 4u : kVepNoCol;
        auto offsets = [&](int i, uint32_t(&o)[R]) {
#pragma unroll
          for (int q = 0; q < R; ++q) o[q] = (uint32_t)s_tok[eng.ep_row(i, q)] + col_bytes;
        };
        f32x4 d[AHEAD][R];
        auto fetch = [&](int i, f32x4(&dd)[R]) {
          uint32_t o[R];
          offsets(i, o);
#pragma unroll
          for (int q = 0; q < R; ++q)
            dd[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o[q], 0, 0));
        };
#pragma unroll
        for (int b = 0; b < AHEAD; ++b) fetch(b, d[b]);
        static_for<Eng::FM>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          uint32_t so[R];
          offsets(i, so);
          float wt[R];
#pragma unroll
          for (int q = 0; q < R; ++q) wt[q] = s_wt[eng.ep_row(i, q)];
          eng.template ep_stage<false>(i);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f32x4 v[H];
#pragma unroll
            for (int u = 0; u < H; ++u) v[u] = eng.ep_read(h * H + u);
#pragma unroll
            for (int u = 0; u < H; ++u) {
              const int q = h * H + u;
              f32x4 o = d[i % AHEAD][q];
              o[0] += wt[q] * v[u][0];
              o[1] += wt[q] * v[u][1];
              o[2] += wt[q] * v[u][2];
              o[3] += wt[q] * v[u][3];
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rs, so[q], 0,
                                                     kBufStoreThrough);
            }
          }
          if constexpr (i + AHEAD < Eng::FM) fetch(i + AHEAD, d[i % AHEAD]);
        });
      } else {
        // Per wave and 32-row block i: the destination rows come into LDS by
        // DMA, the accumulators are staged, and weight * row is added and
        // stored through.  Block i+1's rows are requested before block i's
        // stores, so a store never delays the next loads (vmcnt counts loads
        // and stores in issue order).  Each block goes in two halves of H
        // reads, which bounds the registers the results hold.  Lanes past the
        // last row or column read and write the sink instead, so every live
        // block issues exactly H loads and H stores per half and the waits can
        // count them; blocks past the last row (or a wave past the last
        // column) issue nothing.  Issue order: D(i) h0, D(i) h1 [block 0 only],
        // then per half h of block i: D(i+1) h, S(i) h.
        constexpr int H = Eng::EP_READS / 2;
        const int col = eng.ep_col();
        const bool col_ok = n0 + col < N;
        float* const sink = reinterpret_cast<float*>(a.ws + kWsSink) + 4 * (t & 63);
        const int row_w = m0 + eng.ep_row0();
        const int live = (!skip && n0 + eng.ep_col0() < N && row_w < rows_e)
                             ? min(Eng::FM, (int)cdiv(rows_e - row_w, 32))
                             : 0;
        // destinations of half h of block i (the token reads go out together)
        auto dests = [&](int i, int h, float* (&p)[H]) {
          int tok[H];
  #pragma unroll
          for (int u = 0; u < H; ++u) tok[u] = s_tok[eng.ep_row(i, h * H + u)];
  #pragma unroll
          for (int u = 0; u < H; ++u)
            p[u] = (tok[u] >= 0 && col_ok)
                       ? reinterpret_cast<float*>(a.out) + (int64_t)tok[u] * N + n0 + col
                       : sink;
        };
        if (live > 0) {
          float* p0[H];
          float* p1[H];
          dests(0, 0, p0);
          dests(0, 1, p1);
  #pragma unroll
          for (int u = 0; u < H; ++u) eng.ep_fetch(u, p0[u]);
  #pragma unroll
          for (int u = 0; u < H; ++u) eng.ep_fetch(H + u, p1[u]);
        }
  #pragma unroll
        for (int i = 0; i < Eng::FM; ++i) {
          if (i < live) {
            eng.ep_stage(i);
            const bool next = i + 1 < live;
  #pragma unroll
            for (int h = 0; h < 2; ++h) {
              // Wait for D(i) h.  Issued after it: block 0: D(0) h1 (h = 0);
              // D(1) h0 if any, S(0) h0 (h = 1).  Block i > 0: S(i-1) h0,
              // D(i) h1, S(i-1) h1 (h = 0); S(i-1) h1, D(i+1) h0 if any,
              // S(i) h0 (h = 1).
              if (i == 0 && h == 0) wait_vm_mem<H>();
              else if (h == 0) wait_vm_mem<3 * H>();
              else if (i == 0) { if (next) wait_vm_mem<2 * H>(); else wait_vm_mem<H>(); }
              else { if (next) wait_vm_mem<3 * H>(); else wait_vm_mem<2 * H>(); }
              f32x4 o[H];
  #pragma unroll
              for (int u = 0; u < H; ++u) {
                const int q = h * H + u;
                const f32x4 v = eng.ep_read(q);
                const float wt = s_wt[eng.ep_row(i, q)];
                o[u] = eng.ep_fetched(q);
                o[u][0] += wt * v[0];
                o[u][1] += wt * v[1];
                o[u][2] += wt * v[2];
                o[u][3] += wt * v[3];
              }
              float* pc[H];
              float* pn[H];
              dests(i, h, pc);
              if (next) dests(i + 1, h, pn);
              wait_lgkm_mem();   // these slots are read: block i+1 may land in them
              if (next) {
  #pragma unroll
                for (int u = 0; u < H; ++u) eng.ep_fetch(h * H + u, pn[u]);
              }
  #pragma unroll
              for (int u = 0; u < H; ++u) store_through(pc[u], o[u]);
            }
          }
        }
      }
      // The tile's flag goes out once every wave's stores have completed:
      // at the next tile's first K-step wait (which drains them while that
      // tile's first stage loads), or after the last tile.
      if (s_abort == 0) pending = (int)(gm * a.tiles_n + tn);
    } else {
      // H rows in expert-sorted order, 16-bit.
      const int col = eng.ep_col();
      const bool col_ok = n0 + col < N;
      // Blocks by compile-time index: with the activation's code the body
      // is too large for the unroller, and a runtime block index would move
      // the accumulators to scratch.
      static_for<Eng::FM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        eng.ep_stage(i);
#pragma unroll
        for (int q = 0; q < Eng::EP_READS; ++q) {
          const int lr = m0 + eng.ep_row(i, q);
          f32x4 v = eng.ep_read(q);
          if constexpr (ACT) {
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = apply_act(a.act, v[k]);
          }
          if (lr < rows_e && col_ok) {
            // non-temporal: H is not read again in this launch, and these
            // stores would otherwise push the operands out of L2 (layer 0
            // 0.636 against 0.644 ms at EP=8, the combine that reads H next
            // unchanged)
            const u32x2 pk = {E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
            __builtin_nontemporal_store(
                pk, reinterpret_cast<u32x2*>(a.out + ((int64_t)(row_base + lr) * N + n0 + col) * 2));
          }
        }
      });
    }
    eng.ep_end();
    if constexpr (SCATTER) {
      if (s_abort) break;
      if (t == 0) s_dup = 0;   // read by every thread before ep_end's barrier
      cq = s_next_q[it & 1];
      ct = s_next_t[it & 1];
      if (ct == -2) {
        // Every thread has read the slot before thread 0 refills it.
        __syncthreads();
        if (t == 0) {
          int q = 0;
          const int v = steal(q);
          s_next_q[it & 1] = q;
          s_next_t[it & 1] = v;
        }
        __syncthreads();
        cq = s_next_q[it & 1];
        ct = s_next_t[it & 1];
      }
    } else {
      L2 += G;
    }
  }
  if constexpr (SCATTER) {
    if (pending >= 0) {
      wait_vmcnt<0>();   // this wave's write-through stores are complete
      __syncthreads();
      publish();
    }
    // Every workgroup checks in once its tiles are done (or abandoned); the
    // last one resets the count and the queues' ticket counters (every
    // ticket fetch has returned by then) and stores this launch's epoch for
    // the next launch.  Relaxed: only the next launch reads these words, after the
    // kernel boundary (a release here would write back this XCD's L2 once
    // per workgroup).
    __syncthreads();
    if (t == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(a.ws + kCtlDone, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      if (prev == (uint32_t)G - 1) {
        __hip_atomic_store(a.ws + kCtlDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int q = 0; q < kMaxQueues; ++q)
          __hip_atomic_store(a.ws + kCtlQueue + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.ws + kCtlEpoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

namespace {

struct MoeTile {
  int bm, bn, nw;
};

// 256x256 tiles.  Layer 0 runs two waves per SIMD: on N(0,1) data 2% faster
// than one (0.649 vs 0.660 ms at EP=8).  The combine runs one wave per SIMD
// with the two-sub-step fragment read-ahead, which its DMA-fed epilogue
// leaves the registers for: 0.769 vs 0.775 ms.
MoeTile moe_tile(bool scatter) {
  const int nw_default = scatter ? 4 : 8;
  if (const char* env = std::getenv("FM_MOE_TILE")) {
    int bm = 0, bn = 0, nw = 0;
    const int got = std::sscanf(env, "%dx%dw%d", &bm, &bn, &nw);
    if (got >= 2 && (bm == 128 || bm == 256) && (bn == 128 || bn == 256)) {
      if (got < 3 || (nw != 4 && nw != 8)) nw = (bm == 256 && bn == 256) ? nw_default : 4;
      if (!(bm == 128 && bn == 128 && nw == 8)) return {bm, bn, nw};
    }
  }
  return {256, 256, nw_default};
}

// Producer workgroups for layer 0's own token copies: one per ~5 MiB, a
// multiple of 8 (one per XCD per round), 8..64.  The consumer tile count
// lives on the device, so unlike the dense operator the choice cannot count
// tile waves.  On the EP=8 workload (7 chunks of 16 MiB, ~5.5 waves of
// tiles, so every producer CU costs compute) 8/16/24/32/48/64 producers took
// 0.79/0.70/0.69/0.74/0.74/0.80 ms (non-fused layer 0: 0.65 ms).
int moe_producers_default(int64_t bytes) {
  if (const char* env = std::getenv("FM_PRODUCERS")) {
    const int p = std::atoi(env);
    if (p >= 8 && p <= device_cu_count() / 2 && p % 8 == 0) return p;
  }
  const int64_t p = (cdiv(bytes, 5ll << 20) + 7) / 8 * 8;
  return (int)std::min<int64_t>(64, std::max<int64_t>(8, p));
}

// M-tiles per band of the token-AllGather order.  At the EP=8 shape two
// 256-row tiles of one expert span about a quarter of a 2048-token chunk, so
// the first waves need only the earliest chunks.  Measured with copy-engine
// arrival (all chunks in ~0.3 ms): ECT 0.11 ms with bands of 2, 0.16 ms with
// whole experts; with kernel copies (~0.13 ms) the band size hardly matters.
int moe_ag_group() {
  if (const char* env = std::getenv("FM_MOE_AG_GROUP")) {
    const int g = std::atoi(env);
    if (g >= 1 && g <= 16) return g;
  }
  return 2;
}

template <bool SCATTER, bool PULL = false, bool ACT = false, bool VEP = false>
void launch_moe_part(fm_dtype_t dt, MoeTile cfg, const MoeArgs& a, hipStream_t stream);

// Layer 0 splits a half-empty last wave into 256x128 halves (part 1, a second
// launch; it finds no work when the device-side tile count needs no split).
// The combine (layer 1) keeps whole tiles: its per-column ordering counts
// one tile per column and M-tile.
template <bool SCATTER>
fm_status_t launch_moe(fm_dtype_t dt, MoeTile cfg, MoeArgs& a, hipStream_t stream) {
  a.tiles_n = (int)cdiv(a.N, cfg.bn);
  a.group_m = 8;
  a.g_ref = device_cu_count();
  const char* env = std::getenv("FM_SPLIT_TAIL");
  // (no split with producer workgroups: producers and consumers share one launch)
  a.split = (!SCATTER && cfg.bm == 256 && cfg.bn == 256 && !(env && env[0] == '0') &&
             a.prod.n_prod == 0)
                ? 1
                : 0;
  a.part = 0;
  auto launch_part = [&](MoeTile c) {
    if constexpr (SCATTER) {
      if (a.out_records) launch_moe_part<true, false, false, true>(dt, c, a, stream);
      else launch_moe_part<true>(dt, c, a, stream);
    } else {
      if (a.pull_src[0]) launch_moe_part<false, true>(dt, c, a, stream);
      else if (a.act != FM_ACT_NONE) launch_moe_part<false, false, true>(dt, c, a, stream);
      else launch_moe_part<false>(dt, c, a, stream);
    }
  };
  launch_part(cfg);
  if (a.split) {
    a.part = 1;
    launch_part(MoeTile{256, 128, 4});
  }
  return launch_status();
}

// Grid of the combine: one workgroup per CU.  Its tiles are handed out by
// ticket, so any grid size is correct; FM_COMBINE_GRID (1..4096) overrides the
// size, which the tests use to run more workgroups than can be resident.
int combine_grid() {
  if (const char* env = std::getenv("FM_COMBINE_GRID")) {
    const int g = std::atoi(env);
    if (g >= 1 && g <= 4096) return g;
  }
  return device_cu_count();
}

template <bool SCATTER, bool PULL, bool ACT, bool VEP>
void launch_moe_part(fm_dtype_t dt, MoeTile cfg, const MoeArgs& a, hipStream_t stream) {
  const dim3 grid(SCATTER ? combine_grid() : device_cu_count());
#define FM_LAUNCH(E, BM, BN, NW)                                                              \
  do {                                                                                        \
    if (a.K % kBK) /* ragged K: the 4-wave, LDS-DMA forms keep the tail path spill-free */    \
      hipLaunchKernelGGL((moe_kernel<E, BM, BN, 4, SCATTER, true, PULL, ACT, false>), grid,   \
                         dim3(256), 0, stream, a);                                            \
    else                                                                                      \
      hipLaunchKernelGGL((moe_kernel<E, BM, BN, NW, SCATTER, false, PULL, ACT, VEP>), grid,   \
                         dim3(64 * NW), 0, stream, a);                                        \
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
}

fm_status_t check_route_args(int64_t T, int32_t topk, int32_t n_local, const int32_t* topk_ids,
                             const int32_t* sorted_pairs, const int32_t* expert_offsets,
                             const void* ws, size_t ws_bytes) {
  if (T < 0 || topk < 1 || n_local < 1 || n_local > kMaxLocalExperts) return FM_ERR_INVALID_ARG;
  if (T * topk >= (1ll << 31)) return FM_ERR_UNSUPPORTED;
  if (!expert_offsets || (T > 0 && (!topk_ids || !sorted_pairs))) return FM_ERR_INVALID_ARG;
  if (!ws || !aligned16(ws) || ws_bytes < (size_t)(kWsRoute + kRouteWords) * 4)
    return FM_ERR_INVALID_ARG;
  return FM_OK;
}

}  // namespace
}  // namespace fm

using namespace fm;

extern "C" size_t fm_moe_workspace_bytes(int64_t T, int32_t topk, int64_t hidden,
                                         int32_t n_local) {
  if (T < 0 || topk < 1 || hidden < 0 || n_local < 1 || n_local > kMaxLocalExperts) return 0;
  return moe_ws_bytes(T * topk, hidden, n_local);
}

extern "C" fm_status_t fm_moe_route(int64_t T, int32_t topk, int32_t expert_begin,
                                    int32_t n_local, const int32_t* topk_ids,
                                    int32_t* sorted_pairs, int32_t* expert_offsets, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  const fm_status_t st = check_route_args(T, topk, n_local, topk_ids, sorted_pairs,
                                          expert_offsets, ws, ws_bytes);
  if (st != FM_OK) return st;
  const int64_t P = T * topk;
  const int64_t ch = route_chunk_pairs(P, n_local);
  const int n_chunks = (int)std::max<int64_t>(1, cdiv(P, ch));
  uint32_t* counts = static_cast<uint32_t*>(ws) + kWsRoute;
  hipLaunchKernelGGL(route_count_kernel, dim3(n_chunks), dim3(kRouteThreads), 0, stream,
                     topk_ids, P, (int)expert_begin, (int)n_local, ch, counts);
  hipLaunchKernelGGL(route_place_kernel, dim3(n_chunks), dim3(kRouteThreads), 0, stream,
                     topk_ids, P, (int)expert_begin, (int)n_local, ch, n_chunks,
                     (const uint32_t*)counts, sorted_pairs, expert_offsets);
  return launch_status();
}

namespace fm {
namespace {

fm_status_t moe_gather_impl(fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn, int32_t topk,
                            int32_t expert_begin, int32_t n_local, const void* X,
                            const int32_t* topk_ids, const void* W1, void* H,
                            int32_t* sorted_pairs, int32_t* expert_offsets, int32_t n_chunks,
                            const uint32_t* flags, uint32_t epoch, const int32_t* order,
                            int32_t* err_word, int64_t spin_limit, void* ws, size_t ws_bytes,
                            hipStream_t stream,
                            const void* const* src = nullptr, uint32_t* counters = nullptr,
                            int32_t n_producers = 0, const void* const* pull = nullptr,
                            int act = FM_ACT_NONE) {
  if (dt != FM_F16 && dt != FM_BF16) return FM_ERR_UNSUPPORTED;
  fm_status_t st = check_route_args(T, topk, n_local, topk_ids, sorted_pairs, expert_offsets,
                                    ws, ws_bytes);
  if (st != FM_OK) return st;
  if (hidden < 0 || ffn < 0 || hidden % 8 || ffn % 8) return FM_ERR_INVALID_ARG;
  // pull mode reads the chunks in place: no gathered X.  With hidden = 0 the
  // sum over K is empty (H = act(0) on the local rows): X and W1 may be null.
  if (T > 0 && ffn > 0 &&
      (!H || !aligned16(H) ||
       (hidden > 0 && ((!pull && (!X || !aligned16(X))) || !W1 || !aligned16(W1)))))
    return FM_ERR_INVALID_ARG;
  if (pull) {
    if (!flags || n_chunks < 1 || n_chunks > 64) return FM_ERR_INVALID_ARG;
    for (int c = 0; c < n_chunks; ++c)
      if (hidden > 0 && (!pull[c] || !aligned16(pull[c]))) return FM_ERR_INVALID_ARG;
  }
  uint8_t pos[64] = {};
  if (flags) {
    if (n_chunks < 1 || n_chunks > 64 || T % n_chunks || spin_limit < 0 ||
        (reinterpret_cast<uintptr_t>(flags) & 3u))
      return FM_ERR_INVALID_ARG;
    bool seen[64] = {};
    for (int i = 0; i < n_chunks; ++i) {
      const int c = order ? order[i] : i;
      if (c < 0 || c >= n_chunks || seen[c]) return FM_ERR_INVALID_ARG;
      seen[c] = true;
      pos[c] = (uint8_t)i;
    }
  }
  // Producer workgroups: sources must be aligned and lie outside X.
  const int64_t chunk_bytes = flags ? (T / n_chunks) * hidden * 2 : 0;
  if (src) {
    if (!counters || (reinterpret_cast<uintptr_t>(counters) & 3u)) return FM_ERR_INVALID_ARG;
    if (n_producers != 0 && (n_producers < 8 || n_producers % 8 ||
                             n_producers > device_cu_count() / 2))
      return FM_ERR_INVALID_ARG;
    const char* xb = (const char*)X;
    for (int c = 0; c < n_chunks; ++c) {
      const char* sc = (const char*)src[c];
      if (!sc) continue;
      if (!aligned16(sc)) return FM_ERR_INVALID_ARG;
      if (xb && sc < xb + T * hidden * 2 && xb < sc + chunk_bytes) return FM_ERR_INVALID_ARG;
    }
  }
  // gathered-row byte offsets are 32-bit
  if (hidden >= (1ll << 22) || ffn >= (1ll << 22) || T * hidden >= (1ll << 31))
    return FM_ERR_UNSUPPORTED;
  st = fm_moe_route(T, topk, expert_begin, n_local, topk_ids, sorted_pairs, expert_offsets, ws,
                    ws_bytes, stream);
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
  a.rows_cap = T * topk;
  a.n_local = n_local;
  if (flags) {
    a.flags = flags;
    a.chunk_epoch = epoch;
    a.chunk_tokens = T / n_chunks;
    a.err_word = err_word;
    a.chunk_spin = spin_limit ? spin_limit : (1ll << 24);
    std::memcpy(a.chunk_pos, pos, sizeof(pos));
  }
  if (pull)
    for (int c = 0; c < n_chunks; ++c) a.pull_src[c] = (const char*)pull[c];
  if (src) {
    const int P = n_producers ? n_producers : moe_producers_default(chunk_bytes * n_chunks);
    fill_producers(a.prod, P, n_chunks, chunk_bytes, src, order, const_cast<void*>(X),
                   const_cast<uint32_t*>(flags), counters, epoch);
  }
  a.ag_group = moe_ag_group();
  a.act = act;
  return launch_moe<false>(dt, moe_tile(false), a, stream);
}

}  // namespace
}  // namespace fm

extern "C" fm_status_t fm_moe_gather_gemm(fm_dtype_t dt, int64_t T, int64_t hidden,
                                          int64_t ffn, int32_t topk, int32_t expert_begin,
                                          int32_t n_local, const void* X,
                                          const int32_t* topk_ids, const void* W1, void* H,
                                          int32_t* sorted_pairs, int32_t* expert_offsets,
                                          void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_gather_impl(dt, T, hidden, ffn, topk, expert_begin, n_local, X, topk_ids, W1, H,
                         sorted_pairs, expert_offsets, 0, nullptr, 0, nullptr, nullptr, 0, ws,
                         ws_bytes, stream);
}

extern "C" fm_status_t fm_moe_gather_gemm_act(fm_dtype_t dt, int64_t T, int64_t hidden,
                                              int64_t ffn, int32_t topk, int32_t expert_begin,
                                              int32_t n_local, const void* X,
                                              const int32_t* topk_ids, const void* W1, void* H,
                                              int32_t* sorted_pairs, int32_t* expert_offsets,
                                              fm_act_t act, void* ws, size_t ws_bytes,
                                              hipStream_t stream) {
  if ((int)act < FM_ACT_NONE || (int)act > FM_ACT_SILU) return FM_ERR_INVALID_ARG;
  return moe_gather_impl(dt, T, hidden, ffn, topk, expert_begin, n_local, X, topk_ids, W1, H,
                         sorted_pairs, expert_offsets, 0, nullptr, 0, nullptr, nullptr, 0, ws,
                         ws_bytes, stream, nullptr, nullptr, 0, nullptr, (int)act);
}

extern "C" fm_status_t fm_moe_ag_gather_gemm(fm_dtype_t dt, int64_t T, int64_t hidden,
                                             int64_t ffn, int32_t topk, int32_t expert_begin,
                                             int32_t n_local, const void* X,
                                             const int32_t* topk_ids, const void* W1, void* H,
                                             int32_t* sorted_pairs, int32_t* expert_offsets,
                                             int32_t n_chunks, const uint32_t* flags,
                                             uint32_t epoch, const int32_t* order,
                                             int32_t* err_word, int64_t spin_limit, void* ws,
                                             size_t ws_bytes, hipStream_t stream) {
  if (!flags) return FM_ERR_INVALID_ARG;
  return moe_gather_impl(dt, T, hidden, ffn, topk, expert_begin, n_local, X, topk_ids, W1, H,
                         sorted_pairs, expert_offsets, n_chunks, flags, epoch, order, err_word,
                         spin_limit, ws, ws_bytes, stream);
}

extern "C" fm_status_t fm_moe_ag_gather_gemm_producers(
    fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn, int32_t topk, int32_t expert_begin,
    int32_t n_local, void* X, const int32_t* topk_ids, const void* W1, void* H,
    int32_t* sorted_pairs, int32_t* expert_offsets, int32_t n_chunks, const void* const* src,
    uint32_t* flags, uint32_t* counters, uint32_t epoch, const int32_t* order,
    int32_t n_producers, int32_t* err_word, int64_t spin_limit, void* ws, size_t ws_bytes,
    hipStream_t stream) {
  if (!flags || !src) return FM_ERR_INVALID_ARG;
  return moe_gather_impl(dt, T, hidden, ffn, topk, expert_begin, n_local, X, topk_ids, W1, H,
                         sorted_pairs, expert_offsets, n_chunks, flags, epoch, order, err_word,
                         spin_limit, ws, ws_bytes, stream, src, counters, n_producers);
}

extern "C" fm_status_t fm_moe_ag_gather_gemm_pull(
    fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn, int32_t topk, int32_t expert_begin,
    int32_t n_local, const void* const* chunks, const int32_t* topk_ids, const void* W1, void* H,
    int32_t* sorted_pairs, int32_t* expert_offsets, int32_t n_chunks, const uint32_t* flags,
    uint32_t epoch, const int32_t* order, int32_t* err_word, int64_t spin_limit, void* ws,
    size_t ws_bytes, hipStream_t stream) {
  if (!flags || !chunks) return FM_ERR_INVALID_ARG;
  return moe_gather_impl(dt, T, hidden, ffn, topk, expert_begin, n_local, nullptr, topk_ids, W1,
                         H, sorted_pairs, expert_offsets, n_chunks, flags, epoch, order,
                         err_word, spin_limit, ws, ws_bytes, stream, nullptr, nullptr, 0, chunks);
}

namespace fm {
namespace {

// ---------------------------------------------------------------------------
// Scratch of fm_moe_gemm_scatter_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Layout as the workspace's control
// words and sink ([0, 320)), then the completion flags.  Host code never uses
// the array's name as an address: the per-device address comes from
// hipGetSymbolAddress.
// ---------------------------------------------------------------------------
constexpr int64_t kNoAllocWords = 65536;                 // 256 KiB
constexpr int64_t kNoAllocFlags0 = kWsRoute;             // flags follow the sink
static __device__ __align__(256) uint32_t scratch[kNoAllocWords];

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// The device address of this device's `scratch`, looked up (and the array
// zero-filled on `stream`, by a kernel) on the first call on each device;
// nullptr if the lookup fails.
uint32_t* noalloc_scratch(hipStream_t stream) {
  static std::mutex mu;
  static uint32_t* addr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(64), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), kNoAllocWords);
    if (hipGetLastError() != hipSuccess) return nullptr;
    addr[dev] = static_cast<uint32_t*>(p);
  }
  return addr[dev];
}

// Arguments of the combine, shared by both entry points.
fm_status_t check_combine_args(fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn,
                               int32_t topk, int32_t n_local, const void* H, const void* W2,
                               const int32_t* sorted_pairs, const int32_t* expert_offsets,
                               const float* topk_weights, float* out, int64_t spin_limit) {
  if (dt != FM_F16 && dt != FM_BF16) return FM_ERR_UNSUPPORTED;
  if (T < 0 || topk < 1 || n_local < 1 || n_local > kMaxLocalExperts) return FM_ERR_INVALID_ARG;
  if (hidden < 0 || ffn < 0 || hidden % 8 || ffn % 8 || spin_limit < 0) return FM_ERR_INVALID_ARG;
  if (!expert_offsets) return FM_ERR_INVALID_ARG;
  if (T == 0 || hidden == 0) return FM_OK;
  // With ffn = 0 the sum over K is empty (each local pair adds weight x 0):
  // H and W2 may be null.
  if ((ffn > 0 && (!H || !W2 || !aligned16(H) || !aligned16(W2))) || !sorted_pairs ||
      !topk_weights || !out || !aligned16(out))
    return FM_ERR_INVALID_ARG;
  if (hidden >= (1ll << 22) || ffn >= (1ll << 22) || T * topk * ffn >= (1ll << 31))
    return FM_ERR_UNSUPPORTED;
  return FM_OK;
}

fm_status_t launch_combine(fm_dtype_t dt, int64_t T, int64_t hidden, int64_t ffn, int32_t topk,
                           int32_t n_local, const void* H, const void* W2,
                           const int32_t* sorted_pairs, const int32_t* expert_offsets,
                           const float* topk_weights, float* out, int32_t* err_word,
                           int64_t spin_limit, uint32_t* ctl, uint32_t* flags,
                           hipStream_t stream) {
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
  a.rows_cap = T * topk;
  a.n_local = n_local;
  a.ws = ctl;
  a.tile_done = flags;   // sized for the smallest tile
  a.err_word = err_word;
  a.spin_limit = spin_limit ? spin_limit : (1ll << 24);
  // The register-fetch epilogue addresses out through a buffer resource
  // (32-bit offsets, out below 2 GiB); FM_COMBINE_DMA=1 selects the LDS-DMA
  // form for any size.
  const int64_t out_bytes = T * hidden * 4;
  const char* env = std::getenv("FM_COMBINE_DMA");
  a.out_records = (out_bytes <= (int64_t)kVepMaxRecords && !(env && env[0] == '1'))
                      ? (uint32_t)out_bytes
                      : 0u;
  return launch_moe<true>(dt, moe_tile(true), a, stream);
}

}  // namespace
}  // namespace fm

extern "C" fm_status_t fm_moe_gemm_scatter_noalloc(fm_dtype_t dt, int64_t T, int64_t hidden,
                                                   int64_t ffn, int32_t topk, int32_t n_local,
                                                   const void* H, const void* W2,
                                                   const int32_t* sorted_pairs,
                                                   const int32_t* expert_offsets,
                                                   const float* topk_weights, float* out,
                                                   int32_t* err_word, int64_t spin_limit,
                                                   hipStream_t stream) {
  const fm_status_t st = check_combine_args(dt, T, hidden, ffn, topk, n_local, H, W2,
                                            sorted_pairs, expert_offsets, topk_weights, out,
                                            spin_limit);
  if (st != FM_OK || T == 0 || hidden == 0) return st;
  if (kNoAllocFlags0 + combine_flag_words(T * topk, hidden, n_local) > kNoAllocWords)
    return FM_ERR_UNSUPPORTED;
  uint32_t* ctl = noalloc_scratch(stream);
  if (!ctl) return FM_ERR_HIP;
  return launch_combine(dt, T, hidden, ffn, topk, n_local, H, W2, sorted_pairs, expert_offsets,
                        topk_weights, out, err_word, spin_limit, ctl, ctl + kNoAllocFlags0,
                        stream);
}

extern "C" fm_status_t fm_moe_gemm_scatter(fm_dtype_t dt, int64_t T, int64_t hidden,
                                           int64_t ffn, int32_t topk, int32_t n_local,
                                           const void* H, const void* W2,
                                           const int32_t* sorted_pairs,
                                           const int32_t* expert_offsets,
                                           const float* topk_weights, float* out,
                                           int32_t* err_word, int64_t spin_limit, void* ws,
                                           size_t ws_bytes, hipStream_t stream) {
  const fm_status_t st = check_combine_args(dt, T, hidden, ffn, topk, n_local, H, W2,
                                            sorted_pairs, expert_offsets, topk_weights, out,
                                            spin_limit);
  if (st != FM_OK) return st;
  if (!ws || !aligned16(ws) || ws_bytes < moe_ws_bytes(T * topk, hidden, n_local))
    return FM_ERR_INVALID_ARG;
  if (T == 0 || hidden == 0) return FM_OK;
  uint32_t* w = static_cast<uint32_t*>(ws);
  return launch_combine(dt, T, hidden, ffn, topk, n_local, H, W2, sorted_pairs, expert_offsets,
                        topk_weights, out, err_word, spin_limit, w, w + kWsFlags, stream);
}
