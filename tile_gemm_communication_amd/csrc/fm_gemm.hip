// fm_gemm.hip -- dense persistent GEMM kernels and their C-ABI entry points:
// plain GEMM, AllGather-GEMM (chunk-flag waits in the tile prologue) and
// GEMM-ReduceScatter (fp32 add into per-rank row slices in the epilogue).
//
// FLUX review, section 三: "细粒度分解" / "内核融合" / "瓦片映射" -- communication
// and computation are split into tiles, fused into one kernel, and each
// dependent compute tile is bound to a thread block (here: a workgroup of a
// persistent grid).  "AllGather 重叠" and "ReduceScatter 重叠" describe the two
// fused forms implemented below.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "fm_sched.hpp"
#include "fm_tile.hpp"

namespace fm {

// RS: ReduceScatter epilogue for tiles that never straddle a slice (slice
// rows a multiple of BM) with plain adds; RSG: any slice size, or atomic adds.
// AGP: AllGather in pull mode, each chunk read in place from its own buffer.
// AGX: AllGather with its own producer workgroups (the first n_prod of the
// grid copy the chunks into X and publish them; the rest run AG tiles).
enum class Mode : int { Gemm = 0, AG = 1, RS = 2, RSG = 3, AGP = 4, AGX = 5 };

constexpr int kMaxRanks = 16;
// Dense kernels with one wave per SIMD may use the 16x16x32 MFMA form (the
// engine's MF16 path).  It passes every parity test but measured no faster
// than 32x32x16 here (AG shape 0.51 vs 0.50 ms, GEMM-RS 0.54 vs 0.53 ms), so
// it is off; the compile-time switch keeps it for later tuning.
#ifndef FM_MFMA16
#define FM_MFMA16 0
#endif
constexpr bool kMfma16 = FM_MFMA16 != 0;
// In-tile byte offsets are 32-bit (tile rows x row pitch), which bounds each
// dimension to 2^22 elements.
constexpr int64_t kMaxDim = 1ll << 22;
constexpr int kMaxChunks = 64;

struct DenseArgs {
  const char* A;
  const char* B;
  char* C;
  int64_t M, N, K;
  // AllGather: chunk flags
  const uint32_t* flags;
  int32_t* err_word;
  int64_t chunk_rows;
  int64_t spin_limit;
  uint32_t epoch;
  // AllGather, pull mode: chunk c's rows live at chunk_a[c]; M-tile tm is
  // tile tm % tiles_per_chunk of chunk tm / tiles_per_chunk, so no tile
  // straddles two buffers (a ragged chunk ends in a partial tile).
  int tiles_per_chunk;
  const char* chunk_a[kMaxChunks];
  // AllGather with producer workgroups (AGX): the first prod.n_prod
  // workgroups copy the chunks into X.
  ProducerArgs prod;
  // ReduceScatter: destination slices
  int32_t atomic;
  int64_t slice_rows;
  float* dst[kMaxRanks];
  TileOrder order;
  // This launch covers schedule positions [pos0, pos_end) of `order`, each
  // split into sub_n tiles of BN columns (order's tiles are sub_n * BN wide).
  int pos0, pos_end, sub_n;
};

// Store a run of 4 consecutive outputs at element index idx of C.
template <class E, bool OUT32>
__device__ __forceinline__ void store_run(char* C, int64_t idx, const f32x4& v) {
  if constexpr (OUT32) {
    *reinterpret_cast<f32x4*>(C + idx * 4) = v;
  } else {
    const u32x2 p = {E::pack2(v[0], v[1]), E::pack2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(C + idx * 2) = p;
  }
}

// Point the engine's DMA at the `rows` A rows starting at a_tile (the tile's
// first row; rows past the last are clamped to it) and the B columns
// [n0, n0+BN) of one tile.
template <class Eng>
__device__ __forceinline__ void setup_operands(Eng& eng, const DenseArgs& args,
                                               const char* a_tile, int rows, int64_t n0) {
  const int64_t N = args.N, K = args.K;
  eng.set_a_base(a_tile);
#pragma unroll
  for (int i = 0; i < Eng::A_DMA; ++i) {
    const int row = min(eng.a_dma_row(i), rows - 1);
    eng.set_a(i, (uint32_t)(row * K * 2));
  }
  eng.set_b(args.B, N * 2, n0, N);
}

// Store epilogue (between ep_begin and ep_end): round to 16 bits (or keep
// fp32) and store runs of 4 columns, a wave covering whole rows per access.
template <class E, bool OUT32, class Eng>
__device__ __forceinline__ void store_tile(Eng& eng, const DenseArgs& args, int64_t m0,
                                           int64_t m_end, int64_t n0) {
  const int64_t N = args.N;
  const int col = eng.ep_col();
  const bool col_ok = n0 + col < N;
  constexpr int EB = OUT32 ? 4 : 2;
  char* base = args.C + (m0 * N + n0) * EB;
  const int lim = col_ok ? (int)(m_end - m0) - eng.ep_row(0, 0) : 0;
#pragma unroll
  for (int i = 0; i < Eng::FM; ++i) {
    eng.ep_stage(i);
    char* p0 = base + (uint32_t)(eng.ep_row(i, 0) * (int)N + col) * EB;
#pragma unroll
    for (int q = 0; q < Eng::EP_READS; ++q) {
      const f32x4 v = eng.ep_read(q);
      if (i * 32 + q * Eng::EP_RPI < lim)
        store_run<E, OUT32>(p0 + (uint32_t)(q * Eng::EP_RPI * (int)N * EB), 0, v);
    }
  }
}

template <class E, int BM, int BN, int NW, Mode MODE, bool OUT32, bool KTAIL>
__global__ __launch_bounds__(64 * NW, 1) void dense_kernel(const DenseArgs args) {
  // One wave per SIMD has the register room for a two-sub-step read-ahead,
  // or for the 16x16x32 MFMA form.
  // 256x128 and 128x128 tiles keep three LDS stages in flight (their K steps
  // are short); 256x256 tiles have room for two.
  using Eng = Engine<E, BM, BN, KTAIL, NW, 4, NW == 4 ? 2 : 1, kMfma16 && NW == 4 && !KTAIL, false,
                     BN == 128 ? 3 : 2>;
  // The ReduceScatter epilogue of full tiles keeps its destination rows in
  // LDS (the one-wave-per-SIMD form: with two, its registers would spill).
  constexpr bool kRsDma = MODE == Mode::RS && NW == 4;
  constexpr int kSmem =
      (kRsDma && Eng::EP_RMW_LDS > Eng::LDS_BYTES) ? Eng::EP_RMW_LDS : Eng::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ int s_abort;

  int wg = blockIdx.x, G = gridDim.x;
  if constexpr (MODE == Mode::AGX) {
    // The producers take the first workgroup ids, so they are dispatched
    // before any consumer that may wait on them.
    if (wg < args.prod.n_prod) {
      produce_chunks<64 * NW>(args.prod);
      return;
    }
    wg -= args.prod.n_prod;
    G -= args.prod.n_prod;
  }
  Eng eng(smem, args.K);
  const int64_t M = args.M, N = args.N, K = args.K;
  const int slot = xcd_slot(wg, G);
  uint64_t ready = 0;

  const int n_pos = (args.pos_end - args.pos0) * args.sub_n;
  for (int L = slot; L < n_pos; L += G) {
    const int P = args.pos0 + L / args.sub_n, sub = L % args.sub_n;
    int tm_pos, tn;
    band_coords(P, args.order.tiles_m, args.order.tiles_n, args.order.group_m, tm_pos, tn);
    // uniform, but a table lookup is not always seen as such: the A base
    // derived from it must sit in scalar registers for the DMA
    const int tm = __builtin_amdgcn_readfirstlane(
        args.order.has_morder ? (int)args.order.morder[tm_pos] : tm_pos);
    const int64_t n0 = ((int64_t)tn * args.sub_n + sub) * BN;
    int64_t m0, m_end;       // output rows of the tile
    const char* a_tile;      // its first A row
    if constexpr (MODE == Mode::AGP) {
      const int c = tm / args.tiles_per_chunk;
      const int64_t r0 = (int64_t)(tm - c * args.tiles_per_chunk) * BM;
      m0 = c * args.chunk_rows + r0;
      m_end = c * args.chunk_rows + min(r0 + BM, args.chunk_rows);
      // The chunk index is uniform, but the table lookup is not seen as such:
      // the DMA base must sit in scalar registers.  readfirstlane yields a
      // signed int, so each half goes through uint32_t before widening (a
      // sign-extended low half would corrupt the upper address bits).
      const uint64_t pa = (uint64_t)(uintptr_t)(args.chunk_a[c] + r0 * K * 2);
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)pa);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(pa >> 32));
      a_tile = (const char*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
    } else {
      m0 = (int64_t)tm * BM;
      m_end = min(m0 + BM, M);
      a_tile = args.A + m0 * K * 2;
    }
    if (n0 >= N) continue;   // a part of an edge tile that lies past N

    if constexpr (MODE == Mode::AG || MODE == Mode::AGP || MODE == Mode::AGX) {
      // Tile prologue: wait for every chunk overlapping rows [m0, m_end).
      if (threadIdx.x == 0) {
        const bool ok = wait_chunks(args.flags, args.epoch, (int)(m0 / args.chunk_rows),
                                    (int)((m_end - 1) / args.chunk_rows), ready,
                                    args.spin_limit, args.err_word);
        s_abort = ok ? 0 : 1;
      }
      __syncthreads();
      const int abort_now = s_abort;
      __syncthreads();
      if (abort_now) return;
    }

    setup_operands(eng, args, a_tile, (int)(m_end - m0), n0);
    eng.run();

    // Epilogue through the LDS staging regions: each global access of a wave
    // covers Eng::EP_RPI whole rows of its sub-tile.
    eng.ep_begin();
    const int col = eng.ep_col();
    const bool col_ok = n0 + col < N;
    if constexpr (MODE == Mode::RS || MODE == Mode::RSG) {
      // Add the fp32 partial into the owning rank's row slice.
      const int64_t Ms = args.slice_rows;
      const int s_lo = (int)(m0 / Ms), s_hi = (int)((m_end - 1) / Ms);
      float* const base = args.dst[s_lo] + (m0 - (int64_t)s_lo * Ms) * N + n0;
      // Element offset of this lane's first value; the empty asm makes it
      // opaque per tile, so that the addresses derived from it are formed
      // here rather than hoisted out of the tile loop, where they would stay
      // live through the K loop.
      int lane_off = eng.ep_row(0, 0) * (int)N + col;
      asm volatile("" : "+v"(lane_off));
      if constexpr (MODE == Mode::RS) {
        if (kRsDma && m_end - m0 == BM && n0 + BN <= N) {
          // A full tile in one slice: the slice rows come into LDS by DMA
          // (non-temporal: each is read once), block i+1's before block
          // i's stores (vmcnt counts loads and stores in issue order, so
          // loads issued after a store would wait for it), each block in
          // two halves of H reads.  Every lane is valid, so each
          // half issues exactly H loads and H stores and the waits count them.
          // Issue order: D(0) h0, D(0) h1, then per half h of block i:
          // D(i+1) h, S(i) h.
          constexpr int H = Eng::EP_READS / 2;
          auto at = [&](int i, int q) {
            return base + (uint32_t)(lane_off + (32 * i + q * Eng::EP_RPI) * (int)N);
          };
#pragma unroll
          for (int q = 0; q < Eng::EP_READS; ++q) eng.ep_fetch_once(q, at(0, q));
#pragma unroll
          for (int i = 0; i < Eng::FM; ++i) {
            eng.ep_stage(i);
            const bool next = i + 1 < Eng::FM;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              // Wait for D(i) h.  Issued after it: block 0: D(0) h1 (h = 0);
              // D(1) h0, S(0) h0 (h = 1).  Block i > 0: S(i-1) h0, D(i) h1,
              // S(i-1) h1 (h = 0); S(i-1) h1, D(i+1) h0 if any, S(i) h0 (h = 1).
              if (i == 0 && h == 0) wait_vm_mem<H>();
              else if (h == 0) wait_vm_mem<3 * H>();
              else if (i == 0) { if (next) wait_vm_mem<2 * H>(); else wait_vm_mem<H>(); }
              else { if (next) wait_vm_mem<3 * H>(); else wait_vm_mem<2 * H>(); }
              f32x4 o[H];
#pragma unroll
              for (int u = 0; u < H; ++u)
                o[u] = eng.ep_fetched(h * H + u) + eng.ep_read(h * H + u);
              wait_lgkm_mem();   // these slots are read: block i+1 may land in them
              if (next) {
#pragma unroll
                for (int u = 0; u < H; ++u) eng.ep_fetch_once(h * H + u, at(i + 1, h * H + u));
              }
#pragma unroll
              for (int u = 0; u < H; ++u)
                __builtin_nontemporal_store(o[u], reinterpret_cast<f32x4*>(at(i, h * H + u)));
            }
          }
        } else {
          // An edge tile in one slice.  Uniform base, 32-bit lane offsets
          // (row < BM, N < 2^22), the loads of half a block in flight first.
          // rows of block i, run q are valid while i*32 + q*EP_RPI < lim
          const int lim = col_ok ? (int)(m_end - m0) - eng.ep_row(0, 0) : 0;
          // at most 8 slice loads in flight per lane (32 VGPRs): the 4-wave
          // tile has 16 per block, which would crowd out the loop state
          constexpr int QH = Eng::EP_READS > 8 ? 8 : Eng::EP_READS;
#pragma unroll
          for (int i = 0; i < Eng::FM; ++i) {
            float* p0 = base + (uint32_t)(eng.ep_row(i, 0) * (int)N + col);
#pragma unroll
            for (int q0 = 0; q0 < Eng::EP_READS; q0 += QH) {
              // the slice rows are requested first; the accumulators are
              // staged while the first loads fly
              f32x4 old[QH];
#pragma unroll
              for (int q = q0; q < q0 + QH; ++q)
                if (i * 32 + q * Eng::EP_RPI < lim)
                  old[q - q0] =
                      *reinterpret_cast<const f32x4*>(p0 + (uint32_t)(q * Eng::EP_RPI * (int)N));
              if (q0 == 0) eng.ep_stage(i);
#pragma unroll
              for (int q = q0; q < q0 + QH; ++q) {
                const f32x4 v = eng.ep_read(q);
                if (i * 32 + q * Eng::EP_RPI < lim)
                  *reinterpret_cast<f32x4*>(p0 + (uint32_t)(q * Eng::EP_RPI * (int)N)) =
                      old[q - q0] + v;
              }
            }
          }
        }
      } else {
        (void)s_hi;
        // A tile across slices, or atomic accumulation: slice by slice (a
        // uniform loop, so each destination base stays scalar), one run at a
        // time.
        const int row_l = eng.ep_row(0, 0);
#pragma unroll
        for (int i = 0; i < Eng::FM; ++i) {
          eng.ep_stage(i);
          for (int s = s_lo; s <= s_hi; ++s) {
            const int64_t r0 = (int64_t)s * Ms;
            // tile-relative row range of slice s, shifted to this lane's rows
            const int lo = (int)(max(r0, m0) - m0) - row_l - i * 32;
            const int hi = (int)(min(r0 + Ms, m_end) - m0) - row_l - i * 32;
            const int64_t off = (m0 - r0 + row_l + i * 32) * N + n0 + col;
#pragma unroll 1
            for (int q = 0; q < Eng::EP_READS; ++q) {
              const int rq = q * Eng::EP_RPI;
              if (!col_ok || rq < lo || rq >= hi) continue;
              float* d = args.dst[s] + off + (int64_t)rq * N;
              const f32x4 v = eng.ep_read(q);
              if (args.atomic) {
                unsafeAtomicAdd(d + 0, v[0]);
                unsafeAtomicAdd(d + 1, v[1]);
                unsafeAtomicAdd(d + 2, v[2]);
                unsafeAtomicAdd(d + 3, v[3]);
              } else {
                *reinterpret_cast<f32x4*>(d) = *reinterpret_cast<const f32x4*>(d) + v;
              }
            }
          }
        }
      }
    } else {
      store_tile<E, OUT32>(eng, args, m0, m_end, n0);
    }
    eng.ep_end();
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {

struct TileCfg {
  int bm, bn, nw;
};

// Tile shape for an M x N output on G CUs: the fewest full-machine waves of
// work, weighting smaller tiles by their lower MFMA:load ratio.
// A last partial wave of at most G/2 256x256 tiles runs as twice as many
// 256x128 tiles (one wave of half-size tiles instead of a half-empty wave).
bool split_tail_ok(TileCfg cfg, int64_t tiles, int G) {
  if (cfg.bn != 256) return false;
  if (const char* env = std::getenv("FM_SPLIT_TAIL"))
    if (env[0] == '0') return false;
  const int64_t rem = tiles % G;
  return rem > 0 && 2 * rem <= G;
}

// split: the launch may run a half-full last wave as 256x128 halves.
TileCfg choose_tile(int64_t M, int64_t N, int G, bool split = true) {
  if (const char* env = std::getenv("FM_TILE")) {
    int bm = 0, bn = 0, nw = 0;
    const int got = std::sscanf(env, "%dx%dw%d", &bm, &bn, &nw);
    if (got >= 2 && (bm == 128 || bm == 256) && (bn == 128 || bn == 256)) {
      if (got < 3 || (nw != 4 && nw != 8)) nw = 4;
      if (!(bm == 128 && bn == 128 && nw == 8)) return {bm, bn, nw};
    }
  }
  const TileCfg cands[3] = {{256, 256, 4}, {256, 128, 4}, {128, 128, 4}};
  const double eff[3] = {1.0, 0.85, 0.7};
  TileCfg best = cands[0];
  double best_cost = 1e300;
  for (int c = 0; c < 3; ++c) {
    const int64_t tiles = cdiv(M, cands[c].bm) * cdiv(N, cands[c].bn);
    const double area = (double)cands[c].bm * cands[c].bn / eff[c];
    double cost = (double)cdiv(tiles, G) * area;
    if (split && split_tail_ok(cands[c], tiles, G))   // last partial wave as 256x128 halves
      cost = (double)(tiles / G) * area + 256.0 * 128.0 / eff[1];
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = cands[c];
    }
  }
  return best;
}

int group_m_default() {
  if (const char* env = std::getenv("FM_GROUP_M")) {
    const int g = std::atoi(env);
    if (g >= 1 && g <= 64) return g;
  }
  return 8;   // 8 M-tiles per band: the 32 tiles in flight per XCD form an 8 x 4 block
}

void fill_order(TileOrder& o, int64_t M, int64_t N, TileCfg cfg) {
  std::memset(&o, 0, sizeof(o));
  o.tiles_m = (int)cdiv(M, cfg.bm);
  o.tiles_n = (int)cdiv(N, cfg.bn);
  o.total = o.tiles_m * o.tiles_n;
  o.group_m = std::min(group_m_default(), o.tiles_m);
  o.has_morder = 0;
}

// Stable order of M-tiles by a key (arrival position / destination rank).
void set_morder(TileOrder& o, const std::vector<int>& key) {
  if (o.tiles_m > kMaxMOrder) return;   // identity order still covers every tile
  std::vector<int> idx(o.tiles_m);
  for (int i = 0; i < o.tiles_m; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return key[a] < key[b]; });
  for (int i = 0; i < o.tiles_m; ++i) o.morder[i] = (uint16_t)idx[i];
  o.has_morder = 1;
}

bool valid_ab(fm_dtype_t dt) { return dt == FM_F16 || dt == FM_BF16; }

template <Mode MODE, bool OUT32>
void launch_one(fm_dtype_t dt, TileCfg cfg, const DenseArgs& args, hipStream_t stream) {
  const int n_pos = (args.pos_end - args.pos0) * args.sub_n;
  const int P = args.prod.n_prod;
  const dim3 grid(P + std::min(n_pos, device_cu_count() - P));
#define FM_LAUNCH(E, BM, BN, NW)                                                              \
  do {                                                                                        \
    if (args.K % kBK) /* ragged K: the 4-wave form keeps the tail path spill-free */          \
      hipLaunchKernelGGL((dense_kernel<E, BM, BN, 4, MODE, OUT32, true>), grid, dim3(256), 0, \
                         stream, args);                                                       \
    else                                                                                      \
      hipLaunchKernelGGL((dense_kernel<E, BM, BN, NW, MODE, OUT32, false>), grid,             \
                         dim3(64 * NW), 0, stream, args);                                     \
  } while (0)
#define FM_LAUNCH_E(E)                                                                        \
  do {                                                                                        \
    if (cfg.bm == 256 && cfg.bn == 256) {                                                     \
      if (cfg.nw == 8) FM_LAUNCH(E, 256, 256, 8); else FM_LAUNCH(E, 256, 256, 4);             \
    } else if (cfg.bm == 256) {                                                               \
      if (cfg.nw == 8) FM_LAUNCH(E, 256, 128, 8); else FM_LAUNCH(E, 256, 128, 4);             \
    } else {                                                                                  \
      FM_LAUNCH(E, 128, 128, 4);                                                              \
    }                                                                                         \
  } while (0)
  if (dt == FM_F16) FM_LAUNCH_E(F16); else FM_LAUNCH_E(BF16);
#undef FM_LAUNCH_E
#undef FM_LAUNCH
}

// One launch over the whole schedule, or -- when the last wave would be at
// most half full -- the full waves first, then the remaining 256x256 tiles as
// 256x128 halves in a second launch on the same stream.  Each output element
// is still summed over K by one workgroup in the same order, so the split
// does not change a single bit of the result.
template <Mode MODE, bool OUT32>
fm_status_t launch_dense(fm_dtype_t dt, TileCfg cfg, DenseArgs& args, hipStream_t stream) {
  const int T = args.order.total;
  if (T <= 0) return FM_OK;
  const int G = device_cu_count();
  if (split_tail_ok(cfg, T, G)) {
    const int rem = T % G, full = T - rem;
    const TileCfg half{cfg.bm, 128, 4};
    if (MODE == Mode::AG || MODE == Mode::AGP) {
      // AllGather: the halves take the first positions (the chunks that
      // arrive first), so the wave that may wait on arrivals is made of the
      // shorter tiles, and the full tiles run once every chunk is likely in.
      args.pos0 = 0;
      args.pos_end = rem;
      args.sub_n = 2;
      launch_one<MODE, OUT32>(dt, half, args, stream);
      if (full > 0) {
        args.pos0 = rem;
        args.pos_end = T;
        args.sub_n = 1;
        launch_one<MODE, OUT32>(dt, cfg, args, stream);
      }
      return launch_status();
    }
    if (full > 0) {
      args.pos0 = 0;
      args.pos_end = full;
      args.sub_n = 1;
      launch_one<MODE, OUT32>(dt, cfg, args, stream);
    }
    args.pos0 = full;
    args.pos_end = T;
    args.sub_n = 2;
    launch_one<MODE, OUT32>(dt, half, args, stream);
  } else {
    args.pos0 = 0;
    args.pos_end = T;
    args.sub_n = 1;
    launch_one<MODE, OUT32>(dt, cfg, args, stream);
  }
  return launch_status();
}

}  // namespace
}  // namespace fm

using namespace fm;

extern "C" fm_status_t fm_gemm(fm_dtype_t ab, fm_dtype_t c, int64_t M, int64_t N, int64_t K,
                               const void* A, const void* B, void* C, hipStream_t stream) {
  if (!valid_ab(ab) || !(c == ab || c == FM_F32)) return FM_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || N % 8 || K % 8) return FM_ERR_INVALID_ARG;
  if (!A || !B || !C || !aligned16(A) || !aligned16(B) || !aligned16(C)) return FM_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FM_OK;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FM_ERR_UNSUPPORTED;
  const TileCfg cfg = choose_tile(M, N, device_cu_count());
  DenseArgs args;
  std::memset(&args, 0, sizeof(args));
  args.A = (const char*)A;
  args.B = (const char*)B;
  args.C = (char*)C;
  args.M = M;
  args.N = N;
  args.K = K;
  fill_order(args.order, M, N, cfg);
  if (c == FM_F32) return launch_dense<Mode::Gemm, true>(ab, cfg, args, stream);
  return launch_dense<Mode::Gemm, false>(ab, cfg, args, stream);
}

extern "C" fm_status_t fm_ag_gemm(fm_dtype_t dt, int64_t M, int64_t N, int64_t K,
                                  int32_t n_chunks, const void* X, const void* W, void* C,
                                  const uint32_t* flags, uint32_t epoch, const int32_t* order,
                                  int32_t* err_word, int64_t spin_limit, hipStream_t stream) {
  if (!valid_ab(dt)) return FM_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || N % 8 || K % 8) return FM_ERR_INVALID_ARG;
  if (n_chunks < 1 || n_chunks > kMaxChunks || M % n_chunks) return FM_ERR_INVALID_ARG;
  if (!X || !W || !C || !flags || !aligned16(X) || !aligned16(W) || !aligned16(C))
    return FM_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(flags) & 3u) || spin_limit < 0) return FM_ERR_INVALID_ARG;
  std::vector<int> pos(n_chunks, -1);
  for (int a = 0; a < n_chunks; ++a) {
    const int c = order ? order[a] : a;
    if (c < 0 || c >= n_chunks || pos[c] != -1) return FM_ERR_INVALID_ARG;
    pos[c] = a;
  }
  if (M == 0 || N == 0) return FM_OK;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FM_ERR_UNSUPPORTED;
  const TileCfg cfg = choose_tile(M, N, device_cu_count());
  DenseArgs args;
  std::memset(&args, 0, sizeof(args));
  args.A = (const char*)X;
  args.B = (const char*)W;
  args.C = (char*)C;
  args.M = M;
  args.N = N;
  args.K = K;
  args.flags = flags;
  args.epoch = epoch;
  args.chunk_rows = M / n_chunks;
  args.err_word = err_word;
  args.spin_limit = spin_limit ? spin_limit : (1ll << 24);
  fill_order(args.order, M, N, cfg);
  // Tiles of the earliest-arriving chunks first (a tile that straddles chunks
  // is keyed by the last of them to arrive).
  std::vector<int> key(args.order.tiles_m);
  for (int tm = 0; tm < args.order.tiles_m; ++tm) {
    const int64_t r0 = (int64_t)tm * cfg.bm, r1 = std::min<int64_t>(r0 + cfg.bm, M) - 1;
    int k = 0;
    for (int64_t c = r0 / args.chunk_rows; c <= r1 / args.chunk_rows; ++c) k = std::max(k, pos[c]);
    key[tm] = k;
  }
  set_morder(args.order, key);
  return launch_dense<Mode::AG, false>(dt, cfg, args, stream);
}

extern "C" fm_status_t fm_ag_gemm_pull(fm_dtype_t dt, int64_t M, int64_t N, int64_t K,
                                       int32_t n_chunks, const void* const* chunks,
                                       const void* W, void* C, const uint32_t* flags,
                                       uint32_t epoch, const int32_t* order, int32_t* err_word,
                                       int64_t spin_limit, hipStream_t stream) {
  if (!valid_ab(dt)) return FM_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || N % 8 || K % 8) return FM_ERR_INVALID_ARG;
  if (n_chunks < 1 || n_chunks > kMaxChunks || M % n_chunks) return FM_ERR_INVALID_ARG;
  if (!chunks || !W || !C || !flags || !aligned16(W) || !aligned16(C)) return FM_ERR_INVALID_ARG;
  for (int c = 0; c < n_chunks; ++c)
    if (!chunks[c] || !aligned16(chunks[c])) return FM_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(flags) & 3u) || spin_limit < 0) return FM_ERR_INVALID_ARG;
  std::vector<int> pos(n_chunks, -1);
  for (int a = 0; a < n_chunks; ++a) {
    const int c = order ? order[a] : a;
    if (c < 0 || c >= n_chunks || pos[c] != -1) return FM_ERR_INVALID_ARG;
    pos[c] = a;
  }
  if (M == 0 || N == 0) return FM_OK;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FM_ERR_UNSUPPORTED;
  const int64_t Mc = M / n_chunks;
  // The tile shape is chosen as for fm_ag_gemm; tiles are then cut per chunk.
  const TileCfg cfg = choose_tile(M, N, device_cu_count());
  const int tpc = (int)cdiv(Mc, cfg.bm);
  DenseArgs args;
  std::memset(&args, 0, sizeof(args));
  args.B = (const char*)W;
  args.C = (char*)C;
  args.M = M;
  args.N = N;
  args.K = K;
  args.flags = flags;
  args.epoch = epoch;
  args.chunk_rows = Mc;
  args.err_word = err_word;
  args.spin_limit = spin_limit ? spin_limit : (1ll << 24);
  args.tiles_per_chunk = tpc;
  for (int c = 0; c < n_chunks; ++c) args.chunk_a[c] = (const char*)chunks[c];
  fill_order(args.order, (int64_t)n_chunks * tpc * cfg.bm, N, cfg);
  std::vector<int> key(args.order.tiles_m);
  for (int tm = 0; tm < args.order.tiles_m; ++tm) key[tm] = pos[tm / tpc];
  set_morder(args.order, key);
  return launch_dense<Mode::AGP, false>(dt, cfg, args, stream);
}

// Producer workgroups for an M x N AllGather-GEMM that copies `bytes`: the
// largest multiple of 8 (one per XCD per round) that keeps the consumers'
// tile waves at their minimum, capped at one producer per MiB copied and at
// half the CUs.  More producers copy faster, and the chip clocks higher with
// fewer CUs in the GEMM, until the consumers lose a wave.  Measured on the
// TP=8 AllGather (384 tiles, 7 chunks of 12.58 MB): 8/16/32/48/64 producers
// took 0.75/0.69/0.64/0.60/0.59 ms; 80, which leaves 176 consumers and a
// third wave, 0.97 ms.
int producers_default(int64_t M, int64_t N, int64_t bytes, int cus) {
  if (const char* env = std::getenv("FM_PRODUCERS")) {
    const int p = std::atoi(env);
    if (p >= 8 && p <= cus / 2 && p % 8 == 0) return p;
  }
  const int cap = (int)std::max<int64_t>(
      8, std::min<int64_t>(cus / 2 / 8 * 8, (cdiv(bytes, 1ll << 20) + 7) / 8 * 8));
  int best = 8;
  double best_cost = 1e300;
  for (int P = 8; P <= cap; P += 8) {
    const int G = cus - P;
    const TileCfg cfg = choose_tile(M, N, G, false);
    const double eff = cfg.bn == 256 ? 1.0 : (cfg.bm == 256 ? 0.85 : 0.7);
    const int64_t tiles = cdiv(M, cfg.bm) * cdiv(N, cfg.bn);
    const double cost = (double)cdiv(tiles, G) * cfg.bm * cfg.bn / eff;
    if (cost <= best_cost * 1.0001) {   // ties go to more producers
      best_cost = std::min(best_cost, cost);
      best = P;
    }
  }
  return best;
}

extern "C" fm_status_t fm_ag_gemm_producers(fm_dtype_t dt, int64_t M, int64_t N, int64_t K,
                                            int32_t n_chunks, const void* const* src, void* X,
                                            const void* W, void* C, uint32_t* flags,
                                            uint32_t* counters, uint32_t epoch,
                                            const int32_t* order, int32_t n_producers,
                                            int32_t* err_word, int64_t spin_limit,
                                            hipStream_t stream) {
  if (!valid_ab(dt)) return FM_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || N % 8 || K % 8) return FM_ERR_INVALID_ARG;
  if (n_chunks < 1 || n_chunks > kMaxChunks || M % n_chunks) return FM_ERR_INVALID_ARG;
  if (!src || !X || !W || !C || !flags || !counters || !aligned16(X) || !aligned16(W) ||
      !aligned16(C))
    return FM_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(flags) & 3u) || (reinterpret_cast<uintptr_t>(counters) & 3u) ||
      spin_limit < 0)
    return FM_ERR_INVALID_ARG;
  if (n_producers != 0 && (n_producers < 8 || n_producers % 8)) return FM_ERR_INVALID_ARG;
  const int64_t chunk_bytes = (M / n_chunks) * K * 2;
  const char* xb = (const char*)X;
  int64_t copy_bytes = 0;
  for (int c = 0; c < n_chunks; ++c) {
    const char* sc = (const char*)src[c];
    if (!sc) continue;
    if (!aligned16(sc)) return FM_ERR_INVALID_ARG;
    if (sc < xb + M * K * 2 && xb < sc + chunk_bytes) return FM_ERR_INVALID_ARG;   // overlaps X
    copy_bytes += chunk_bytes;
  }
  std::vector<int> pos(n_chunks, -1);
  for (int a = 0; a < n_chunks; ++a) {
    const int c = order ? order[a] : a;
    if (c < 0 || c >= n_chunks || pos[c] != -1) return FM_ERR_INVALID_ARG;
    pos[c] = a;
  }
  if (M == 0 || N == 0) return FM_OK;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FM_ERR_UNSUPPORTED;
  const int cus = device_cu_count();
  const int P = n_producers ? n_producers : producers_default(M, N, copy_bytes, cus);
  if (P > cus / 2) return FM_ERR_INVALID_ARG;
  // The consumers hold the CUs the producers leave free.
  const TileCfg cfg = choose_tile(M, N, cus - P, false);
  DenseArgs args;
  std::memset(&args, 0, sizeof(args));
  args.A = xb;
  args.B = (const char*)W;
  args.C = (char*)C;
  args.M = M;
  args.N = N;
  args.K = K;
  args.flags = flags;
  args.epoch = epoch;
  args.chunk_rows = M / n_chunks;
  args.err_word = err_word;
  args.spin_limit = spin_limit ? spin_limit : (1ll << 24);
  fill_producers(args.prod, P, n_chunks, chunk_bytes, src, order, X, flags, counters, epoch);
  fill_order(args.order, M, N, cfg);
  std::vector<int> key(args.order.tiles_m);
  for (int tm = 0; tm < args.order.tiles_m; ++tm) {
    const int64_t r0 = (int64_t)tm * cfg.bm, r1 = std::min<int64_t>(r0 + cfg.bm, M) - 1;
    int k = 0;
    for (int64_t c = r0 / args.chunk_rows; c <= r1 / args.chunk_rows; ++c) k = std::max(k, pos[c]);
    key[tm] = k;
  }
  set_morder(args.order, key);
  // one launch: producers and consumers must run together
  args.pos0 = 0;
  args.pos_end = args.order.total;
  args.sub_n = 1;
  launch_one<Mode::AGX, false>(dt, cfg, args, stream);
  return launch_status();
}

extern "C" fm_status_t fm_gemm_rs(fm_dtype_t dt, int64_t M, int64_t N, int64_t K,
                                  int32_t n_ranks, int32_t rank, const void* A, const void* W,
                                  float* const* dst, int32_t atomic, hipStream_t stream) {
  if (!valid_ab(dt)) return FM_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || N % 8 || K % 8) return FM_ERR_INVALID_ARG;
  if (n_ranks < 1 || n_ranks > kMaxRanks || M % n_ranks || rank < 0 || rank >= n_ranks)
    return FM_ERR_INVALID_ARG;
  if (!A || !W || !dst || !aligned16(A) || !aligned16(W) || (atomic != 0 && atomic != 1))
    return FM_ERR_INVALID_ARG;
  for (int r = 0; r < n_ranks; ++r)
    if (!dst[r] || !aligned16(dst[r])) return FM_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return FM_OK;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FM_ERR_UNSUPPORTED;
  const TileCfg cfg = choose_tile(M, N, device_cu_count());
  DenseArgs args;
  std::memset(&args, 0, sizeof(args));
  args.A = (const char*)A;
  args.B = (const char*)W;
  args.M = M;
  args.N = N;
  args.K = K;
  args.atomic = atomic;
  args.slice_rows = M / n_ranks;
  for (int r = 0; r < n_ranks; ++r) args.dst[r] = dst[r];
  fill_order(args.order, M, N, cfg);
  // Destination-rank order starting at rank+1, so that on a real TP group the
  // ranks start on different slices (slice of a tile = slice of its first row).
  std::vector<int> key(args.order.tiles_m);
  for (int tm = 0; tm < args.order.tiles_m; ++tm) {
    const int s = (int)(((int64_t)tm * cfg.bm) / args.slice_rows);
    key[tm] = ((s - (rank + 1)) % n_ranks + n_ranks) % n_ranks;
  }
  set_morder(args.order, key);
  if (!atomic && args.slice_rows % cfg.bm == 0)
    return launch_dense<Mode::RS, false>(dt, cfg, args, stream);
  return launch_dense<Mode::RSG, false>(dt, cfg, args, stream);
}
