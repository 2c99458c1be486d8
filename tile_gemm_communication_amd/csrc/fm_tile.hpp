// fm_tile.hpp -- the MFMA macro-tile engine shared by every GEMM-shaped
// kernel in libfluxmi (dense, AllGather, ReduceScatter, grouped MoE).
//
// One workgroup = 4 wave64 (one per SIMD) arranged 2x2 over a BM x BN output
// tile; each wave owns a (BM/2) x (BN/2) sub-tile made of 32x32 blocks
// computed with v_mfma_f32_32x32x16_{f16,bf16} into fp32 accumulators.
//
// Data path per K step of 64:
//   HBM/L2 --128-bit loads--> VGPRs --ds_write--> LDS (two stages) --ds_read_b128--> MFMA
// A tiles ([M,K] row-major) are stored in LDS as rows of 64 K-elements.  B
// tiles ([K,N] row-major) are transposed while staging (an 8x8 / 4x8 block
// transpose of 16-bit elements in registers) so that LDS holds B^T rows of 64
// K-elements too; both MFMA operands are then single 16-byte LDS reads.
// Each 128-byte LDS row is split into eight 16-byte chunks placed at
// chunk ^ ((row ^ row>>3) & 7), which keeps both the staging writes and the
// fragment reads free of bank conflicts.
//
// The MFMA is issued with B^T as the first operand and A as the second, so
// the 32x32 result block is C^T in the instruction's layout: lane l holds row
// m = l % 32 of C and, for item 4r+q, column n = 8r + 4(l/32) + q.  Every lane
// therefore owns runs of 4 consecutive output columns, which the epilogues
// store (or read-add-write) as 8- or 16-byte vectors.
#pragma once

#include "fm_common.hpp"

namespace fm {

__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ lds_swz(row)) << 4);
}

// Pack 16-bit element `c` (0..7) of two 8-element rows into one dword
// (lo = row x, hi = row y).
template <int c>
__device__ __forceinline__ uint32_t pick2(const u32x4& x, const u32x4& y) {
  constexpr uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
  return __builtin_amdgcn_perm(y[c >> 1], x[c >> 1], sel);
}

template <class E, int BM, int BN>
struct Engine {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_LOADS = BM / 32;   // 16-byte A chunks per thread per stage
  static constexpr int B_ROWS = BN / 32;    // B rows (of 8 columns) per thread per stage
  static constexpr int B_NG = BN / 8;       // 8-column groups across the tile
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = BN * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(BM == 128 || BM == 256, "BM must be 128 or 256");
  static_assert(B_ROWS == 8 || B_ROWS == 4, "BN must be 128 or 256");

  char* smem;
  int t, lane, wm, wn;
  int64_t K;

  f32x16 acc[FM][FN];
  u32x4 ra[A_LOADS];
  u32x4 rb[B_ROWS];

  // Per-tile operand sources (set by the kernel before run()).
  const char* a_row[A_LOADS];   // start of the A row feeding staging slot i
  const char* b_col;            // B + (this thread's 8-column group) elements
  int64_t ldb_bytes;            // B row pitch in bytes

  __device__ __forceinline__ Engine(char* s, int64_t K_) : smem(s), K(K_) {
    t = threadIdx.x;
    lane = t & 63;
    int w = t >> 6;
    wm = w >> 1;
    wn = w & 1;
  }

  // Row (within the tile) of staging slot i, and this thread's A chunk.
  __device__ __forceinline__ int a_stage_row(int i) const { return (t >> 3) + 32 * i; }
  __device__ __forceinline__ int a_chunk() const { return t & 7; }
  // This thread's B k-group and 8-column group.
  __device__ __forceinline__ int b_group() const { return t / B_NG; }
  __device__ __forceinline__ int b_colgroup() const { return t % B_NG; }

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
  }

  // Global -> registers for K step kt.  CHECK zero-fills K positions >= K.
  template <bool CHECK>
  __device__ __forceinline__ void gload(int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
    const int64_t ka = k0 + 8 * a_chunk();
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      if (!CHECK || ka < K)
        ra[i] = *reinterpret_cast<const u32x4*>(a_row[i] + ka * 2);
      else
        ra[i] = u32x4{0, 0, 0, 0};
    }
    const int64_t kb = k0 + (int64_t)b_group() * B_ROWS;
#pragma unroll
    for (int j = 0; j < B_ROWS; ++j) {
      if (!CHECK || kb + j < K)
        rb[j] = *reinterpret_cast<const u32x4*>(b_col + (kb + j) * ldb_bytes);
      else
        rb[j] = u32x4{0, 0, 0, 0};
    }
  }

  // Registers -> LDS stage s (A as-is, B transposed).
  __device__ __forceinline__ void lstore(int s) {
    char* sa = smem + s * STAGE;
    char* sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      *reinterpret_cast<u32x4*>(sa + lds_off(a_stage_row(i), a_chunk())) = ra[i];
    const int g = b_group();
    const int nb = 8 * b_colgroup();
    if constexpr (B_ROWS == 8) {
      // rb[j] = 8 columns of K row (8g + j).  Column c becomes LDS row nb + c
      // holding K elements 8g .. 8g+7 = logical chunk g.
#define FM_BT8(c)                                                               \
  {                                                                             \
    u32x4 v = {pick2<c>(rb[0], rb[1]), pick2<c>(rb[2], rb[3]),                  \
               pick2<c>(rb[4], rb[5]), pick2<c>(rb[6], rb[7])};                 \
    *reinterpret_cast<u32x4*>(sb + lds_off(nb + c, g)) = v;                     \
  }
      FM_BT8(0) FM_BT8(1) FM_BT8(2) FM_BT8(3) FM_BT8(4) FM_BT8(5) FM_BT8(6) FM_BT8(7)
#undef FM_BT8
    } else {
      // rb[j] = 8 columns of K row (4g + j): K elements 4g .. 4g+3 are the
      // (g & 1) half of logical chunk g >> 1.
#define FM_BT4(c)                                                               \
  {                                                                             \
    u32x2 v = {pick2<c>(rb[0], rb[1]), pick2<c>(rb[2], rb[3])};                 \
    *reinterpret_cast<u32x2*>(sb + lds_off(nb + c, g >> 1) + ((g & 1) << 3)) = v; \
  }
      FM_BT4(0) FM_BT4(1) FM_BT4(2) FM_BT4(3) FM_BT4(4) FM_BT4(5) FM_BT4(6) FM_BT4(7)
#undef FM_BT4
    }
  }

  // MFMA over one LDS stage (four K sub-steps of 16).
  __device__ __forceinline__ void compute(int s) {
    const char* sa = smem + s * STAGE;
    const char* sb = sa + A_BYTES;
    const int r32 = lane & 31;
    const int half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = 2 * ks + half;
      u32x4 fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[i] = *reinterpret_cast<const u32x4*>(sa + lds_off(wm * WM + i * 32 + r32, chunk));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const u32x4*>(sb + lds_off(wn * WN + j * 32 + r32, chunk));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = E::mfma32(fb[j], fa[i], acc[i][j]);
    }
  }

  // Full K loop over KT steps; accumulators start at zero.  Ends with a
  // workgroup barrier, so LDS may be reused right after.
  __device__ __forceinline__ void run() {
    zero_acc();
    const int KT = (int)cdiv(K, kBK);
    if (KT == 0) {
      __syncthreads();
      return;
    }
    const bool tail = (K % kBK) != 0;
    if (tail && KT == 1) gload<true>(0); else gload<false>(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const bool more = kt + 1 < KT;
      if (more) {
        if (tail && kt + 2 == KT) gload<true>(kt + 1); else gload<false>(kt + 1);
      }
      compute(kt & 1);
      if (more) lstore((kt + 1) & 1);
      __syncthreads();
    }
  }

  // Output coordinates (within the tile) owned by this lane.
  __device__ __forceinline__ int out_row(int i) const { return wm * WM + i * 32 + (lane & 31); }
  __device__ __forceinline__ int out_col(int j, int r) const {
    return wn * WN + j * 32 + 8 * r + 4 * (lane >> 5);
  }
  __device__ __forceinline__ f32x4 out_vals(int i, int j, int r) const {
    return f32x4{acc[i][j][4 * r + 0], acc[i][j][4 * r + 1], acc[i][j][4 * r + 2],
                 acc[i][j][4 * r + 3]};
  }
};

}  // namespace fm
