// fm_tile.hpp -- the MFMA macro-tile engine shared by every GEMM-shaped
// kernel in libfluxmi (dense, AllGather, ReduceScatter, grouped MoE).
//
// One workgroup = NW wave64 (4: one per SIMD, 8: two per SIMD) arranged
// 2 x NW/2 over a BM x BN output tile; each wave owns a (BM/2) x (BN/(NW/2))
// sub-tile of 32x32 blocks computed with v_mfma_f32_32x32x16_{f16,bf16} into
// fp32 accumulators (AGPRs).  With two waves per SIMD the matrix core takes
// MFMAs from whichever wave is ready, which covers issue gaps, LDS latency
// and barrier skew of the other.
//
// Data path, one LDS stage = one K step of 64, two stages in flight:
//   HBM/L2 --global_load_lds_dwordx4 (direct to LDS, no VGPR staging)--> LDS
//   LDS --ds_read_b128 (A) / 2 x ds_read_b64_tr_b16 (B)--> VGPR fragments --> MFMA
// LDS layout: [A stage 0 | A stage 1 | B stage 0 | B stage 1].  An A stage is
// BM rows x 64 K-elements (128 B per row); a B stage is 64 K-rows x BN
// N-elements, row-major like B itself.  The transposing LDS read hands each
// lane the K-run of one B column that the MFMA operand needs, so B is never
// transposed in registers.
//
// Bank-conflict-free placement: rows are cut into 16-byte chunks; chunk c of
// A row m is stored at c ^ ((m ^ m>>3) & 7) and chunk c of B row k at
// c ^ BSWZ*(k & 3) (BSWZ = 4 for the 64-bank LDS of gfx950).  A
// direct-to-LDS load writes its 64 lanes' 16 bytes contiguously, so the
// placement is realised by choosing which global chunk each lane fetches.
//
// The loads are issued with inline assembly: the compiler then sees no LDS
// DMA and does not order every later LDS read behind it; the ordering the
// pipeline needs is explicit (s_waitcnt + barrier below).
//
// Pipeline per K step kt (buffer cur = kt & 1).  With a read-ahead of one
// sub-step (two fragment register slots):
//   sub-steps 0..2: MFMAs interleaved with the LDS reads of the next
//                   sub-step's fragments;
//   barrier:        after this wave's DMA of stage kt+1 and its reads of
//                   stage kt are done (stage kt+1 complete, stage kt drained);
//   sub-step 3:     MFMAs interleaved with the reads of sub-step 0 of stage
//                   kt+1 and the DMA of stage kt+2 into buffer cur.
// With a read-ahead of two (four slots, one wave per SIMD) sub-steps 0 and 1
// read sub-steps 2 and 3, the barrier follows sub-step 1, and sub-steps 2
// and 3 read sub-steps 0 and 1 of stage kt+1 while issuing the DMA.
// Every instruction group is fenced with sched_barrier, so the issue order is
// the source order: one LDS read or DMA per MFMA, never a burst of loads
// that would leave the matrix cores idle.
//
// The MFMA takes B^T as its first operand and A as its second, so a 32x32
// result block is C^T in the instruction's layout: lane l holds row
// m = l % 32 of C and, for item 4r+q, column n = 8r + 4(l/32) + q; every lane
// owns runs of 4 consecutive output columns.
//
// MF16 selects v_mfma_f32_16x16x32 instead (one wave per SIMD only).  Under
// the chip's power limit it does more work per joule in isolation: with
// N(0,1) operands a register-only loop ran 1786 TFLOP/s at 1.82 GHz against
// 1650 at 1.65 GHz for the 32x32x16 form, since it moves a quarter of the
// accumulator bits per flop; in the full GEMM (LDS and DMA traffic, one wave
// per SIMD) it measured 1-3% slower, so the kernels build it only on request.
// The MFMA is issued from inline assembly with the accumulator tied in place:
// the builtin's result takes fresh AGPRs, and the copies back filled the K
// loop with ~470 accumulator moves and spills.  A K step then has two sub-steps of 32; the fragments of a 16x16
// block come from the same LDS layout (A: one 16-byte read, rows 16i + l%16,
// K chunk 4ks + l/16; B: two transposing reads, K rows 32ks + 8(l/16) + 0..7
// of column l%16), and the result block (C^T again) gives lane l row
// 16i + l%16 and columns 4(l/16)..+3 of its 16-column block.
#pragma once

#include <type_traits>
#include <utility>

#include "fm_common.hpp"

namespace fm {

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define FM_LDS4(p) ((__attribute__((address_space(3))) s16x4*)(p))

__device__ __forceinline__ int swz_a(int row) { return (row ^ (row >> 3)) & 7; }

// s_waitcnt encodings (gfx9: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_all0() { __builtin_amdgcn_s_waitcnt(0x0070); }
// The same waits as compiler memory barriers: LDS reads of DMA-written data
// are not hoisted above wait_vm_mem, and a DMA into LDS the wave still reads
// is not hoisted above wait_lgkm_mem.
template <int N>
__device__ __forceinline__ void wait_vm_mem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm_mem() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One 16-byte-per-lane direct-to-LDS load: lane i's 16 bytes from
// sbase + voff_i land at LDS byte lds + 16 i.  sbase and lds are wave-uniform.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
// The same from a per-lane 64-bit address (rows of one tile in different
// buffers).
__device__ __forceinline__ void dma16_64(const void* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(vaddr), "s"(lds)
               : "memory", "m0");
}
// The same with the non-temporal hint (data read once: kept out of the way
// of operands that are reused).
__device__ __forceinline__ void dma16_64_nt(const void* vaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(vaddr), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1,
// every iteration its own code (no loop left for the compiler to keep, so
// register arrays indexed by I stay in registers however long the body).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Scheduling hint: alternate MFMAs and LDS reads (one each, READS times),
// then the remaining MFMAs.
template <int MFMAS, int READS>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int q = 0; q < READS; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  if constexpr (MFMAS > READS) __builtin_amdgcn_sched_group_barrier(0x008, MFMAS - READS, 0);
}

template <class E, int BM, int BN, bool KTAIL, int NW = 4, int BSWZ = 4, int DEPTH_ = 1,
          bool MF16 = false, bool A64 = false, int NSTAGE_ = 2>
struct Engine {
  // LDS stages in flight: 2 (double buffering), or 3 for tiles whose stages
  // are small enough (a K step of a 256x128 tile is half as long as one of a
  // 256x256 tile, too short to hide an L2/MALL miss with one stage of
  // look-ahead).  A K tail and the 16x16 form keep 2.
  static constexpr int NSTAGE = (KTAIL || MF16) ? 2 : NSTAGE_;
  static_assert(NSTAGE == 2 || NSTAGE == 3, "2 or 3 LDS stages");
  // Fragment read-ahead in sub-steps: 1 = the next sub-step (two register
  // slots), 2 = two sub-steps ahead (four slots, one per sub-step; needs the
  // register room of one wave per SIMD).  A K tail, and the 16x16 form (whose
  // sub-step is already half a K step), always use 1.
  static constexpr int DEPTH = (KTAIL || MF16) ? 1 : DEPTH_;
  static constexpr int NSLOT = DEPTH == 2 ? 4 : 2;
  static constexpr int NWM = 2, NWN = NW / 2;          // wave grid over the tile
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM_ = BM, BN_ = BN;
  static constexpr int WM = BM / NWM, WN = BN / NWN;
  static constexpr int FM = WM / 32, FN = WN / 32;     // 32x32 blocks per wave
  static constexpr int BMF = MF16 ? 16 : 32;            // MFMA block edge
  static constexpr int FMB = WM / BMF, FNB = WN / BMF;  // MFMA blocks per wave
  static constexpr int NSUB = MF16 ? 2 : 4;             // sub-steps per K step
  static constexpr int A_STAGE = BM * 128;
  static constexpr int B_ROW = BN * 2;
  static constexpr int B_STAGE = 64 * B_ROW;
  static constexpr int LDS_B = NSTAGE * A_STAGE;        // B stages follow the A stages
  static constexpr int LDS_BYTES = NSTAGE * (A_STAGE + B_STAGE);
  static constexpr int A_ROWS = BM / NW;                // A rows each wave stages
  static constexpr int A_DMA = A_ROWS / 8;              // DMA instructions per wave per stage
  static constexpr int B_CPR = BN / 8;                  // 16-byte chunks per B row
  static constexpr int B_RPI = 64 / B_CPR;              // B rows per 1 KB DMA instruction
  static constexpr int B_DMA = BN / (8 * NW);
  static constexpr int DMA = A_DMA + B_DMA;
  static constexpr int READS = FMB + 2 * FNB;           // LDS reads per sub-step
  static constexpr int MFMAS = FMB * FNB;               // MFMAs per sub-step
  static_assert(BM == 128 || BM == 256, "BM must be 128 or 256");
  static_assert(BN == 128 || BN == 256, "BN must be 128 or 256");
  static_assert(BSWZ == 2 || BSWZ == 4, "B swizzle step");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(A_DMA >= 1 && B_DMA >= 1 && WN >= 32, "tile too small for the wave grid");
  static_assert(!MF16 || NW == 4, "the 16x16 form needs the registers of one wave per SIMD");

  char* smem;
  uint32_t lds0;   // LDS byte address of smem (wave-uniform)
  int lane, w, wm, wn;
  int64_t K;
  int KT;

  using AccT = typename std::conditional<MF16, f32x4, f32x16>::type;
  AccT acc[FMB][FNB];
  u32x4 fa[NSLOT][FMB];
  u32x4 fb[NSLOT][FNB];

  // DMA sources: wave-uniform bases (K offset 0) plus per-lane 32-bit offsets.
  const char* a_base;
  const char* b_base;
  uint32_t a_off[A64 ? 1 : A_DMA];
  const char* a_ptr[A64 ? A_DMA : 1];   // A64: per-lane row addresses
  uint32_t b_off[B_DMA];
  int64_t b_step;             // bytes of 64 B rows (one K step)

  // LDS read offsets (bytes from smem): A by (sub-step, block parity), B by
  // block-column variant; everything else is an immediate.
  static constexpr int BV = (BSWZ == 2) ? 2 : 4;   // B address variants
  // MF16: A offsets by swizzle variant p (sub-step ks uses p ^ 2ks), B by
  // bits 1-2 of the block index (bit 0 is an immediate).
  static constexpr int RA_KS = MF16 ? 1 : 4, RA_P = MF16 ? 4 : 2;
  static constexpr int RB_N = MF16 ? 4 : BV;
  uint32_t ra_off[RA_KS][RA_P];
  uint32_t rb_off[RB_N];

  __device__ __forceinline__ Engine(char* s, int64_t K_) : smem(s), K(K_) {
    const int t = threadIdx.x;
    lane = t & 63;
    w = __builtin_amdgcn_readfirstlane(t >> 6);
    wm = w / NWN;
    wn = w % NWN;
    lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)s);
    KT = (int)cdiv(K, kBK);
    if constexpr (MF16) {
      // A fragment of 16x16 block i, sub-step ks: row m = wm*WM + 16i + r16,
      // chunk 4ks + l/16 = 4ks ^ q4; swz_a(m) = s0 ^ 2(i&3) with
      // s0 = (r16 ^ r16>>3) & 7, so the physical chunk is
      // q4 ^ s0 ^ 2((i&3) ^ 2ks): variant p = (i ^ 2ks) & 3.
      const int r16 = lane & 15, q4 = lane >> 4;
      const int s0 = (r16 ^ (r16 >> 3)) & 7;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        ra_off[0][p] = (wm * WM + r16) * 128 + (((q4 ^ s0 ^ (2 * p)) & 7) << 4);
      // B fragment of block j = 2a + b: group g = l/16 covers K rows 8g..+7
      // of the sub-step and the block's 16 columns; lane j16 addresses K row
      // +(j16>>2) (swizzle z) and columns 16j + 4(j16&3), i.e. chunk
      // wn*WN/8 + 4a + 2b + ((j16&3)>>1).  The xor with z only touches bits
      // 2-3, so variant a carries it and b is an immediate of 32 bytes.
      const int j16 = lane & 15;
      const int z = BSWZ * ((j16 >> 2) & 3);
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int X = wn * WN / 8 + 4 * a4 + ((j16 & 3) >> 1);
        rb_off[a4] = LDS_B + (8 * q4 + (j16 >> 2)) * B_ROW + ((X ^ z) << 4) + 8 * (j16 & 1);
      }
      return;
    }
    // A fragment of block i, sub-step ks: row m = wm*WM + 32i + r32, chunk
    // 2ks + hi; swz_a(m) = s0 ^ 4(i&1) with s0 = (r32 ^ r32>>3) & 7.
    const int r32 = lane & 31, hi = lane >> 5;
    const int s0 = (r32 ^ (r32 >> 3)) & 7;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        ra_off[ks][p] = (wm * WM + r32) * 128 + (((2 * ks + hi) ^ s0 ^ (4 * p)) << 4);
    // B fragment of block j: 16-lane group g = lane/16 covers columns
    // 16(g&1)..+15 and K rows 8(g>>1)..+7; lane j16 of the group addresses
    // K row +(j16>>2) and columns +4(j16&3).  Its chunk index is
    // X + 4*BV*(j/BV) with X = wn*WN/8 + 4(j%BV) + 2(g&1) + ((j16&3)>>1), and
    // the swizzle xors it with z = BSWZ*(row&3) < 4*BV, so the j/BV part is an
    // immediate of 64*BV bytes per step.
    const int g = lane >> 4, j16 = lane & 15;
    const int z = BSWZ * ((j16 >> 2) & 3);
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int X = wn * WN / 8 + 4 * v + 2 * (g & 1) + ((j16 & 3) >> 1);
      rb_off[v] = LDS_B + (8 * (g >> 1) + (j16 >> 2)) * B_ROW + ((X ^ z) << 4) + 8 * (j16 & 1);
    }
  }

  // -- DMA placement --------------------------------------------------------
  // A instruction i of this wave fills tile rows w*BM/4 + 8i .. +7; lane L
  // writes physical chunk L&7 of row +L/8, i.e. logical chunk (L&7)^swz.
  __device__ __forceinline__ int a_dma_row(int i) const { return w * A_ROWS + 8 * i + (lane >> 3); }
  __device__ __forceinline__ int a_dma_chunk(int i) const { return (lane & 7) ^ swz_a(a_dma_row(i)); }
  // B instruction i of this wave fills K rows (w*B_DMA + i)*B_RPI .. +B_RPI-1.
  __device__ __forceinline__ int b_dma_row(int i) const { return (w * B_DMA + i) * B_RPI + lane / B_CPR; }
  __device__ __forceinline__ int b_dma_chunk(int i) const {
    return (lane % B_CPR) ^ (BSWZ * (b_dma_row(i) & 3));
  }

  // B operand: element (0,0) at B, row pitch ldb_bytes, tile columns from n0.
  __device__ __forceinline__ void set_b(const char* B, int64_t ldb_bytes, int64_t n0, int64_t N) {
    b_base = B;
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
      const int64_t n = min(n0 + 8 * b_dma_chunk(i), N - 8);
      b_off[i] = (uint32_t)((int64_t)b_dma_row(i) * ldb_bytes + n * 2);
    }
    b_step = 64 * ldb_bytes;
  }
  // A operand: rows come from base + row_off(i) (bytes; < 4 GiB), where
  // row_off(i) is the start of the global row DMA instruction i fetches.
  __device__ __forceinline__ void set_a_base(const char* base) { a_base = base; }
  __device__ __forceinline__ void set_a(int i, uint32_t row_off) {
    a_off[i] = row_off + a_dma_chunk(i) * 16;
  }
  // A64: DMA instruction i of this wave fetches its row from `row` (the
  // row's first element; any buffer).
  __device__ __forceinline__ void set_a64(int i, const char* row) {
    a_ptr[i] = row + a_dma_chunk(i) * 16;
  }
  __device__ __forceinline__ void dma_a(int i, int64_t ka, const char* sa, uint32_t lds) {
    if constexpr (A64)
      dma16_64(a_ptr[i] + ka * 2, lds);
    else
      dma16(a_off[i], sa, lds);
  }

  __device__ __forceinline__ void zero_acc() {
#pragma unroll
    for (int i = 0; i < FMB; ++i)
#pragma unroll
      for (int j = 0; j < FNB; ++j) acc[i][j] = AccT{};
  }

  // Issue the DMA of K step kt into buffer buf.  check: mask K chunks >= K
  // (those LDS slots are zero-filled with ordinary stores instead).
  __device__ __forceinline__ void dma(int kt, int buf, const bool check) {
    const int64_t ka = (int64_t)kt * kBK;
    const char* sa = a_base + ka * 2;
    const char* sb = b_base + (int64_t)kt * b_step;
    const uint32_t la = lds0 + buf * A_STAGE + (w * A_ROWS) * 128;
    const uint32_t lb = lds0 + LDS_B + buf * B_STAGE + (w * B_DMA) * 1024;
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
      if (!check || ka + 8 * a_dma_chunk(i) < K)
        dma_a(i, ka, sa, la + i * 1024);
      else
        *reinterpret_cast<u32x4*>(smem + (la - lds0) + i * 1024 + lane * 16) = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
      if (!check || ka + b_dma_row(i) < K)
        dma16(b_off[i], sb, lb + i * 1024);
      else
        *reinterpret_cast<u32x4*>(smem + (lb - lds0) + i * 1024 + lane * 16) = u32x4{0, 0, 0, 0};
    }
  }

  // -- fragments ------------------------------------------------------------
  // LDS read items of one sub-step, in issue order: for k = 0, 1, ...: A
  // fragment k (if k < FM), then the two halves of B fragment k (if k < FN),
  // so the fragments the first MFMAs need arrive first.  item_code(q) packs
  // (kind, index): kind 0 = A, 1 = B half 0, 2 = B half 1.
  static constexpr int RITEMS = READS;
  static constexpr int item_code(int q) {
    int n = 0;
    for (int k = 0; k < (FMB > FNB ? FMB : FNB); ++k) {
      if (k < FMB) { if (n == q) return k * 4 + 0; ++n; }
      if (k < FNB) {
        if (n == q) return k * 4 + 1;
        ++n;
        if (n == q) return k * 4 + 2;
        ++n;
      }
    }
    return -1;
  }

  __device__ __forceinline__ void read_item(int q, int buf, int ks, int slot) {
    const char* sa = smem + buf * A_STAGE;
    const char* sb = smem + buf * B_STAGE;
    const int code = item_code(q);
    const int j = code >> 2, kind = code & 3;
    if (kind == 0) {
      if constexpr (MF16)
        fa[slot][j] =
            *reinterpret_cast<const u32x4*>(sa + ra_off[0][(j ^ (2 * ks)) & 3] + j * 16 * 128);
      else
        fa[slot][j] = *reinterpret_cast<const u32x4*>(sa + ra_off[ks][j & 1] + j * 32 * 128);
    } else {
      const int hh = kind - 1;
      const char* p = MF16 ? sb + rb_off[(j >> 1) & 3] + (32 * ks + 4 * hh) * B_ROW +
                                 (j & 1) * 32 + (j >> 3) * 256
                           : sb + rb_off[j % RB_N] + (16 * ks + 4 * hh) * B_ROW +
                                 (j / BV) * (64 * BV);
      const s16x4 h = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FM_LDS4(p));
      const u32x2 hv = __builtin_bit_cast(u32x2, h);
      if (hh == 0) { fb[slot][j][0] = hv[0]; fb[slot][j][1] = hv[1]; }
      else { fb[slot][j][2] = hv[0]; fb[slot][j][3] = hv[1]; }
    }
  }

  __device__ __forceinline__ void read_frags(int buf, int ks, int slot) {
#pragma unroll
    for (int q = 0; q < RITEMS; ++q) read_item(q, buf, ks, slot);
  }

  // DMA item d (0 .. DMA-1) of K step kt into buffer buf (full stage).
  __device__ __forceinline__ void dma_item(int d, int kt, int buf) {
    if (d < A_DMA) {
      const uint32_t la = lds0 + buf * A_STAGE + (w * A_ROWS) * 128;
      dma_a(d, (int64_t)kt * kBK, a_base + (int64_t)kt * kBK * 2, la + d * 1024);
    } else {
      const int i = d - A_DMA;
      const uint32_t lb = lds0 + LDS_B + buf * B_STAGE + (w * B_DMA) * 1024;
      dma16(b_off[i], b_base + (int64_t)kt * b_step, lb + i * 1024);
    }
  }

  // One sub-step: the FM x FN MFMAs on fragment slot `cur`, with the reads of
  // the next sub-step (buffer nbuf, sub-step nks, into slot cur^1) and, if
  // DMA_KT >= 0, the DMA of K step DMA_KT into buffer dbuf woven between
  // them.  The source order is the issue order (sched_barrier fences), one
  // memory operation per MFMA where possible.
  __device__ __forceinline__ void substep(int cur, int nbuf, int nks, bool do_read,
                                          int dma_kt, int dbuf) {
    substep_g(cur, nbuf, nks, cur ^ 1, do_read, dma_kt, dbuf, 0, DMA);
  }
  // General form: MFMAs on slot mslot, reads into slot rslot, DMA items
  // [d0, d1) of K step dma_kt.
  __device__ __forceinline__ void substep_g(int mslot, int nbuf, int nks, int rslot,
                                            bool do_read, int dma_kt, int dbuf, int d0, int d1) {
    static_for<MFMAS>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      constexpr int i = q / FNB, j = q % FNB;
      if constexpr (MF16)
        E::mfma16_acc(fb[mslot][j], fa[mslot][i], acc[i][j]);
      else
        acc[i][j] = E::mfma32(fb[mslot][j], fa[mslot][i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      if (do_read && q < RITEMS) {
        read_item(q, nbuf, nks, rslot);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (dma_kt >= 0 && d0 + q < d1) {
        dma_item(d0 + q, dma_kt, dbuf);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
    if (do_read) {       // more read items than MFMAs (small tiles)
#pragma unroll
      for (int q = MFMAS; q < RITEMS; ++q) read_item(q, nbuf, nks, rslot);
    }
    if (dma_kt >= 0) {   // more DMA items than MFMAs
#pragma unroll
      for (int d = d0 + MFMAS; d < d1; ++d) dma_item(d, dma_kt, dbuf);
    }
  }

  // Read-ahead 2: sub-steps 0 and 1 read the fragments of sub-steps 2 and 3
  // of this stage; after the wait and barrier, sub-steps 2 and 3 read
  // sub-steps 0 and 1 of stage kt+1 and issue the DMA of stage kt+2 into
  // buffer cur in two halves.  Every read has a whole sub-step more slack.
  // KIND (two LDS stages only): 0 loads stage kt+2 and reads ahead as
  // usual; 1 (the step before the last) loads nothing; 2 (the last) loads
  // and reads ahead nothing.  With two stages every wait drains all loads,
  // so the steps near the end can skip the loads past K without changing
  // any wait, and the epilogue finds no load in flight; the main loop's body
  // stays free of branches.  With three stages the waits count the loads in
  // flight, so past the end every step loads the last stage again into a
  // buffer nobody reads (KIND 0 throughout).
  template <int KIND = 0>
  __device__ __forceinline__ void step2(int kt) {
    const int cur = kt % NSTAGE, nxt = (kt + 1) % NSTAGE;
    substep_g(0, cur, 2, 2, true, -1, 0, 0, 0);
    substep_g(1, cur, 3, 3, true, -1, 0, 0, 0);
    wait_stage();
    __syncthreads();
    const int dk = KIND != 0 ? -1 : min(kt + NSTAGE, KT - 1);
    substep_g(2, nxt, 0, 0, KIND != 2, dk, cur, 0, DMA / 2);
    substep_g(3, nxt, 1, 1, KIND != 2, dk, cur, DMA / 2, DMA);
  }

  // Before the barrier of K step kt: stage kt+1 has landed (the later stages
  // may still be in flight) and this wave's LDS reads are done.
  __device__ __forceinline__ void wait_stage() {
    if constexpr (NSTAGE == 2) {
      wait_all0();
    } else {
      wait_vmcnt<(NSTAGE - 2) * DMA>();
      wait_lgkm_mem();
    }
  }


  // One K step kt (buffer cur = kt & 1):
  //   sub-steps 0..2: MFMAs on the fragments in registers while the next
  //                   sub-step's fragments are read;
  //   wait for this wave's DMA (stage kt+1) and reads, barrier: stage kt+1 is
  //                   complete and buffer cur is drained;
  //   sub-step 3:     MFMAs while sub-step 0 of stage kt+1 is read and the
  //                   DMA of stage kt+2 is issued into buffer cur.
  // Without a K tail the loads follow KIND as in step2 (each wave only ever
  // writes its own LDS rows, and its loads complete in order, so a later
  // tile's data is never overwritten).
  template <int KIND = 0>
  __device__ __forceinline__ void step(int kt) {
    const int cur = kt % NSTAGE;
    if constexpr (MF16) {
      // two sub-steps of 32: the second reads sub-step 0 of stage kt+1
      substep(0, cur, 1, true, -1, 0);
      wait_all0();
      __syncthreads();
      if constexpr (!KTAIL) {
        substep(1, cur ^ 1, 0, true, min(kt + 2, KT - 1), cur);
      } else {
        if (kt + 2 < KT) dma(kt + 2, cur, kt + 3 == KT);
        substep(1, cur ^ 1, 0, true, -1, 0);
      }
      return;
    }
    substep(0, cur, 1, true, -1, 0);
    substep(1, cur, 2, true, -1, 0);
    substep(0, cur, 3, true, -1, 0);
    wait_stage();
    __syncthreads();
    if constexpr (!KTAIL) {
      const int dk = KIND != 0 ? -1 : min(kt + NSTAGE, KT - 1);
      substep(1, (kt + 1) % NSTAGE, 0, KIND != 2, dk, cur);
    } else {
      if (kt + 2 < KT) dma(kt + 2, cur, kt + 3 == KT);
      substep(1, cur ^ 1, 0, true, -1, 0);
    }
  }

  // Full K loop; accumulators start at zero.  When it returns every wave has
  // passed the last step's barrier, so no wave reads this tile's data any more
  // and the next tile may start its DMA right away.  KTAIL selects the
  // variant that masks a partial last K step (K % 64 != 0).
  //
  // after_first_wait() runs once every wave's memory operations issued before
  // run() have completed (right after the first stage has landed, while the
  // second may still be in flight): a caller can publish there what an
  // earlier tile's stores completed.
  __device__ __forceinline__ void run() { run([] {}); }
  template <class F>
  __device__ __forceinline__ void run(F&& after_first_wait) {
    zero_acc();
    if (KT == 0) {
      wait_vmcnt<0>();
      __syncthreads();
      after_first_wait();
      return;
    }
    if constexpr (NSTAGE == 3) {
      // stages 0, 1 and 2, always three loads so the wait counts them (a
      // short loop loads its last stage again into a buffer it never reads)
      dma(0, 0, false);
      dma(min(1, KT - 1), 1, false);
      dma(min(2, KT - 1), 2, false);
      wait_vmcnt<2 * DMA>();   // stage 0 landed; stages 1 and 2 may be in flight
    } else {
      dma(0, 0, KTAIL && KT == 1);
      if (KT > 1) dma(1, 1, KTAIL && KT == 2);
      if (KT > 1 && !(KTAIL && KT == 2))
        wait_vmcnt<DMA>();   // stage 0 landed; the full stage 1 may still be in flight
      else
        wait_vmcnt<0>();     // a masked stage issues fewer loads: wait for all
    }
    __syncthreads();
    after_first_wait();
    read_frags(0, 0, 0);
    if constexpr (DEPTH == 2) read_frags(0, 1, 1);
    if constexpr (NSTAGE == 2 && !KTAIL && !MF16) {
      // the last two steps load nothing past K (KT >= 1 here)
      int kt = 0;
      for (; kt + 2 < KT; ++kt) {
        if constexpr (DEPTH == 2) step2<0>(kt); else step<0>(kt);
      }
      if (kt + 1 < KT) {
        if constexpr (DEPTH == 2) step2<1>(kt); else step<1>(kt);
        ++kt;
      }
      if constexpr (DEPTH == 2) step2<2>(kt); else step<2>(kt);
    } else {
      for (int kt = 0; kt < KT; ++kt) {
        if constexpr (DEPTH == 2) step2(kt); else step(kt);
      }
    }
  }

  // Pin accumulator block (i, j) in AGPRs at this point of the program, so
  // its copy into VGPRs for the epilogue cannot be hoisted above the stores
  // of earlier blocks (which would need all 256 accumulators in VGPRs).
  __device__ __forceinline__ void pin(int i, int j) { asm volatile("" : "+a"(acc[i][j])); }
  __device__ __forceinline__ f32x4 out_vals(int i, int j, int r) const {
    if constexpr (MF16) {
      return acc[i][j];
    } else {
      return f32x4{acc[i][j][4 * r + 0], acc[i][j][4 * r + 1], acc[i][j][4 * r + 2],
                   acc[i][j][4 * r + 3]};
    }
  }

  // -- LDS-staged epilogue ----------------------------------------------------
  // In the MFMA layout a lane holds 4 columns of one row and a wave's 64 lanes
  // span 32 rows, so a direct global access touches 32 rows x 32 bytes.  The
  // staged epilogue turns each 32-row block of the wave's sub-tile around
  // through a wave-private LDS region: after ep_stage(i) and ep_read(q), lane
  // l holds 4 consecutive fp32 columns of one row and the wave covers EP_RPI
  // whole rows of WN columns, so global loads and stores move full lines.
  // Rows are padded by 16 bytes, which makes both the 16-byte writes (32 rows
  // apart) and the 16-byte reads (row-contiguous) conflict-free.
  static constexpr int EP_STRIDE = WN * 4 + 16;   // bytes per staged row
  static constexpr int EP_LPR = WN / 4;           // lanes per staged row
  static constexpr int EP_RPI = 64 / EP_LPR;      // rows per read instruction
  static constexpr int EP_READS = 32 / EP_RPI;    // reads per 32-row block
  static_assert(NW * 32 * EP_STRIDE <= LDS_BYTES, "staging regions exceed LDS");

  // Before the first ep_stage of a tile: this wave's DMAs have landed and no
  // wave reads K-loop data any more.  After the last ep_read: ep_end() before
  // the next tile's DMA may overwrite the regions.
  __device__ __forceinline__ void ep_begin() {
    if constexpr (MF16) {
      // The 16x16 MFMAs are issued from inline assembly, so the compiler
      // inserts no wait states between the last of them and the epilogue's
      // reads of their accumulators: give them 24 explicitly.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
  __device__ __forceinline__ void ep_end() { __syncthreads(); }
  // PIN: hold each accumulator block in place until its staging (see pin);
  // without it the stores may take the AGPRs as they are.
  template <bool PIN = true>
  __device__ __forceinline__ void ep_stage(int i) {
    // Keep each block's global traffic after its own staging: without this
    // fence the compiler hoists the loads of later blocks and spills.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MF16) {
      // 16x16 blocks 2i and 2i+1: lane l holds row 16h + l%16 of the staged
      // block and columns 16j + 4(l/16)..+3.
      char* reg16 = smem + w * (32 * EP_STRIDE) + (lane & 15) * EP_STRIDE + 16 * (lane >> 4);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < FNB; ++j) {
          pin(2 * i + h, j);
          *reinterpret_cast<f32x4*>(reg16 + 16 * h * EP_STRIDE + 64 * j) = acc[2 * i + h][j];
        }
      return;
    }
    char* reg = smem + w * (32 * EP_STRIDE) + (lane & 31) * EP_STRIDE + 16 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (PIN) pin(i, j);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<f32x4*>(reg + (32 * j + 8 * r) * 4) = out_vals(i, j, r);
    }
  }
  // Tile row and column of the 4 values ep_read(q) returns (block i).
  __device__ __forceinline__ int ep_row(int i, int q) const {
    return wm * WM + i * 32 + q * EP_RPI + lane / EP_LPR;
  }
  __device__ __forceinline__ int ep_col() const { return wn * WN + 4 * (lane % EP_LPR); }
  __device__ __forceinline__ f32x4 ep_read(int q) const {
    return *reinterpret_cast<const f32x4*>(smem + w * (32 * EP_STRIDE) +
                                           (q * EP_RPI + lane / EP_LPR) * EP_STRIDE +
                                           16 * (lane % EP_LPR));
  }

  // Read-modify-write epilogues: after the staging regions each wave owns
  // EP_READS slots of 1 KiB.  ep_fetch(q, p) loads lane l's 16 bytes at p
  // (the destination values of its ep_read(q)) into slot q by DMA, and once
  // that has landed ep_fetched(q) returns them, so a block's destination rows
  // can be in flight without holding registers.
  static constexpr int EP_STAGE_BYTES = NW * 32 * EP_STRIDE;
  static constexpr int EP_RMW_LDS = EP_STAGE_BYTES + NW * EP_READS * 1024;
  __device__ __forceinline__ void ep_fetch(int q, const void* p) const {
    dma16_64(p, lds0 + EP_STAGE_BYTES + (w * EP_READS + q) * 1024);
  }
  // The same as a non-temporal load: for destination rows read only once.
  __device__ __forceinline__ void ep_fetch_once(int q, const void* p) const {
    dma16_64_nt(p, lds0 + EP_STAGE_BYTES + (w * EP_READS + q) * 1024);
  }
  __device__ __forceinline__ f32x4 ep_fetched(int q) const {
    return *reinterpret_cast<const f32x4*>(smem + EP_STAGE_BYTES + (w * EP_READS + q) * 1024 +
                                           lane * 16);
  }
  // First tile row of this wave's epilogue blocks, and its first column.
  __device__ __forceinline__ int ep_row0() const { return wm * WM; }
  __device__ __forceinline__ int ep_col0() const { return wn * WN; }
};

}  // namespace fm
