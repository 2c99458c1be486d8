// fm_probe.hip -- the matrix-core ceiling of the chip under its power limit:
// a register-only MFMA loop (no memory traffic in the loop) whose operands
// change from one instruction to the next, as a GEMM's do.  It gives the rate
// and the shader clock that the dense kernels can at most reach with a given
// MFMA form and operand data, against which their roofline fraction is read.
#include <cstring>
#include <type_traits>

#include "fluxmi_probe.h"
#include "fm_common.hpp"

namespace fm {
namespace {

// 32-bit mixing hash (the finaliser of MurmurHash3).
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// An approximately N(0,1) value: the Irwin-Hall sum of four uniforms on
// [0,1), centred and scaled to unit variance.
__device__ __forceinline__ float gauss_like(uint32_t seed) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (float)(mix32(seed * 4u + (uint32_t)i) >> 8) * (1.f / 16777216.f);
  return (s - 2.f) * 1.7320508f;
}

// Each wave keeps NOP operand fragments per side and NCH independent
// accumulator chains, and issues NOP MFMAs per iteration, each on different
// A and B registers.  Thread 0 of every workgroup records the shader-clock
// and constant-rate (100 MHz) counter differences across the loop, and a word
// derived from the accumulators (so the loop cannot be removed).
template <class E, bool MF16>
__global__ __launch_bounds__(512) void mfma_probe_kernel(int64_t iters, int zero, uint64_t* out) {
  constexpr int NOP = 8;
  constexpr int NCH = MF16 ? 8 : 4;
  using AccT = typename std::conditional<MF16, f32x4, f32x16>::type;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 a[NOP], b[NOP];
#pragma unroll
  for (int q = 0; q < NOP; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t s = (gid * NOP + q) * 8u + 2u * j;
      const uint32_t pa = zero ? 0u : E::pack2(gauss_like(s), gauss_like(s + 1));
      const uint32_t pb = zero ? 0u : E::pack2(gauss_like(~s), gauss_like(~s - 1));
      a[q][j] = pa;
      b[q][j] = pb;
    }
  AccT acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] = AccT{};
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < NOP; ++q) {
      if constexpr (MF16)
        E::mfma16_acc(b[q], a[q], acc[q % NCH]);
      else
        acc[q % NCH] = E::mfma32(b[q], a[q], acc[q % NCH]);
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int k = 0; k < (MF16 ? 4 : 16); ++k) sum += acc[c][k];
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[blockIdx.x * 4 + 0] = c1 - c0;
    out[blockIdx.x * 4 + 1] = r1 - r0;
    out[blockIdx.x * 4 + 2] = (uint64_t)__builtin_bit_cast(uint32_t, sum);
    out[blockIdx.x * 4 + 3] = 0;
  }
}

}  // namespace
}  // namespace fm

using namespace fm;

extern "C" fm_status_t fm_probe_mfma(fm_dtype_t dt, int32_t mfma16, int32_t waves_per_simd,
                                     int64_t iters, int32_t zero_operands, uint64_t* out,
                                     int64_t out_words, hipStream_t stream) {
  if (dt != FM_F16 && dt != FM_BF16) return FM_ERR_UNSUPPORTED;
  if ((mfma16 != 0 && mfma16 != 1) || (waves_per_simd != 1 && waves_per_simd != 2) ||
      iters < 1 || iters > (1ll << 30) || !out || (reinterpret_cast<uintptr_t>(out) & 7u))
    return FM_ERR_INVALID_ARG;
  const dim3 grid(device_cu_count()), block(256 * waves_per_simd);
  if (out_words < 4 * (int64_t)grid.x) return FM_ERR_INVALID_ARG;
  const int zero = zero_operands ? 1 : 0;
  if (dt == FM_F16) {
    if (mfma16)
      hipLaunchKernelGGL((mfma_probe_kernel<F16, true>), grid, block, 0, stream, iters, zero, out);
    else
      hipLaunchKernelGGL((mfma_probe_kernel<F16, false>), grid, block, 0, stream, iters, zero, out);
  } else {
    if (mfma16)
      hipLaunchKernelGGL((mfma_probe_kernel<BF16, true>), grid, block, 0, stream, iters, zero, out);
    else
      hipLaunchKernelGGL((mfma_probe_kernel<BF16, false>), grid, block, 0, stream, iters, zero,
                         out);
  }
  return launch_status();
}
