// fm_common.hpp -- types, vector aliases and small helpers shared by the
// libfluxmi kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fluxmi.h"

namespace fm {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;         // K extent of one LDS stage (128 bytes per row)

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Element traits: the 16-bit input formats and how MFMA consumes them.
struct F16 {
  static constexpr fm_dtype_t id = FM_F16;
  __device__ static inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // 16x16x32 accumulating in place (the accumulator stays in its AGPRs; the
  // builtin's result gets a register of its own and is copied back).
  __device__ static inline void mfma16_acc(u32x4 a, u32x4 b, f32x4& c) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  // Round two fp32 values to nearest-even 16-bit and pack (lo = x, hi = y).
  __device__ static inline uint32_t pack2(float x, float y) {
    _Float16 a = (_Float16)x, b = (_Float16)y;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
};

struct BF16 {
  static constexpr fm_dtype_t id = FM_BF16;
  __device__ static inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline void mfma16_acc(u32x4 a, u32x4 b, f32x4& c) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    __bf16 a = (__bf16)x, b = (__bf16)y;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
};


// Store 16 bytes written through every cache level (system-scope store):
// once the wave's vmcnt drains, the data is visible device-wide without an
// L2 write-back.  Used for data handed to a reader that may run on another
// XCD (each XCD has its own, non-coherent L2): the reader learns of it from a
// flag or count published after that drain, and acquires at agent scope.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void store_through(void* p, const u32x4& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_through(float* p, const f32x4& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}
#pragma clang diagnostic pop

// Raw buffer resources (stride 0): word 3 carries the 32-bit data format,
// which untyped dword loads and stores need.  An access at an offset >= the
// record count is out of range: a load returns 0 and a store is dropped.
// kBufStoreThrough is the store cache policy sc0 | sc1 (written through to
// memory, as store_through).
constexpr int kBufRsrcWord3 = 0x00020000;
constexpr int kBufStoreThrough = 17;

// Device properties cached once per device (compute-unit count).
int device_cu_count();

// Translate the last HIP launch error into a status.
inline fm_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? FM_OK : FM_ERR_HIP;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace fm
