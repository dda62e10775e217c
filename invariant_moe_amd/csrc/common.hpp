// Device-side helpers shared by the kernels of this library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bits_to_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f32_to_bits(float f) { return __float_as_uint(f); }

// bf16 bits (low or high half of a packed word) -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Stores of results that other workgroups of the SAME launch read (the
// single-launch layer kernel): CO = true makes them agent-scope coherent
// stores, visible to every XCD once they complete, so the producer needs no
// L2 write-back fence (measured at 9-35 us per fence on MI355X) before it
// signals; the reader still takes an agent-scope acquire.  CO = false is a
// plain store (separate kernels: the kernel boundary makes results visible).
template <bool CO>
struct Out {
  template <typename T>
  __device__ __forceinline__ static void put(T* p, T v) {
    if constexpr (CO)
      __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *p = v;
  }
  __device__ __forceinline__ static void put2(uint2* p, uint2 v) {  // 8 bytes
    if constexpr (CO)
      __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                         (unsigned long long)v.x | ((unsigned long long)v.y << 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *p = v;
  }
  __device__ __forceinline__ static void put4(int4* p, int4 v) {  // 16 bytes, as two halves
    if constexpr (CO) {
      unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
      __hip_atomic_store(q, (unsigned long long)(unsigned)v.x | ((unsigned long long)(unsigned)v.y << 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(q + 1, (unsigned long long)(unsigned)v.z | ((unsigned long long)(unsigned)v.w << 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      *p = v;
    }
  }
};

// Logical id of a workgroup such that consecutive logical ids run on the same
// XCD (workgroups are dealt round-robin over the 8 XCDs by blockIdx.x).
// Returns -1 when this workgroup has no logical id below `total`.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t b, int64_t total) {
  const int64_t chunk = (total + 7) / 8;
  const int64_t l = (b % 8) * chunk + b / 8;
  return (b / 8 < chunk && l < total) ? l : -1;
}

}  // namespace moe
