// Device helpers shared by the i8mm kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

typedef int32_t v4i32 __attribute__((ext_vector_type(4)));
typedef int32_t v16i32 __attribute__((ext_vector_type(16)));
typedef float v16f32 __attribute__((ext_vector_type(16)));
typedef _Float16 v8f16 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// fp16 bits <-> fp32. The widening conversion is exact; the narrowing one
// rounds to nearest even (the default rounding mode of the hardware).
__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Half element e (0..7) of a 16-byte chunk.
__device__ __forceinline__ uint32_t half_of(const uint4& v, int e) {
  uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

}  // namespace i8mm
