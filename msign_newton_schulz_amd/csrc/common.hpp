// Shared device-side types and helpers for the msign kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msign {

enum DType : int32_t { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct bf16_t { uint16_t bits; };  // storage tags for templates
struct f16_t { uint16_t bits; };

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int size = 4; static constexpr int32_t dt = DT_F32; };
template <> struct Elem<bf16_t> { static constexpr int size = 2; static constexpr int32_t dt = DT_BF16; };
template <> struct Elem<f16_t> { static constexpr int size = 2; static constexpr int32_t dt = DT_F16; };

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
// Round-to-nearest-even conversions (the hardware cvt instructions).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Load element `i` of a buffer of runtime dtype as fp32.
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i, int32_t dt) {
  if (dt == DT_F32) return static_cast<const float*>(p)[i];
  uint16_t b = static_cast<const uint16_t*>(p)[i];
  return dt == DT_BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// Store fp32 value `v` as element `i` of a buffer of runtime dtype.
__device__ __forceinline__ void store_from_f32(void* p, int64_t i, int32_t dt, float v) {
  if (dt == DT_F32) { static_cast<float*>(p)[i] = v; return; }
  uint16_t b = dt == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
  static_cast<uint16_t*>(p)[i] = b;
}

__device__ __forceinline__ int dtype_size(int32_t dt) { return dt == DT_F32 ? 4 : 2; }

}  // namespace msign
