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

// Store w[0..3] to ptr[base + 0..3] (consecutive elements) in one vector store.
__device__ __forceinline__ void store_vec4(void* ptr, int64_t base, int32_t dt, const float* w) {
  if (dt == DT_F32) {
    f32x4 v = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<f32x4*>(static_cast<float*>(ptr) + base) = v;
  } else {
    uint32_t lo, hi;
    if (dt == DT_BF16) {
      lo = f32_to_bf16_bits(w[0]) | ((uint32_t)f32_to_bf16_bits(w[1]) << 16);
      hi = f32_to_bf16_bits(w[2]) | ((uint32_t)f32_to_bf16_bits(w[3]) << 16);
    } else {
      lo = f32_to_f16_bits(w[0]) | ((uint32_t)f32_to_f16_bits(w[1]) << 16);
      hi = f32_to_f16_bits(w[2]) | ((uint32_t)f32_to_f16_bits(w[3]) << 16);
    }
    u32x2 v = {lo, hi};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(ptr) + base) = v;
  }
}

__device__ __forceinline__ void load_vec4(const void* ptr, int64_t base, int32_t dt, float* d) {
  if (dt == DT_F32) {
    f32x4 v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(ptr) + base);
    d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
  } else {
    u32x2 v = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(ptr) + base);
    uint16_t h[4] = {(uint16_t)(v[0] & 0xffff), (uint16_t)(v[0] >> 16),
                     (uint16_t)(v[1] & 0xffff), (uint16_t)(v[1] >> 16)};
#pragma unroll
    for (int r = 0; r < 4; ++r) d[r] = dt == DT_BF16 ? bf16_bits_to_f32(h[r]) : f16_bits_to_f32(h[r]);
  }
}

}  // namespace msign
