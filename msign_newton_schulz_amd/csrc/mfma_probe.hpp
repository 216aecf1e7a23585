// Measurement only: a kernel that issues nothing but 16x16x32 MFMAs, to
// measure the matrix rate the chip sustains under its clock and power
// limits (the published dense peak assumes 2.4 GHz).  Every wave keeps 8
// independent accumulator chains, so consecutive MFMAs never wait on each
// other; operands stay in registers (no memory traffic until one store per
// lane at the end, which keeps the result alive).
#pragma once

#include "common.hpp"

#include <type_traits>

namespace msign {

constexpr int kProbeBlocks = 512;   // 2 per CU
constexpr int kProbeThreads = 256;  // 4 waves: 8 waves per CU, 2 per SIMD
constexpr int kProbeChains = 8;

template <typename T>
__global__ void __launch_bounds__(kProbeThreads) mfma_probe_kernel(int32_t iters, float seed, float* out) {
  const float v = seed + (float)threadIdx.x * 1e-3f;
  uint32_t bits;
  if constexpr (std::is_same<T, bf16_t>::value) {
    bits = (uint32_t)f32_to_bf16_bits(v) * 0x10001u;
  } else {
    bits = (uint32_t)f32_to_f16_bits(v) * 0x10001u;
  }
  const u32x4 a = {bits, bits ^ 0x1u, bits, bits ^ 0x2u};
  const u32x4 b = {bits ^ 0x4u, bits, bits ^ 0x8u, bits};
  // Runtime (nonzero) starting values: with zero-initialised chains the
  // compiler rotated all accumulators through other registers on every
  // iteration (about 6 moves per MFMA).
  f32x4 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4{v + (float)c, v, v, v};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) {
      if constexpr (std::is_same<T, bf16_t>::value)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, b), acc[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                        __builtin_bit_cast(f16x8, b), acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace msign
