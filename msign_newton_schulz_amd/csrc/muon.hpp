// The steps of a Muon update on either side of msign: the momentum
// accumulation before it and the parameter update after it.  Reading of
// "Gram Newton-Schulz" §1.1 (the update rule's formula is lost in the text;
// the section names the momentum coefficient mu, the learning rate eta and
// M_0 = 0) together with the Mousse page, §标准 Muon 算法 (the update is
// -msign of the matrix, -U V^T): M <- mu M + G, W <- W - eta msign(M).
//
// Both kernels are elementwise passes bound by HBM bandwidth: four
// consecutive elements per lane (16-byte fp32 and 8-byte 16-bit accesses
// when the buffers allow it), a grid-stride loop over the whole batch.
#pragma once

#include "common.hpp"

namespace msign {

// m[i] <- mu m[i] + g[i] over n elements (m fp32, g of dtype gdt); vec when
// m and g are aligned for 4-element accesses.
__global__ void __launch_bounds__(256)
momentum_kernel(float* __restrict__ m, const void* __restrict__ g, int32_t gdt, int64_t n, float mu,
                int32_t vec) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += stride) {
    if (vec && i + 4 <= n) {
      float gv[4];
      load_vec4(g, i, gdt, gv);
      f32x4 mv = *reinterpret_cast<const f32x4*>(m + i);
      f32x4 r;
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = fmaf(mu, mv[k], gv[k]);
      *reinterpret_cast<f32x4*>(m + i) = r;
    } else {
      for (int64_t k = i; k < i + 4 && k < n; ++k) m[k] = fmaf(mu, m[k], load_as_f32(g, k, gdt));
    }
  }
}

// w[i] <- w[i] - lr o[i] over n elements (w of dtype wdt, rounded once; o
// fp32); vec when w and o are aligned for 4-element accesses.
__global__ void __launch_bounds__(256)
update_kernel(void* __restrict__ w, int32_t wdt, const float* __restrict__ o, int64_t n, float lr, int32_t vec) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += stride) {
    if (vec && i + 4 <= n) {
      float wv[4];
      load_vec4(w, i, wdt, wv);
      const f32x4 ov = *reinterpret_cast<const f32x4*>(o + i);
#pragma unroll
      for (int k = 0; k < 4; ++k) wv[k] = fmaf(-lr, ov[k], wv[k]);
      store_vec4(w, i, wdt, wv);
    } else {
      for (int64_t k = i; k < i + 4 && k < n; ++k) store_from_f32(w, k, wdt, fmaf(-lr, o[k], load_as_f32(w, k, wdt)));
    }
  }
}

}  // namespace msign
