// Kernels of the improved initial normalisation: they read the acc^2
// slots that the first A A product launch leaves in GemmParams::sumsq.
#pragma once

#include "gemm_nt.hpp"

namespace msign {

// Improved initial normalisation ("msign算子的Newton-Schulz迭代（上）"
// §改良初值): after the first A = X X^T and A2 = A A, the iterate is divided
// by s = (||A2||_F^2 + eps)^(1/8), the fourth root of ||(X X^T)^2||_F.
//
// init_scale_kernel: one block per matrix adds that matrix's acc^2 slots of
// the A A launch `q` (the slot layout of GemmParams::sumsq, `slots` per
// tile, padding blocks of the folded triangle skipped) in a fixed order and
// writes scales[4 bz + k] = s^-(1, 2, 4)[k].  With `nscale` (the first
// update reads the un-normalised input), scales[4 bz] is s^-1 nscale[4 bz + 1].
__global__ void __launch_bounds__(256)
init_scale_kernel(const GemmParams q, int32_t slots, float eps, float* scales, const float* nscale) {
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  float acc = 0.f;
  for (int64_t i = tid; i < (int64_t)q.tpm * slots; i += 256) {
    const int L = (int)(b * q.tpm + i / slots);
    int64_t bz;
    int ti, tj;
    if (tile_of<true>(q, L, bz, ti, tj)) acc += q.sumsq[(int64_t)L * slots + i % slots];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  __shared__ float ws[4];
  if ((tid & 63) == 0) ws[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    const float sum = ((ws[0] + ws[1]) + ws[2]) + ws[3];
    const float s = sqrtf(sqrtf(sqrtf(sum + eps)));
    const float r = 1.f / s;
    scales[4 * b] = nscale != nullptr ? r * nscale[4 * b + 1] : r;
    scales[4 * b + 1] = r * r;
    scales[4 * b + 2] = (r * r) * (r * r);
    scales[4 * b + 3] = 0.f;
  }
}

// B <- (b s^-2) A + (c s^-4) B over `per` elements (a multiple of 4) of each
// matrix: the first B = b A + c A2 of the normalised iterate, with A2 held
// in B.  Four consecutive elements per thread.
__global__ void __launch_bounds__(256)
init_combine_kernel(const void* A, void* B, int64_t per, int32_t dt, float b, float c,
                    const float* scales) {
  const int64_t bz = blockIdx.y;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= per) return;
  const float fa = b * scales[4 * bz + 1], fb = c * scales[4 * bz + 2];
  const int64_t base = bz * per + e;
  float va[4], vb[4], w[4];
  load_vec4(A, base, dt, va);
  load_vec4(B, base, dt, vb);
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = fa * va[k] + fb * vb[k];
  store_vec4(B, base, dt, w);
}

}  // namespace msign
