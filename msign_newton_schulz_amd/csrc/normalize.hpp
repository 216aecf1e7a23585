// Frobenius normalisation X0 = X / sqrt(sum X^2 + eps) ("msign算子的
// Newton-Schulz迭代（上）" §迭代计算 and §参考实现), in two HBM-bound passes:
//
//  1. sumsq_partial_kernel: grid (nblk, batch).  Each block squares and sums
//     one contiguous slice of one matrix in fp32 (16-byte loads when
//     aligned), reduces across the block with a fixed shuffle tree and writes
//     one partial.  Fixed slice boundaries and trees make the sum bit-stable.
//  2. normalize_kernel: grid (64x64 tiles of the padded input, batch).  Each
//     block re-sums that matrix's partials in a fixed order, forms the scale
//     1/sqrt(sum + eps) in fp32, loads its input tile into LDS (16-byte loads
//     when the input's rows allow), and writes every requested copy of the
//     scaled tile: in the input's orientation or transposed (read back
//     column-wise from LDS), in fp32 or the compute dtype, four consecutive
//     elements per store.  Tiles cover the padded extents (multiples of 64),
//     so padding rows and columns of every copy are written as zeros.
//     A null partial pointer means scale 1 (a plain cast/transpose/pad).
#pragma once

#include "common.hpp"

namespace msign {

struct NormOut {
  void* ptr;
  int64_t ld;
  int64_t bstride;
  int32_t dtype;
  int32_t transposed;  // relative to the input's orientation
};

struct NormParams {
  const void* x;
  int32_t x_dtype;
  int64_t rows, cols;           // true input dims; batch stride rows * cols
  int32_t rows_pad, cols_pad;   // extent covered (input orientation)
  const float* partial;         // [batch][nblk] or null (scale 1)
  int32_t nblk;
  float eps;
  NormOut out[3];
  int32_t nout;
};

// MOM (a Muon step's momentum, folded into this pass): x is the fp32
// momentum M, updated in place to fmaf(mu, M, G) (G of dtype gdt, the same
// layout), and the sum is taken over the updated values.  Every element is
// read and written by one thread only.
template <int NT, bool MOM = false>
__global__ void __launch_bounds__(NT)
sumsq_partial_kernel(const void* x, int32_t dt, int64_t count, int32_t nblk, float* partial,
                     const void* g = nullptr, int32_t gdt = DT_F32, float mu = 0.f) {
  const int64_t b = blockIdx.y;
  const int tid = threadIdx.x;
  const int esz = dt == DT_F32 ? 4 : 2;
  const char* base = static_cast<const char*>(x) + b * count * esz;
  const int64_t chunk = (((count + nblk - 1) / nblk) + 7) & ~(int64_t)7;
  const int64_t start = (int64_t)blockIdx.x * chunk;
  const int64_t end = start + chunk < count ? start + chunk : count;

  float s = 0.f;
  if constexpr (MOM) {
    float* m = reinterpret_cast<float*>(const_cast<char*>(base));
    const char* gb = static_cast<const char*>(g) + b * count * (gdt == DT_F32 ? 4 : 2);
    if (start < end) {
      const bool aligned = ((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(gb)) & 15) == 0;
      int64_t done = start;
      if (aligned) {
        const int64_t nvec = (end - start) / 4;
        for (int64_t v = tid; v < nvec; v += NT) {
          const int64_t e = start + v * 4;
          float gv[4];
          load_vec4(gb, e, gdt, gv);
          f32x4 mv = *reinterpret_cast<const f32x4*>(m + e);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            mv[q] = fmaf(mu, mv[q], gv[q]);
            s += mv[q] * mv[q];
          }
          *reinterpret_cast<f32x4*>(m + e) = mv;
        }
        done = start + nvec * 4;
      }
      for (int64_t e = done + tid; e < end; e += NT) {
        const float f = fmaf(mu, m[e], load_as_f32(gb, e, gdt));
        m[e] = f;
        s += f * f;
      }
    }
  } else if (start < end) {
    const bool aligned = (reinterpret_cast<uintptr_t>(base) & 15) == 0;
    int64_t done = start;
    if (aligned) {
      // 8 elements per 16-byte (or two, fp32) load; each thread keeps U
      // loads in flight before summing them (in a fixed order)
      constexpr int U = 4;
      const int64_t nvec = (end - start) / 8;
      auto sum8 = [&](const u32x4& u, const u32x4& w) {
        float t = 0.f;
        if (dt == DT_F32) {
          const f32x4 fu = __builtin_bit_cast(f32x4, u), fw = __builtin_bit_cast(f32x4, w);
#pragma unroll
          for (int q = 0; q < 4; ++q) t += fu[q] * fu[q] + fw[q] * fw[q];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint16_t lo = u[q] & 0xffff, hi = u[q] >> 16;
            const float f0 = dt == DT_BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
            const float f1 = dt == DT_BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
            t += f0 * f0 + f1 * f1;
          }
        }
        return t;
      };
      auto load8 = [&](int64_t v, u32x4& u, u32x4& w) {
        const int64_t e = start + v * 8;
        if (dt == DT_F32) {
          const u32x4* pv = reinterpret_cast<const u32x4*>(base + e * 4);
          u = pv[0];
          w = pv[1];
        } else {
          u = *reinterpret_cast<const u32x4*>(base + e * 2);
        }
      };
      int64_t v = tid;
      for (; v + (U - 1) * NT < nvec; v += U * NT) {
        u32x4 u[U], w[U];
#pragma unroll
        for (int k = 0; k < U; ++k) load8(v + k * NT, u[k], w[k]);
#pragma unroll
        for (int k = 0; k < U; ++k) s += sum8(u[k], w[k]);
      }
      for (; v < nvec; v += NT) {
        u32x4 u, w;
        load8(v, u, w);
        s += sum8(u, w);
      }
      done = start + nvec * 8;
    }
    for (int64_t e = done + tid; e < end; e += NT) {
      const float f = load_as_f32(base, e, dt);
      s += f * f;
    }
  }
  // fixed-order block reduction
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  __shared__ float ws[NT / 64];
  if ((tid & 63) == 0) ws[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < NT / 64; ++w) t += ws[w];
    partial[b * nblk + blockIdx.x] = t;
  }
}

// Per-matrix factors of a normalisation left to the products: one block
// per matrix adds its partial sums in a fixed order and writes
// out[4 b] = 1 / (sum + eps) and out[4 b + 1] = 1 / sqrt(sum + eps), the
// factors of X X^T and of X in the first products of the iteration.
__global__ void __launch_bounds__(256)
norm_scale_kernel(const float* partial, int32_t nblk, float eps, float* out) {
  __shared__ float wsum[4];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int i = tid; i < nblk; i += 256) s += partial[b * nblk + i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    const float r = 1.0f / sqrtf(((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) + eps);
    out[4 * b] = r * r;
    out[4 * b + 1] = r;
    out[4 * b + 2] = 0.f;
    out[4 * b + 3] = 0.f;
  }
}

__global__ void __launch_bounds__(256)
normalize_kernel(const NormParams p) {
  __shared__ float tile[64][65];
  __shared__ float s_scale;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  if (tid < 64) {
    float scale = 1.f;
    if (p.partial != nullptr) {
      float s = 0.f;
      for (int i = tid; i < p.nblk; i += 64) s += p.partial[b * p.nblk + i];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
      scale = 1.0f / sqrtf(s + p.eps);
    }
    if (tid == 0) s_scale = scale;
  }
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int64_t xb = b * p.rows * p.cols;
  const bool wide16 = p.x_dtype != DT_F32;
  const int per_chunk = wide16 ? 8 : 4;  // elements per 16-byte chunk
  const bool vec_in = (p.cols % per_chunk) == 0 &&
                      (reinterpret_cast<uintptr_t>(p.x) & 15) == 0;
  if (vec_in) {
    // rows hold whole chunks: a chunk is either inside the matrix or not
    const int cpr = 64 / per_chunk;
    for (int q = tid; q < 64 * cpr; q += 256) {
      const int rr = q / cpr, cc = (q % cpr) * per_chunk;
      const int64_t r = r0 + rr, c = c0 + cc;
      float v[8];
      if (r < p.rows && c < p.cols) {
        const int64_t e = xb + r * p.cols + c;
        if (wide16) {
          const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.x) + e);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint16_t lo = u[k] & 0xffff, hi = u[k] >> 16;
            v[2 * k] = p.x_dtype == DT_BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo);
            v[2 * k + 1] = p.x_dtype == DT_BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi);
          }
        } else {
          const f32x4 u = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.x) + e);
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = u[k];
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.f;
      }
      for (int k = 0; k < per_chunk; ++k) tile[rr][cc + k] = v[k];
    }
  } else {
    const int tx = tid & 63, ty = tid >> 6;
    for (int rr = ty; rr < 64; rr += 4) {
      const int64_t r = r0 + rr, c = c0 + tx;
      tile[rr][tx] = (r < p.rows && c < p.cols) ? load_as_f32(p.x, xb + r * p.cols + c, p.x_dtype) : 0.f;
    }
  }
  __syncthreads();
  const float sc = s_scale;
  for (int o = 0; o < p.nout; ++o) {
    const NormOut& os = p.out[o];
    // quad q: row (or, transposed, column) q / 16 of the tile, 4 elements
    // starting at 4 (q % 16) along the other index
    for (int q = tid; q < 1024; q += 256) {
      const int u = q >> 4, w0 = (q & 15) * 4;
      float v[4];
      int64_t base;
      bool inside;
      if (!os.transposed) {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = tile[u][w0 + k] * sc;
        base = b * os.bstride + (int64_t)(r0 + u) * os.ld + c0 + w0;
        inside = r0 + u < p.rows_pad && c0 + w0 + 3 < p.cols_pad;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = tile[w0 + k][u] * sc;
        base = b * os.bstride + (int64_t)(c0 + u) * os.ld + r0 + w0;
        inside = c0 + u < p.cols_pad && r0 + w0 + 3 < p.rows_pad;
      }
      if (inside) store_vec4(os.ptr, base, os.dtype, v);
    }
  }
}

// normalize_direct_kernel: the same normalisation when no output is
// transposed and the input rows hold whole 16-byte chunks (every wide
// input).  No LDS tile: each thread scales 8 consecutive elements of a row
// straight from its load into its stores; a block covers 64 rows x 256
// columns of the padded extent (zeros past the input).  The scale comes from
// the matrix's partial sums, added by all 256 threads in a fixed order.
__global__ void __launch_bounds__(256)
normalize_direct_kernel(const NormParams p) {
  __shared__ float wsum[4];
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  float sc = 1.f;
  if (p.partial != nullptr) {
    float s = 0.f;
    for (int i = tid; i < p.nblk; i += 256) s += p.partial[b * p.nblk + i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if ((tid & 63) == 0) wsum[tid >> 6] = s;
    __syncthreads();
    sc = 1.0f / sqrtf(((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) + p.eps);
  }
  const int64_t xb = b * p.rows * p.cols;
  const int c = blockIdx.x * 256 + (tid & 31) * 8;  // first of this thread's 8 columns
  if (c >= p.cols_pad) return;
  for (int rr = tid >> 5; rr < 64; rr += 8) {
    const int64_t r = (int64_t)blockIdx.y * 64 + rr;
    if (r >= p.rows_pad) break;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.f;
    if (r < p.rows) {
      const int64_t e = xb + r * p.cols + c;
      if (p.x_dtype != DT_F32) {
        if (c < p.cols) {  // cols is a multiple of 8: the chunk is whole
          const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.x) + e);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint16_t lo = u[k] & 0xffff, hi = u[k] >> 16;
            v[2 * k] = (p.x_dtype == DT_BF16 ? bf16_bits_to_f32(lo) : f16_bits_to_f32(lo)) * sc;
            v[2 * k + 1] = (p.x_dtype == DT_BF16 ? bf16_bits_to_f32(hi) : f16_bits_to_f32(hi)) * sc;
          }
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (c + 4 * h < p.cols) {  // cols is a multiple of 4
            const f32x4 u = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.x) + e + 4 * h);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[4 * h + k] = u[k] * sc;
          }
      }
    }
    for (int o = 0; o < p.nout; ++o) {
      const NormOut& os = p.out[o];
      const int64_t base = b * os.bstride + r * os.ld + c;
      store_vec4(os.ptr, base, os.dtype, v);
      store_vec4(os.ptr, base + 4, os.dtype, v + 4);
    }
  }
}

}  // namespace msign
