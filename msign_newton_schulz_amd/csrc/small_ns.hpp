// Whole-iteration kernel for small matrices: standard Newton-Schulz
// ("msign算子的Newton-Schulz迭代（上）" §迭代计算, §参考实现) of one matrix per
// workgroup, every step in one launch.
//
// A problem of n x m (after the transpose of a tall input) with 64 < n <= 128
// and n m <= 32768 (padded: 128 x mp, mp <= 256) is bound by the latency of
// the 3 T dependent product launches of the tiled path, not by its flops
// (about 21 Mflop per step at 128 x 256).  Here one workgroup of 16 waves
// keeps everything on one CU:
//   - the fp32 iterate X in registers, 32 values per lane, laid out as the
//     MFMA output of the B X product (wave w owns rows 32 (w / 4) .. + 31 and
//     columns 64 (w % 4) .. + 63 of the 128 x 256 padded X);
//   - its compute-dtype copy Xh (128 x mp) and A, B (128 x 128) in LDS, rows
//     padded by 16 bytes (conflict-free 16-byte fragment reads).
// Per step, separated by barriers:
//   A = Xh Xh^T      (every 32 x 32 tile, K = mp), stored in the compute dtype;
//   B = c A A + b A  (A symmetric: A A = A A^T, K = 128);
//   X <- a X + B X   (B rows against Xh read K-major with transpose reads, the
//                     a X term from the fp32 registers), then Xh <- X.
// Products run on v_mfma_f32_16x16x32_{bf16,f16} with fp32 accumulation,
// in the same precision scheme as the tiled path (fp32 iterate, operands
// rounded once).  Zero padding (rows past n, columns past m) stays zero.
#pragma once

#include "gemm_nt.hpp"

namespace msign {

constexpr int kSmallN = 128;           // padded n of the small kernel
constexpr int kSmallMaxM = 256;        // largest padded m
constexpr int kSmallThreads = 1024;    // 16 waves
constexpr int kSmallXPitch = kSmallMaxM * 2 + 16;  // bytes per Xh row
constexpr int kSmallAPitch = kSmallN * 2 + 16;     // bytes per A / B row

struct SmallNsParams {
  const void* x;
  void* y;
  int32_t rows, cols;     // input dims (the matrix b at x + b rows cols)
  int32_t n, m, mp;       // wide view: n <= m, mp = m padded to 64
  int32_t tall;           // X = M^T
  int32_t io_dtype;
  int32_t steps;
  float eps;
  float abc[MSIGN_MAX_STEPS][3];
};

template <typename T>
__global__ void __launch_bounds__(kSmallThreads)
small_ns_kernel(const SmallNsParams p) {
  // the coefficient table is indexed by the runtime step: read it in place
  // from the kernel-argument segment (indexing the by-value argument would
  // copy it to scratch memory)
  const SmallNsParams& P = *(const SmallNsParams*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int XB = kSmallXPitch, AB = kSmallAPitch;
  __shared__ __attribute__((aligned(16))) unsigned char xs[kSmallN * XB];
  __shared__ __attribute__((aligned(16))) unsigned char as[kSmallN * AB];
  __shared__ __attribute__((aligned(16))) unsigned char bs[kSmallN * AB];
  __shared__ float red[16];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t bz = blockIdx.x;
  const int esz = p.io_dtype == DT_F32 ? 4 : 2;
  const char* xin = static_cast<const char*>(p.x) + bz * (int64_t)p.rows * p.cols * esz;

  // element (j, i) of X: input M[j][i] (wide) or M[i][j] (tall)
  auto in_index = [&](int j, int i) -> int64_t {
    return p.tall ? (int64_t)i * p.cols + j : (int64_t)j * p.cols + i;
  };
  // This lane's 32 iterate values: fragment (fj, fi) of the wave's 32 x 64
  // tile, register r holds X[j0 + 16 fj + 4 g + r][i0 + 16 fi + l16].
  const int j0 = 32 * (w >> 2), i0 = 64 * (w & 3);
  float x32[2][4][4];
  float ss = 0.f;
#pragma unroll
  for (int fj = 0; fj < 2; ++fj)
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 16 * fj + 4 * g + r, i = i0 + 16 * fi + l16;
        float v = 0.f;
        if (j < p.n && i < p.m) v = load_as_f32(xin, in_index(j, i), p.io_dtype);
        x32[fj][fi][r] = v;
        ss += v * v;
      }
  // Frobenius norm: fixed-order wave and block sums
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) tot += red[k];
  const float scale = 1.0f / sqrtf(tot + p.eps);

  auto store_h = [&](unsigned char* base, int pitch, int row, int col, float v) {
    const uint16_t h = Elem<T>::dt == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
    *reinterpret_cast<uint16_t*>(base + row * pitch + col * 2) = h;
  };
  auto load_h = [&](const unsigned char* base, int pitch, int row, int col) -> float {
    const uint16_t h = *reinterpret_cast<const uint16_t*>(base + row * pitch + col * 2);
    return Elem<T>::dt == DT_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
  };
  // Xh <- X (every lane writes its 32 values; with the zero padding they
  // cover the whole 128 x 256 extent)
  auto write_xh = [&]() {
#pragma unroll
    for (int fj = 0; fj < 2; ++fj)
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store_h(xs, XB, j0 + 16 * fj + 4 * g + r, i0 + 16 * fi + l16, x32[fj][fi][r]);
  };
#pragma unroll
  for (int fj = 0; fj < 2; ++fj)
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int r = 0; r < 4; ++r) x32[fj][fi][r] *= scale;
  write_xh();
  __syncthreads();

  // 16-byte fragment: row `row` of a row-major LDS matrix, 8 elements from
  // column 8 * chunk
  auto frag = [&](const unsigned char* base, int pitch, int row, int chunk) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(base + row * pitch + chunk * 16);
  };
  // n x n tile of wave w: rows 32 (w / 4), columns 32 (w % 4)
  const int ta = 32 * (w >> 2), tb = 32 * (w & 3);

  for (int t = 0; t < p.steps; ++t) {
    const float a = P.abc[t][0], b = P.abc[t][1], c = P.abc[t][2];
    {  // A = Xh Xh^T
      f32x4 acc[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) acc[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kk = 0; kk < p.mp / 32; ++kk) {
        const int ch = 4 * kk + g;
        u32x4 fa[2], fb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          fa[u] = frag(xs, XB, ta + 16 * u + l16, ch);
          fb[u] = frag(xs, XB, tb + 16 * u + l16, ch);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int v = 0; v < 2; ++v) Mma<T>::run(acc[u][v], fa[u], fb[v]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r) store_h(as, AB, ta + 16 * u + 4 * g + r, tb + 16 * v + l16, acc[u][v][r]);
    }
    __syncthreads();
    {  // B = c A A + b A
      f32x4 acc[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) acc[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kSmallN / 32; ++kk) {
        const int ch = 4 * kk + g;
        u32x4 fa[2], fb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          fa[u] = frag(as, AB, ta + 16 * u + l16, ch);
          fb[u] = frag(as, AB, tb + 16 * u + l16, ch);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int v = 0; v < 2; ++v) Mma<T>::run(acc[u][v], fa[u], fb[v]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = ta + 16 * u + 4 * g + r, col = tb + 16 * v + l16;
            store_h(bs, AB, row, col, c * acc[u][v][r] + b * load_h(as, AB, row, col));
          }
    }
    __syncthreads();
    {  // X <- a X + B X: rows j from B, columns i of X read K-major
      f32x4 acc[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kSmallN / 32; ++kk) {
        u32x4 fa[2], fb[4];
#pragma unroll
        for (int u = 0; u < 2; ++u) fa[u] = frag(bs, AB, j0 + 16 * u + l16, 4 * kk + g);
        // transpose reads: lane (g, l16) points at K row 32 kk + 8 g + l16 / 4
        // (and that + 4), columns i + 4 (l16 % 4) .. + 3; afterwards it holds
        // column i + l16 at K rows 32 kk + 8 g + 0..7
        const int k0r = 32 * kk + 8 * g + (l16 >> 2);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int col = i0 + 16 * v + 4 * (l16 & 3);
          fb[v] = lds_read_tr16_pair(xs, k0r * XB + col * 2, (k0r + 4) * XB + col * 2);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) Mma<T>::run(acc[u][v], fa[u], fb[v]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r) x32[u][v][r] = fmaf(a, x32[u][v][r], acc[u][v][r]);
    }
    if (t + 1 < p.steps) {
      __syncthreads();  // every read of Xh and B done
      write_xh();
      __syncthreads();
    }
  }

  // y (io dtype, input orientation)
  char* yout = static_cast<char*>(p.y) + bz * (int64_t)p.rows * p.cols * esz;
#pragma unroll
  for (int fj = 0; fj < 2; ++fj)
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 16 * fj + 4 * g + r, i = i0 + 16 * fi + l16;
        if (j < p.n && i < p.m) store_from_f32(yout, in_index(j, i), p.io_dtype, x32[fj][fi][r]);
      }
}

}  // namespace msign
