// MFMA tile kernel for every matrix product of the iteration (gfx950).
//
// Computes, per matrix of a batch,
//     C = alpha * P Q^T + beta * D + diag * I
// with P (M x K) and Q (N x K) both row-major, i.e. both operands are read
// along K.  Every product of the method is brought to this form:
//   X X^T                  P = Q = X                    ("Newton-Schulz" A)
//   c A A + b A            P = Q = A, D = A             (A is symmetric)
//   B X + a X              P = B, Q = X^T, D = X        (rectangular step)
//   Gram R R, Q Z, R Z ... P, Q symmetric, so Q^T = Q
// The n x n products are symmetric, so in triangle mode (TRI) only tiles with
// ti <= tj are launched; each is stored normally and its transpose is stored
// into the mirrored tile (the flash-muon X X^T operator on nil9.net computes
// upper tiles and stores transposed copies into the lower ones; "Gram
// Newton-Schulz" §4 uses a triangular scheduler and the fused form
// C <- aAB + bC + gI).  In a diagonal tile only elements with i <= j are
// kept, so C is bitwise symmetric.
//
// Data path: 16-byte global loads of 128-byte K slices into registers, then
// into a double-buffered LDS tile whose 16-byte chunks are XOR-swizzled by
// row (conflict-free ds_read_b128 for the MFMA fragments); one barrier per
// K slice.  bf16/f16 use v_mfma_f32_16x16x32_{bf16,f16} (one 16-byte fragment
// per lane per MFMA); fp32 uses v_mfma_f32_16x16x4_f32, four per fragment.
// The K order inside a fragment is the same for both operands, so the
// product does not depend on the hardware's K lane assignment.
// Accumulator layout of the 16x16 MFMA: lane l, register r holds
// C[4 * (l / 16) + r][l % 16].
//
// The epilogue works in fp32 on the accumulator: alpha*acc + beta*D (D read
// through its transpose Dt[j][i], four consecutive values per lane), plus a
// per-output diagonal term, then up to three stores of different dtype and
// orientation (normal C[i][j] or transposed C[j][i]).
#pragma once

#include "common.hpp"

namespace msign {

#define MSIGN_MAX_OUT 3

struct OutSpec {
  void* ptr;
  int64_t ld;        // row pitch (elements) of the destination
  int64_t bstride;   // batch stride (elements)
  int32_t dtype;
  int32_t transposed;  // full mode: store C[i][j] at ptr[j * ld + i]
  int32_t rows_lim;    // store only i < rows_lim and j < cols_lim
  int32_t cols_lim;
  float diag;          // added where i == j and i < diag_lim
  int32_t diag_lim;
  int32_t vec_ok;      // 4 consecutive transposed elements may be one store
};

struct GemmParams {
  const void* P; int64_t ldp, sp;
  const void* Q; int64_t ldq, sq;
  int32_t M, N, K;     // load bounds; K a multiple of 16 bytes of elements
  float alpha, beta;
  const void* Dt; int64_t ldd, sd; int32_t d_dtype; int32_t d_vec_ok;
  OutSpec out[MSIGN_MAX_OUT];
  int32_t nout;
  int32_t tiles_m, tiles_n;
};

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  static __device__ __forceinline__ void run(f32x4& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mma<f16_t> {
  static __device__ __forceinline__ void run(f32x4& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x4& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a[e]),
                                                 __builtin_bit_cast(float, b[e]), acc, 0, 0, 0);
  }
};

__device__ __forceinline__ void store_elem(const OutSpec& os, int64_t bz, int64_t r, int64_t c, float v) {
  store_from_f32(os.ptr, bz * os.bstride + r * os.ld + c, os.dtype, v);
}

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

template <typename T, int BM, int BN, int WGM, int WGN, bool TRI>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_nt_kernel(const GemmParams p) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int ESZ = Elem<T>::size;
  constexpr int CE = 16 / ESZ;   // elements per 16-byte chunk
  constexpr int KTE = 8 * CE;    // elements per 128-byte K slice
  constexpr int ACH = BM * 8 / NT, BCH = BN * 8 / NT;
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile/thread mismatch");
  static_assert(!TRI || BM == BN, "triangle mode needs square tiles");

  __shared__ u32x4 lds[2][(BM + BN) * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t bz = blockIdx.z;

  int ti, tj;
  if constexpr (TRI) {
    int t = blockIdx.x, r = 0, rowlen = p.tiles_n;
    while (t >= rowlen) { t -= rowlen; ++r; --rowlen; }
    ti = r;
    tj = r + t;
  } else {
    ti = blockIdx.x % p.tiles_m;
    tj = blockIdx.x / p.tiles_m;
  }
  const int m0 = ti * BM, n0 = tj * BN;

  const char* Pb = static_cast<const char*>(p.P) + bz * p.sp * ESZ;
  const char* Qb = static_cast<const char*>(p.Q) + bz * p.sq * ESZ;

  u32x4 ra[ACH], rb[BCH];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  auto gload = [&](int k0) {
#pragma unroll
    for (int s = 0; s < ACH; ++s) {
      const int cid = tid + s * NT, row = cid >> 3, ch = cid & 7;
      const int gr = m0 + row, kk = k0 + ch * CE;
      ra[s] = (gr < p.M && kk < p.K)
                  ? *reinterpret_cast<const u32x4*>(Pb + ((int64_t)gr * p.ldp + kk) * ESZ)
                  : zero4;
    }
#pragma unroll
    for (int s = 0; s < BCH; ++s) {
      const int cid = tid + s * NT, row = cid >> 3, ch = cid & 7;
      const int gr = n0 + row, kk = k0 + ch * CE;
      rb[s] = (gr < p.N && kk < p.K)
                  ? *reinterpret_cast<const u32x4*>(Qb + ((int64_t)gr * p.ldq + kk) * ESZ)
                  : zero4;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int s = 0; s < ACH; ++s) {
      const int cid = tid + s * NT, row = cid >> 3, ch = cid & 7;
      lds[buf][row * 8 + (ch ^ (row & 7))] = ra[s];
    }
#pragma unroll
    for (int s = 0; s < BCH; ++s) {
      const int cid = tid + s * NT, row = cid >> 3, ch = cid & 7;
      lds[buf][(BM + row) * 8 + (ch ^ (row & 7))] = rb[s];
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = (p.K + KTE - 1) / KTE;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * KTE);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      u32x4 a[FM], b[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int row = wm * WM + fm * 16 + (lane & 15);
        a[fm] = lds[buf][row * 8 + (ch ^ (row & 7))];
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int row = wn * WN + fn * 16 + (lane & 15);
        b[fn] = lds[buf][(BM + row) * 8 + (ch ^ (row & 7))];
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) Mma<T>::run(acc[fm][fn], a[fm], b[fn]);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  const bool diag_tile = TRI && (ti == tj);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int i0 = m0 + wm * WM + fm * 16 + 4 * (lane >> 4);
      const int j = n0 + wn * WN + fn * 16 + (lane & 15);
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = p.alpha * acc[fm][fn][r];
      if (p.Dt != nullptr && j < p.N && i0 < p.M) {
        float d[4];
        const int64_t base = bz * p.sd + (int64_t)j * p.ldd + i0;
        if (p.d_vec_ok && i0 + 3 < p.M) {
          load_vec4(p.Dt, base, p.d_dtype, d);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) d[r] = (i0 + r < p.M) ? load_as_f32(p.Dt, base + r, p.d_dtype) : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += p.beta * d[r];
      }
      for (int o = 0; o < p.nout; ++o) {
        const OutSpec& os = p.out[o];
        float w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + r;
          w[r] = v[r] + ((i == j && i < os.diag_lim) ? os.diag : 0.f);
        }
        if (j >= os.cols_lim) continue;
        if (TRI || !os.transposed) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = i0 + r;
            if (i < os.rows_lim && (!diag_tile || i <= j)) store_elem(os, bz, i, j, w[r]);
          }
        }
        if (TRI || os.transposed) {
          // element (i, j) goes to ptr[j * ld + i]; in triangle mode this is the mirror
          const int64_t base = bz * os.bstride + (int64_t)j * os.ld + i0;
          if (os.vec_ok && !diag_tile && i0 + 3 < os.rows_lim) {
            store_vec4(os.ptr, base, os.dtype, w);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = i0 + r;
              if (i < os.rows_lim && (!diag_tile || i < j)) store_from_f32(os.ptr, base + r, os.dtype, w[r]);
            }
          }
        }
      }
    }
  }
}

}  // namespace msign
