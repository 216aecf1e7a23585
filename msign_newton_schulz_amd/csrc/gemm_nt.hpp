// MFMA tile kernel for every matrix product of the iteration (gfx950).
//
// Computes, per matrix of a batch,
//     C = alpha * P Q^T + beta * D + diag * I
// with P (M x K) and Q (N x K) both row-major, i.e. both operands are read
// along K.  Every product of the method is brought to this form:
//   X X^T                  P = Q = X                    ("Newton-Schulz" A)
//   c A A + b A            P = Q = A, D = A             (A is symmetric)
//   B X + a X              computed as X^T B + a X^T: P = X read K-major
//                          (AT), Q = B (symmetric), D = X, stored transposed
//   Gram R R, Q Z, R Z ... P, Q symmetric, so Q^T = Q
// The n x n products are symmetric, so in triangle mode (TRI) only tiles with
// ti <= tj are launched; each is stored normally and its transpose is stored
// into the mirrored tile (the flash-muon X X^T operator on nil9.net computes
// upper tiles and stores transposed copies into the lower ones; "Gram
// Newton-Schulz" §4 uses a triangular scheduler and the fused form
// C <- aAB + bC + gI).  In a diagonal tile only elements with i <= j are
// kept, so C is bitwise symmetric.
//
// Data path: 128-byte (256 x 256 tiles) or 64-byte (128 x 128) K slices go
// from global memory straight into a double-buffered LDS tile (buffer_load
// ... lds); the 64 x 64 tier stages them through registers.  The tile's
// 16-byte chunks are XOR-swizzled by row (conflict-free ds_read_b128 for the
// MFMA fragments; K-major operands are read back with ds_read_b64_tr_b16);
// one barrier per K slice.  bf16/f16 use v_mfma_f32_16x16x32_{bf16,f16} (one 16-byte fragment
// per lane per MFMA); fp32 uses v_mfma_f32_16x16x4_f32, four per fragment.
// The K order inside a fragment is the same for both operands, so the
// product does not depend on the hardware's K lane assignment.
// Accumulator layout of the 16x16 MFMA: lane l, register r holds
// C[4 * (l / 16) + r][l % 16].
//
// The epilogue works in fp32 on the accumulator: fma(alpha, acc, beta*D),
// written out so that every epilogue path rounds alike (D read
// through its transpose Dt[j][i], four consecutive values per lane), plus a
// per-output diagonal term, then up to three stores of different dtype and
// orientation (normal C[i][j] or transposed C[j][i]).
#pragma once

#include "common.hpp"

#include <type_traits>
#include <utility>

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
  int32_t update;      // 0: store the value v; 1: update in place, out <- out + axpy v
  float axpy;
};

struct GemmParams {
  const void* P; int64_t ldp, sp;
  const void* Q; int64_t ldq, sq;
  int32_t M, N, K;     // load bounds; K a multiple of 64 elements
  float alpha, beta;
  const void* Dt; int64_t ldd, sd; int32_t d_dtype; int32_t d_vec_ok;
  OutSpec out[MSIGN_MAX_OUT];
  int32_t nout;
  int32_t tiles_m, tiles_n;
  // Blocks enumerate tiles over the whole batch (tpm tiles per matrix).  The
  // first nfull tiles are computed whole; each later tile is split along K
  // into `split` parts whose fp32 sums go to `partial` and are added in a
  // fixed order by gemm_nt_reduce_kernel.
  int32_t tpm, nfull, split;
  float* partial;
  // Optional per-matrix factor computed on the device: every value
  // (alpha acc + beta D) is multiplied by vscale[4 bz].
  const float* vscale;
  // K-major P (AT) only: rows of P that exist (0: all K); rows from kvalid
  // up to K read as zeros.
  int32_t kvalid;
  // Optional, triangle products: sums of acc^2 over each tile (off-diagonal
  // tiles counted twice, for their mirror), one per (tile, wave, fragment
  // row) at sumsq[((bz tpm + tile) WG + wave) FM + fm]; the slots of the
  // padding blocks of the folded triangle are not written.
  float* sumsq;
};

// One launch may cover up to kMaxGroups problems of one product kind
// and tile configuration (a grouped launch): group g owns the blocks from
// bstart[g] up to the next group's first block, and numbers its tiles, its
// K split and its partial sums on its own.  Unused entries have bstart =
// INT32_MAX.  A single product is launched with a one-entry table (NG = 1:
// the kernel argument stays small and there is no lookup).
constexpr int kMaxGroups = 4;

template <int NG>
struct GemmGroups {
  GemmParams g[NG];
  int32_t bstart[NG];
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
  // Bit-cast the whole fragment first: a bit_cast of one vector element
  // does not select that element.
  static __device__ __forceinline__ void run(f32x4& acc, const u32x4& a, const u32x4& b) {
    const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[e], fb[e], acc, 0, 0, 0);
  }
};

// Element idx of output os gets v, or (an update output) out + axpy v in
// fp32, rounded once to the output's dtype.  UPD: the kernel may have
// update outputs (rectangular products only: the last product of a fused
// Muon step); triangle kernels compile without the branch.
template <bool UPD>
__device__ __forceinline__ void out_elem(const OutSpec& os, int64_t idx, float v) {
  if (UPD && os.update) v = fmaf(os.axpy, v, load_as_f32(os.ptr, idx, os.dtype));
  store_from_f32(os.ptr, idx, os.dtype, v);
}

// The same for four consecutive elements idx .. idx + 3 (one vector access).
template <bool UPD>
__device__ __forceinline__ void out_vec4(const OutSpec& os, int64_t idx, const float* w) {
  if (UPD && os.update) {
    float o[4];
    load_vec4(os.ptr, idx, os.dtype, o);
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = fmaf(os.axpy, w[r], o[r]);
    store_vec4(os.ptr, idx, os.dtype, o);
  } else {
    store_vec4(os.ptr, idx, os.dtype, w);
  }
}

template <bool UPD>
__device__ __forceinline__ void store_elem(const OutSpec& os, int64_t bz, int64_t r, int64_t c, float v) {
  out_elem<UPD>(os, bz * os.bstride + r * os.ld + c, v);
}

// 16-byte chunk position inside an LDS row of CPR chunks: XOR swizzle so
// that the 16 lanes reading one fragment column (16 consecutive rows, same
// logical chunk) hit distinct bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int row, int ch) {
  if constexpr (CPR == 8) return ch ^ (row & 7);
  else return ch ^ ((row >> 1) & 3);
}

// 16-byte chunk position inside a row of a K-major ("transposed") A tile,
// [k][m] with m contiguous.  A transpose read of 16-bit data fetches, per
// half-wave, K rows k0..k0+3 and k0+8..k0+11 (k0 a multiple of 4) x 32
// bytes; XOR-ing the chunk pair index with bits 0, 1 and 3 of k puts those
// 8 rows on 8 distinct 32-byte bank groups (rows of 8 chunks only allow
// bits 0 and 1).  The fp32 reads fetch 4 groups of rows 4 apart x 64 bytes.
// CPRA: chunks per row (at least 8 for 16-bit, 16 for fp32).
template <int ESZ, int CPRA>
__device__ __forceinline__ int swz_t(int k, int ch) {
  if constexpr (ESZ == 2 && CPRA >= 16) return ch ^ (((k & 3) | ((k >> 1) & 4)) << 1);
  else if constexpr (ESZ == 2) return ch ^ ((k & 3) << 1);
  else return ch ^ (((k >> 2) & 3) << 2);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define MSIGN_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Two LDS transpose reads (ds_read_b64_tr_b16) at byte offsets off0 and off1
// of an LDS tile, concatenated into one 16-byte MFMA fragment.  Per 16-lane
// group, lanes 4b .. 4b + 3 point at K row b, columns 0, 4, 8, 12; after the
// read, lane j holds column j at K rows 0..3.
__device__ __forceinline__ u32x4 lds_read_tr16_pair(const void* tile, int off0, int off1) {
  const char* base = static_cast<const char*>(tile);
  const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + off0));
  const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + off1));
  const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
  return u32x4{w0[0], w0[1], w1[0], w1[1]};
}

// Buffer descriptor over `bytes` bytes at `base`: loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2; renumber so that every XCD works on one contiguous range of tiles.
__device__ __forceinline__ int xcd_contiguous(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7, l = b >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + l;
}

// Wait for every load and LDS access of this wave, then the workgroup
// barrier.  The wait is the compiler's own s_waitcnt (not inline asm), so
// its waitcnt pass knows that nothing is in flight after it; the empty asm
// before it keeps earlier memory accesses on its near side, the barrier's
// asm keeps later ones after it.
__device__ __forceinline__ void wait_all_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("s_barrier" ::: "memory");
}

// f(integral_constant<int, I>) for I = 0 .. N - 1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Tile coordinates of linear tile L over the batch: matrix bz, tile
// (ti, tj).  Rectangular grids are walked in groups of GM tile rows, column
// by column, so that concurrently running tiles share operand strips in L2.
// The upper triangle of a Tv x Tv grid (Tv = T rounded up to even) is folded
// into a Tv/2 x (Tv+1) rectangle: folded row f holds tile row f (Tv - f
// tiles) followed by tile row Tv-1-f (f + 1 tiles).  Returns false for the
// virtual tiles that pad an odd T.
template <bool TRI>
__device__ __forceinline__ bool tile_of(const GemmParams& p, int L, int64_t& bz, int& ti, int& tj) {
  constexpr int GM = 8;
  bz = L / p.tpm;
  const int idx = L - (int)bz * p.tpm;
  if constexpr (TRI) {
    const int TT = p.tiles_n, Tv = TT + (TT & 1), H = Tv / 2, W = Tv + 1;
    const int per = GM * W, g = idx / per, first = g * GM;
    const int gm = H - first < GM ? H - first : GM;
    const int rr = idx - g * per;
    const int f = first + rr % gm, c = rr / gm;
    if (c < Tv - f) { ti = f; tj = f + c; }
    else { ti = Tv - 1 - f; tj = ti + (c - (Tv - f)); }
    return tj < TT;
  } else {
    const int tm = p.tiles_m;
    const int per = GM * p.tiles_n, g = idx / per, first = g * GM;
    const int gm = tm - first < GM ? tm - first : GM;
    const int rr = idx - g * per;
    ti = first + rr % gm;
    tj = rr / gm;
    return true;
  }
}

// Epilogue of one 16 x 16 fragment (fm, fn) of wave `wave` of a tile, from
// its fp32 accumulators in the MFMA lane layout (lane l, register r holds
// row 4 (l / 16) + r, column l % 16) and the four D values of those rows
// (already loaded): alpha*acc + beta*D, times the per-matrix factor if any,
// a per-output diagonal term, then each output's stores.  Triangle mode
// stores the tile and its mirror; in a diagonal tile only i <= j is kept.
// Returns this lane's sum of acc^2 over the fragment.
template <int BM, int BN, int WGM, int WGN, bool TRI>
__device__ __forceinline__ float epilogue_frag(const GemmParams& p, int64_t bz, int ti, int tj,
                                               int wave, int fm, int fn, const f32x4& a,
                                               const float (&d)[4]) {
  constexpr int WM = BM / WGM, WN = BN / WGN;
  const int lane = threadIdx.x & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  const int m0 = ti * BM, n0 = tj * BN;
  const bool diag_tile = TRI && (ti == tj);
  const int i0 = m0 + wm * WM + fm * 16 + 4 * (lane >> 4);
  const int j = n0 + wn * WN + fn * 16 + (lane & 15);
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = fmaf(p.alpha, a[r], p.beta * d[r]);
  if (p.vscale != nullptr) {
    const float f = p.vscale[4 * bz];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] *= f;
  }
  // constant output indices (a runtime index into the by-value kernel
  // argument would make the compiler copy the whole struct to scratch)
#pragma unroll
  for (int o = 0; o < MSIGN_MAX_OUT; ++o) {
    if (o >= p.nout) break;
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
        if (i < os.rows_lim && (!diag_tile || i <= j)) store_elem<!TRI>(os, bz, i, j, w[r]);
      }
    }
    if (TRI || os.transposed) {
      // element (i, j) goes to ptr[j * ld + i]; in triangle mode this is the mirror
      const int64_t base = bz * os.bstride + (int64_t)j * os.ld + i0;
      if (os.vec_ok && !diag_tile && i0 + 3 < os.rows_lim) {
        out_vec4<!TRI>(os, base, w);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + r;
          if (i < os.rows_lim && (!diag_tile || i < j)) out_elem<!TRI>(os, base + r, w[r]);
        }
      }
    }
  }
  return a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3];
}

// The D values (read through Dt[j][i], four consecutive i per lane) of NR
// fragment rows fm0.. of wave `wave`; zeros where there is no D or it is out
// of bounds.  When the tile lies inside D and rows allow vector loads, all
// NR * FN loads are issued before any is used (one round trip, not one per
// fragment); otherwise element loads with bounds checks.
template <int BM, int BN, int WGM, int WGN, int NR>
__device__ __forceinline__ void epilogue_load_d(const GemmParams& p, int64_t bz, int ti, int tj, int wave,
                                                int fm0, float (&d)[NR * (BN / WGN / 16)][4]) {
  constexpr int WM = BM / WGM, WN = BN / WGN, FN = WN / 16, NF = NR * FN;
  const int lane = threadIdx.x & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  const int m0 = ti * BM, n0 = tj * BN;
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) d[f][r] = 0.f;
  if (p.Dt == nullptr) return;
  auto base_of = [&](int f) {
    const int i0 = m0 + wm * WM + (fm0 + f / FN) * 16 + 4 * (lane >> 4);
    const int j = n0 + wn * WN + (f % FN) * 16 + (lane & 15);
    return bz * p.sd + (int64_t)j * p.ldd + i0;
  };
  if (p.d_vec_ok && m0 + BM <= p.M && n0 + BN <= p.N) {
    if (p.d_dtype == DT_F32) {
      f32x4 t[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) t[f] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.Dt) + base_of(f));
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) d[f][r] = t[f][r];
    } else {
      u32x2 t[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) t[f] = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.Dt) + base_of(f));
      const bool bf = p.d_dtype == DT_BF16;
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint16_t h = (uint16_t)(t[f][r >> 1] >> (16 * (r & 1)));
          d[f][r] = bf ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
        }
    }
    return;
  }
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int i0 = m0 + wm * WM + (fm0 + f / FN) * 16 + 4 * (lane >> 4);
    const int j = n0 + wn * WN + (f % FN) * 16 + (lane & 15);
    if (j < p.N) {
      const int64_t base = base_of(f);
#pragma unroll
      for (int r = 0; r < 4; ++r) d[f][r] = (i0 + r < p.M) ? load_as_f32(p.Dt, base + r, p.d_dtype) : 0.f;
    }
  }
}

// Epilogue of NR fragment rows fm0.. of wave `wave` (acc[f] is fragment
// (fm0 + f / FN, f % FN)); sq[k] gets this lane's acc^2 sum of row fm0 + k.
template <int BM, int BN, int WGM, int WGN, bool TRI, int NR>
__device__ __forceinline__ void epilogue_rows(const GemmParams& p, int64_t bz, int ti, int tj, int wave,
                                              int fm0, const f32x4 (&acc)[NR * (BN / WGN / 16)],
                                              float (&sq)[NR]) {
  constexpr int FN = BN / WGN / 16;
  float d[NR * FN][4];
  epilogue_load_d<BM, BN, WGM, WGN, NR>(p, bz, ti, tj, wave, fm0, d);
  // (compile-time loops: a runtime index into acc would put it in scratch)
  static_for<NR>([&](auto K) {
    constexpr int k = decltype(K)::value;
    sq[k] = 0.f;
    static_for<FN>([&](auto FNI) {
      constexpr int fn = decltype(FNI)::value;
      sq[k] += epilogue_frag<BM, BN, WGM, WGN, TRI>(p, bz, ti, tj, wave, fm0 + k, fn, acc[k * FN + fn],
                                                   d[k * FN + fn]);
    });
  });
}

// Sum of v over the wave (fixed butterfly, so bit-stable), stored by lane 0.
__device__ __forceinline__ void wave_sum_store(float v, float* dst) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) *dst = v;
}

// Slot of (tile L, wave, fragment row fm) among the acc^2 sums.
template <int BM, int WGM, int WGN>
__device__ __forceinline__ float* sumsq_slot(const GemmParams& p, int L, int wave, int fm) {
  return p.sumsq + ((int64_t)L * (WGM * WGN) + wave) * (BM / WGM / 16) + fm;
}

// Epilogue of a rectangular tile whose outputs are all stored transposed
// (C[i][j] at ptr[j ld + i]) with 4-wide stores and lie wholly in bounds.
// The MFMA lane layout gives each store instruction 16 rows j x 4 values:
// partial cache lines.  Instead each wave stages one 16-column group (16 j
// x its 64 i) at a time in its own LDS region (rows padded to 68 floats:
// conflict-free 16-byte writes and reads) and reads it back by rows, so 16
// lanes store one row's 64 consecutive i (256 bytes fp32, 128 bytes 16-bit)
// per instruction.  Returns false, having done nothing, when the tile does
// not qualify.  The LDS ring must be free (after the K loop's last barrier).
template <int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ bool epilogue_staged(const GemmParams& p, int64_t bz, int ti, int tj,
                                                const f32x4 (&acc)[BM / WGM / 16][BN / WGN / 16],
                                                int wave, float* stage) {
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 16, FN = WN / 16;
  constexpr int PITCH = 68;
  static_assert(WM == 64, "16 lanes x 4 values cover a row of the wave tile");
  const int m0 = ti * BM, n0 = tj * BN;
  if (p.nout < 1) return false;
#pragma unroll
  for (int o = 0; o < MSIGN_MAX_OUT; ++o) {
    if (o >= p.nout) break;
    const OutSpec& os = p.out[o];
    if (!os.transposed || !os.vec_ok || os.diag_lim > 0 || m0 + BM > os.rows_lim || n0 + BN > os.cols_lim)
      return false;
  }
  const bool has_d = p.Dt != nullptr;
  if (has_d && !(p.d_vec_ok && m0 + BM <= p.M && n0 + BN <= p.N)) return false;
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wm = wave / WGN, wn = wave % WGN;
  float* st = stage + wave * (16 * PITCH);
  const float f = p.vscale != nullptr ? p.vscale[4 * bz] : 1.f;
  static_for<FN>([&](auto FNI) {
    constexpr int fn = decltype(FNI)::value;
    const int jf = n0 + wn * WN + fn * 16;  // first j of the group
    float d[FM][4];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) d[fm][r] = 0.f;
    if (has_d) {
      const int64_t base = bz * p.sd + (int64_t)(jf + c) * p.ldd + m0 + wm * WM + 4 * g;
      if (p.d_dtype == DT_F32) {
        f32x4 t[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          t[fm] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.Dt) + base + fm * 16);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int r = 0; r < 4; ++r) d[fm][r] = t[fm][r];
      } else {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) load_vec4(p.Dt, base + fm * 16, p.d_dtype, d[fm]);
      }
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      f32x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = fmaf(p.alpha, acc[fm][fn][r], p.beta * d[fm][r]) * f;
      *reinterpret_cast<f32x4*>(st + c * PITCH + fm * 16 + 4 * g) = v;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 4 * q + g;
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(st + row * PITCH + 4 * c);
      const float w[4] = {w4[0], w4[1], w4[2], w4[3]};
      const int j = jf + row;
      const int i = m0 + wm * WM + 4 * c;
#pragma unroll
      for (int o = 0; o < MSIGN_MAX_OUT; ++o) {
        if (o >= p.nout) break;
        const OutSpec& os = p.out[o];
        out_vec4<true>(os, bz * os.bstride + (int64_t)j * os.ld + i, w);
      }
    }
  });
  return true;
}

// Same for an off-diagonal tile of a triangle product, which is stored
// twice: C[i][j] at ptr[i ld + j] and its mirror at ptr[j ld + i].  Two
// passes through the wave's LDS region: 16-column groups read back by rows
// give the mirror stores, 16-row groups read back by rows the direct ones.
// D (symmetric, as every D of a triangle product is) is added after the
// read-back, loaded by rows too.  In a diagonal tile only the waves wholly
// above the diagonal (all i < j) qualify; the others (masking, diagonal
// terms) return false.
template <int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ bool epilogue_staged_tri(const GemmParams& p, int64_t bz, int ti, int tj,
                                                    const f32x4 (&acc)[BM / WGM / 16][BN / WGN / 16],
                                                    int wave, float* stage) {
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 16, FN = WN / 16;
  constexpr int PITCH = 68;
  static_assert(WM == 64 && WN % 64 == 0, "16 lanes x 4 values cover a row of the wave tile");
  // a diagonal tile qualifies only for the waves wholly above its diagonal
  if (p.nout < 1 || (ti == tj && wave / WGN >= wave % WGN)) return false;
  const int m0 = ti * BM, n0 = tj * BN;
#pragma unroll
  for (int o = 0; o < MSIGN_MAX_OUT; ++o) {
    if (o >= p.nout) break;
    const OutSpec& os = p.out[o];
    if (!os.vec_ok || m0 + BM > os.rows_lim || n0 + BN > os.cols_lim || n0 + BN > os.rows_lim ||
        m0 + BM > os.cols_lim)
      return false;
  }
  const bool has_d = p.Dt != nullptr;
  if (has_d && !(p.d_vec_ok && m0 + BM <= p.M && n0 + BN <= p.N)) return false;
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wm = wave / WGN, wn = wave % WGN;
  const int ib = m0 + wm * WM, jb = n0 + wn * WN;  // first row and column of the wave tile
  float* st = stage + wave * (16 * PITCH);
  // D is symmetric, so D[r][c] = Dt[r ldd + c].  D values are loaded ahead
  // of the stores that need them, 16-bit D two groups (eight chunks of four
  // values) at a time, fp32 D one group at a time: the compiler cannot tell
  // D from the outputs, so a load placed after a store waits for it, and a
  // load per chunk between the stores would wait out a memory round trip
  // each time.  The D dtype is a template argument of the passes, so each
  // form holds only its own registers (a whole pass's chunks at once spill
  // in the 128-register budget).
  const float f = p.vscale != nullptr ? p.vscale[4 * bz] : 1.f;
  auto passes = [&](auto DKI) {
    constexpr int DK = decltype(DKI)::value;  // 0: no D, 1: 16-bit, 2: fp32
    constexpr int GA = DK == 2 ? 1 : 2;       // groups per D batch
    using DV = typename std::conditional<DK == 2, f32x4, u32x2>::type;
    auto d_at = [&](int r0, int c0) {
      const int64_t idx = bz * p.sd + (int64_t)r0 * p.ldd + c0;
      if constexpr (DK == 2) return *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.Dt) + idx);
      else if constexpr (DK == 1) return *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.Dt) + idx);
      else return u32x2{0u, 0u};
    };
    // four consecutive values of C at (r0, c0 .. c0 + 3) from the staged
    // accumulators a and the D chunk dv, stored at ptr[r0 ld + c0] of every
    // output
    auto finish = [&](const f32x4& a, const DV& dv, int r0, int c0) {
      float d[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (DK == 1) {
        const bool bf = p.d_dtype == DT_BF16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint16_t hb = (uint16_t)(dv[r >> 1] >> (16 * (r & 1)));
          d[r] = bf ? bf16_bits_to_f32(hb) : f16_bits_to_f32(hb);
        }
      } else if constexpr (DK == 2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) d[r] = dv[r];
      }
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = fmaf(p.alpha, a[r], p.beta * d[r]) * f;
#pragma unroll
      for (int o = 0; o < MSIGN_MAX_OUT; ++o) {
        if (o >= p.nout) break;
        const OutSpec& os = p.out[o];
        store_vec4(os.ptr, bz * os.bstride + (int64_t)r0 * os.ld + c0, os.dtype, w);
      }
    };
    // mirror: column group fn staged as [j][i], rows j stored at ptr[j ld + i]
    static_assert(FN % 2 == 0 && (FM * (FN / 4)) % 2 == 0, "groups go in pairs");
    static_for<FN / GA>([&](auto PI) {
      constexpr int fn0 = GA * decltype(PI)::value;
      DV dv[4 * GA];
#pragma unroll
      for (int k = 0; k < 4 * GA; ++k) dv[k] = d_at(jb + (fn0 + k / 4) * 16 + 4 * (k % 4) + g, ib + 4 * c);
#pragma unroll
      for (int e = 0; e < GA; ++e) {
        const int fn = fn0 + e;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          *reinterpret_cast<f32x4*>(st + c * PITCH + fm * 16 + 4 * g) = acc[fm][fn];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 4 * q + g;
          finish(*reinterpret_cast<const f32x4*>(st + row * PITCH + 4 * c), dv[4 * e + q], jb + fn * 16 + row,
                 ib + 4 * c);
        }
      }
    });
    // direct: row group fm staged as [i][j], 64 columns j at a time, rows i
    // stored at ptr[i ld + j]
    constexpr int NH = FN / 4;
    static_for<FM * NH / GA>([&](auto PI) {
      constexpr int fh0 = GA * decltype(PI)::value;
      DV dv[4 * GA];
#pragma unroll
      for (int k = 0; k < 4 * GA; ++k) {
        const int fh = fh0 + k / 4;
        dv[k] = d_at(ib + (fh / NH) * 16 + 4 * (k % 4) + g, jb + 64 * (fh % NH) + 4 * c);
      }
#pragma unroll
      for (int e = 0; e < GA; ++e) {
        const int fm = (fh0 + e) / NH, h = (fh0 + e) % NH;
#pragma unroll
        for (int f4 = 0; f4 < 4; ++f4)
#pragma unroll
          for (int r = 0; r < 4; ++r) st[(4 * g + r) * PITCH + f4 * 16 + c] = acc[fm][4 * h + f4][r];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 4 * q + g;
          finish(*reinterpret_cast<const f32x4*>(st + row * PITCH + 4 * c), dv[4 * e + q], ib + fm * 16 + row,
                 jb + 64 * h + 4 * c);
        }
      }
    });
  };
  if (!has_d) passes(std::integral_constant<int, 0>{});
  else if (p.d_dtype == DT_F32) passes(std::integral_constant<int, 2>{});
  else passes(std::integral_constant<int, 1>{});
  return true;
}

template <int BM, int BN, int WGM, int WGN, bool TRI>
__device__ __forceinline__ void epilogue(const GemmParams& p, int L, int64_t bz, int ti, int tj,
                                         const f32x4 (&acc)[BM / WGM / 16][BN / WGN / 16],
                                         int wave, float* stage = nullptr) {
  constexpr int FM = BM / WGM / 16, FN = BN / WGN / 16;
  if constexpr (!TRI && BM / WGM == 64) {
    if (stage != nullptr && epilogue_staged<BM, BN, WGM, WGN>(p, bz, ti, tj, acc, wave, stage)) return;
  }
  if constexpr (TRI && BM / WGM == 64 && (BN / WGN) % 64 == 0) {
    // acc^2 sums per fragment row (off-diagonal tiles counted twice, for
    // their mirror)
    auto sums = [&]() {
      if (p.sumsq == nullptr) return;
      const float w = ti != tj ? 2.f : 1.f;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        float sq = 0.f;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int r = 0; r < 4; ++r) sq += acc[fm][fn][r] * acc[fm][fn][r];
        wave_sum_store(w * sq, sumsq_slot<BM, WGM, WGN>(p, L, wave, fm));
      }
    };
    // In a diagonal tile the waves wholly below the diagonal store nothing:
    // every element there is the mirror of one above it (i > j), which the
    // waves above the diagonal store.
    if (ti == tj && wave / WGN > wave % WGN) {
      sums();
      return;
    }
    if (stage != nullptr && epilogue_staged_tri<BM, BN, WGM, WGN>(p, bz, ti, tj, acc, wave, stage)) {
      sums();
      return;
    }
  }
  // fragment rows whose D loads share a round trip: two, except in the
  // 16-wave rectangular tile, whose 128-register budget (next to its
  // K-major A addressing) holds only one row's D values without spilling
  constexpr int NR = (FM >= 2 && (WGM * WGN < 16 || TRI)) ? 2 : 1;
  const float w2 = (TRI && ti != tj) ? 2.f : 1.f;
  static_for<FM / NR>([&](auto I) {
    constexpr int fm0 = decltype(I)::value * NR;
    f32x4 rows[NR * FN];
#pragma unroll
    for (int f = 0; f < NR * FN; ++f) rows[f] = acc[fm0 + f / FN][f % FN];
    float sq[NR];
    epilogue_rows<BM, BN, WGM, WGN, TRI, NR>(p, bz, ti, tj, wave, fm0, rows, sq);
    if (TRI && p.sumsq != nullptr) {
#pragma unroll
      for (int k = 0; k < NR; ++k) wave_sum_store(w2 * sq[k], sumsq_slot<BM, WGM, WGN>(p, L, wave, fm0 + k));
    }
  });
}

// Block b of the launch of problem p (b counts from the problem's first
// block).
template <typename T, int BM, int BN, int WGM, int WGN, int BKB, int NST, bool TRI, int KW, bool AT>
__device__ __forceinline__ void gemm_nt_block(const GemmParams& p, const int b) {
  constexpr int NT = WGM * WGN * KW * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int ESZ = Elem<T>::size;
  constexpr int CE = 16 / ESZ;      // elements per 16-byte chunk
  constexpr int CPR = BKB / 16;     // chunks per row of one K slice
  constexpr int KTE = CPR * CE;     // elements per K slice
  constexpr int KSUB = CPR / 4;     // MFMA K sub-steps per slice (4 lane groups)
  constexpr int ACH = BM * CPR * KW / NT, BCH = BN * CPR * KW / NT;
  static_assert(CPR == 4 || CPR == 8, "K slice must be 64 or 128 bytes");
  // KW > 1: KW waves share one tile (WGM = WGN = 1), wave w taking K slices
  // w, w + KW, ...; one load step brings KW consecutive slices, thread group
  // s of a step moving slice s (so NT / CPR must equal the tile edge)
  static_assert(KW == 1 || (WGM == 1 && WGN == 1 && BM == BN && NT / CPR == BM), "K-split waves");
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "tile/thread mismatch");
  static_assert(!TRI || BM == BN, "triangle mode needs square tiles");
  // NST: K slices of register prefetch (1..3), or 0 for direct global->LDS
  // loads (buffer_load ... lds) into a 2-stage ring
  static_assert(NST >= 0 && NST <= 3 && (NST > 0 || KW == 1), "prefetch depth");
  // AT: P is stored K-major ([K][M], row pitch ldp): the A tile of a slice is
  // KTE rows of BM elements (CPRA chunks each) in LDS, read back with
  // transpose reads (16-bit) or element reads (fp32).
  static_assert(!AT || !TRI, "transposed A only for rectangular products");
  constexpr int CPRA = AT ? BM * ESZ / 16 : CPR;
  static_assert(!AT || (CPRA >= (ESZ == 2 ? 8 : 16) && (KTE * CPRA * KW) % NT == 0), "transposed A tile layout");

  __shared__ u32x4 lds[2][KW * (BM + BN) * CPR];  // [stage][A slices, then B slices]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kw = KW > 1 ? tid >> 6 : 0;    // K share of this wave
  const int wave = KW > 1 ? 0 : tid >> 6;  // position of this wave in the tile
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- tile (or K part of a tile) of this block ----
  // Whole tiles come first in block order, renumbered XCD-contiguously among
  // themselves; the K parts of the split tiles follow, dealt round-robin.
  int L, part = -1, unit = 0;
  if (b < p.nfull) {
    L = xcd_contiguous(b, p.nfull);
  } else {
    unit = b - p.nfull;
    L = p.nfull + unit / p.split;
    part = unit % p.split;
  }
  int64_t bz;
  int ti, tj;
  if (!tile_of<TRI>(p, L, bz, ti, tj)) return;  // whole block, before any barrier
  const int m0 = ti * BM, n0 = tj * BN;

  // Buffer descriptors start at this tile's first row; rows past M (or N)
  // fall outside num_records, so those loads return zeros without branches.
  const char* Pt = static_cast<const char*>(p.P) + (bz * p.sp + (int64_t)m0 * p.ldp) * ESZ;
  const char* Qt = static_cast<const char*>(p.Q) + (bz * p.sq + (int64_t)n0 * p.ldq) * ESZ;
  const int prow = p.M - m0 < BM ? p.M - m0 : BM;
  const int qrow = p.N - n0 < BN ? p.N - n0 : BN;
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Pt, (short)0, prow > 0 ? (int)((int64_t)prow * p.ldp * ESZ) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Qt, (short)0, qrow > 0 ? (int)((int64_t)qrow * p.ldq * ESZ) : 0, 0x00020000);

  // Each thread moves chunks (row0 + s * RSTEP, ch) for s < ACH (and BCH):
  // the same K column and swizzle for every s, since RSTEP is a multiple of
  // the swizzle period.
  constexpr int RSTEP = NT / CPR;
  static_assert(RSTEP % 8 == 0, "row step must keep the swizzle");
  const int row0 = tid / CPR, ch0 = tid % CPR;
  const int kcol = ch0 * CE;
  const int a_base = (row0 * (int)p.ldp + kcol) * ESZ;
  const int b_base = (row0 * (int)p.ldq + kcol) * ESZ;
  const int a_step = KW > 1 ? KTE * ESZ : RSTEP * (int)p.ldp * ESZ;
  const int b_step = KW > 1 ? KTE * ESZ : RSTEP * (int)p.ldq * ESZ;
  const int lds_w = row0 * CPR + swz<CPR>(row0, ch0);  // + s * RSTEP * CPR
  // AT: chunk s * NT + tid of a slice is K row kr = (s * NT + tid) / CPRA,
  // logical chunk tid % CPRA (NT is a multiple of CPRA), stored at its
  // swizzled position.  Each slice gets its own descriptor starting at its
  // first K row (column m0), so offsets stay small and reads past the
  // matrix's last row return zeros; columns past M feed only rows of the
  // result that are never stored.
  const char* Pk = static_cast<const char*>(p.P) + (bz * p.sp + m0) * ESZ;
  const int64_t pk_bytes = ((int64_t)(p.kvalid > 0 ? p.kvalid : p.K) * p.ldp - m0) * ESZ;
  // Chunk s sits NT / CPRA K rows below chunk 0 (with K-split waves, the
  // same row of slice s); when that is a multiple of the swizzle's period in
  // k (16) its LDS slot is chunk 0's plus s NT.
  constexpr int AT_RSTEP = AT ? NT / CPRA : 1;
  const int at_kr = tid / CPRA, at_c = tid % CPRA;
  const int at_goff = (at_kr * (int)p.ldp + at_c * CE) * ESZ;
  const int at_gstep = AT_RSTEP * (int)p.ldp * ESZ;
  auto at_slot = [&](int s) {
    if constexpr (AT_RSTEP % 16 == 0) {
      return at_kr * CPRA + swz_t<ESZ, CPRA>(at_kr, at_c) + s * NT;
    } else {
      const int kr = at_kr + s * AT_RSTEP;
      return kr * CPRA + swz_t<ESZ, CPRA>(kr, at_c);
    }
  };


  // K is a multiple of 64 elements (host contract), so every slice is whole;
  // slices past the end (the last prefetches) read past the row or past
  // num_records and are never copied into LDS.
  auto gload = [&](u32x4* dst, int k0) {
    if constexpr (AT) {
      const int64_t left = pk_bytes - (int64_t)k0 * p.ldp * ESZ;
      const int64_t span = (int64_t)ACH * AT_RSTEP * p.ldp * ESZ;  // the K rows of one load step
      const int nrec = left <= 0 ? 0 : (int)(left < span ? left : span);
      const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(Pk + (int64_t)k0 * p.ldp * ESZ, nrec);
#pragma unroll
      for (int s = 0; s < ACH; ++s)
        dst[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, at_goff + s * at_gstep, 0, 0));
    } else {
#pragma unroll
      for (int s = 0; s < ACH; ++s)
        dst[s] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rP, a_base + s * a_step + k0 * ESZ, 0, 0));
    }
#pragma unroll
    for (int s = 0; s < BCH; ++s)
      dst[ACH + s] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rQ, b_base + s * b_step + k0 * ESZ, 0, 0));
  };
  auto lstore = [&](const u32x4* src, int buf) {
#pragma unroll
    for (int s = 0; s < ACH; ++s) {
      if constexpr (AT) {
        lds[buf][at_slot(s)] = src[s];
      } else {
        lds[buf][lds_w + s * RSTEP * CPR] = src[s];
      }
    }
#pragma unroll
    for (int s = 0; s < BCH; ++s) lds[buf][KW * BM * CPR + lds_w + s * RSTEP * CPR] = src[ACH + s];
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Small wave tiles read all A and B fragments of a sub-step before its
  // MFMAs (the reads overlap each other and the first products); the
  // 128 x 128 wave tile holds its A fragments and streams B fragments one at
  // a time to stay within the register file next to 256 accumulators.
  constexpr bool kAllFrags = (FM + FN) <= 12;
  // Triangle products with direct loads and two MFMA sub-steps per slice
  // put the barrier between the sub-steps (measured on the 256 x 256 tier:
  // X X^T and A A 2.5-7 % faster, bit-identical; the rectangular product with
  // its transpose reads gained nothing).
  constexpr bool DEFER = !AT && NST == 0 && KSUB == 2 && kAllFrags && KW == 1;
  // A fragments of MFMA sub-step kk of the K slice in `stage`
  auto read_a = [&](const u32x4* stage, const int kk, u32x4 (&a)[FM]) {
    const int ch = kk * 4 + (lane >> 4);
    if constexpr (AT && ESZ == 2) {
      // K rows 32 kk + 8 g + (r / 4) and that + 4, columns m .. m + 3 of
      // the fragment's 16: after the transpose reads lane (g, r) holds
      // column r at K = 32 kk + 8 g + 0..7, the order of the B fragment
      const int g = lane >> 4, r = lane & 15;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int m = wm * WM + fm * 16 + 4 * (r & 3);
        const int k0r = kk * 32 + 8 * g + (r >> 2), k1r = k0r + 4;
        const int off0 = k0r * CPRA * 16 + swz_t<2, CPRA>(k0r, m >> 3) * 16 + (m & 7) * 2;
        const int off1 = k1r * CPRA * 16 + swz_t<2, CPRA>(k1r, m >> 3) * 16 + (m & 7) * 2;
        a[fm] = lds_read_tr16_pair(stage + kw * BM * CPR, off0, off1);
      }
    } else if constexpr (AT) {
      // fp32: lane (g, r) reads column r at K = 16 kk + 4 g + 0..3
      const int g = lane >> 4, r = lane & 15;
      const float* base = reinterpret_cast<const float*>(stage + kw * BM * CPR);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int m = wm * WM + fm * 16 + r;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = kk * 16 + 4 * g + e;
          v[e] = base[k * CPRA * 4 + swz_t<4, CPRA>(k, m >> 2) * 4 + (m & 3)];
        }
        a[fm] = __builtin_bit_cast(u32x4, v);
      }
    } else {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int row = wm * WM + fm * 16 + (lane & 15);
        a[fm] = stage[(kw * BM + row) * CPR + swz<CPR>(row, ch)];
      }
    }
  };
  // A and B fragments of sub-step kk (all-fragments wave tiles)
  auto read_frags = [&](const u32x4* stage, const int kk, u32x4 (&a)[FM], u32x4 (&b)[FN]) {
    const int ch = kk * 4 + (lane >> 4);
    read_a(stage, kk, a);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int row = wn * WN + fn * 16 + (lane & 15);
      b[fn] = stage[(KW * BM + kw * BN + row) * CPR + swz<CPR>(row, ch)];
    }
  };
  // the sub-step's products, B fragment by B fragment (each B fragment is
  // dead after its FM products, so its register can take the next read)
  auto mma_frags = [&](const u32x4 (&a)[FM], const u32x4 (&b)[FN]) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) Mma<T>::run(acc[fm][fn], a[fm], b[fn]);
    __builtin_amdgcn_s_setprio(0);
  };
  auto compute = [&](const u32x4* stage) {
    __builtin_amdgcn_s_setprio(1);  // favour waves that are issuing MFMAs
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      u32x4 a[FM];
      read_a(stage, kk, a);
      if constexpr (kAllFrags) {
        u32x4 b[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int row = wn * WN + fn * 16 + (lane & 15);
          b[fn] = stage[(KW * BM + kw * BN + row) * CPR + swz<CPR>(row, ch)];
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) Mma<T>::run(acc[fm][fn], a[fm], b[fn]);
      } else {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int row = wn * WN + fn * 16 + (lane & 15);
          const u32x4 b = stage[(KW * BM + kw * BN + row) * CPR + swz<CPR>(row, ch)];
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) Mma<T>::run(acc[fm][fn], a[fm], b);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Register prefetch of NST K slices: slice t lives in stg[t % NST] from
  // its load (issued NST iterations ahead) until it is copied into LDS
  // buffer t % 2 one iteration before its use.  Prefetches are issued
  // unconditionally (past the end of K they read nothing that is used), so
  // the wait before an LDS copy covers only the oldest slice and leaves the
  // newer ones in flight.
  const int KT = (p.K + KTE - 1) / KTE;
  int kt0 = 0, nk = KT;
  if (part >= 0) {
    kt0 = (int)((int64_t)part * KT / p.split);
    nk = (int)((int64_t)(part + 1) * KT / p.split) - kt0;
  }
  if constexpr (NST == 0) {
    // Direct loads: a wave's load instruction s writes the 64 consecutive
    // LDS slots s * NT + 64 wave + lane, i.e. row (or K row) row0 + s RSTEP,
    // physical chunk tid % CPR (CPRA); the lane fetches the logical chunk
    // that the swizzle puts there (an involution, the same for every s).
    // Slice j + 1 loads into the other stage while slice j is computed; a
    // wave waits for its own loads (vmcnt) and reads (lgkmcnt) before each
    // barrier, so after it slice j + 1 is whole and stage j is free.
    const int uw = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS destinations
    int dma_a = 0;
    if constexpr (AT) dma_a = (at_kr * (int)p.ldp + swz_t<ESZ, CPRA>(at_kr, at_c) * CE) * ESZ;
    else dma_a = (row0 * (int)p.ldp + swz<CPR>(row0, ch0) * CE) * ESZ;
    const int dma_b = (row0 * (int)p.ldq + swz<CPR>(row0, ch0) * CE) * ESZ;
    auto issue = [&](u32x4* stage, int k0) {
      if constexpr (AT) {
        const int64_t left = pk_bytes - (int64_t)k0 * p.ldp * ESZ;
        const int64_t span = (int64_t)ACH * AT_RSTEP * p.ldp * ESZ;
        const int nrec = left <= 0 ? 0 : (int)(left < span ? left : span);
        const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(Pk + (int64_t)k0 * p.ldp * ESZ, nrec);
#pragma unroll
        for (int s = 0; s < ACH; ++s) {
          const int off = dma_a + s * at_gstep;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, MSIGN_LDS(stage + s * NT + uw * 64), 16, off, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < ACH; ++s) {
          const int off = dma_a + s * a_step + k0 * ESZ;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, MSIGN_LDS(stage + s * NT + uw * 64), 16, off, 0, 0, 0);
        }
      }
#pragma unroll
      for (int s = 0; s < BCH; ++s) {
        const int off = dma_b + s * b_step + k0 * ESZ;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, MSIGN_LDS(stage + BM * CPR + s * NT + uw * 64), 16, off,
                                                 0, 0, 0);
      }
    };
    // In both loop forms slice s is loaded after barrier E(s - 1) into
    // stage s & 1 (whose previous slice, s - 2, every wave finished reading
    // before E(s - 1)), every loader waits for its loads before its next
    // barrier, and slice s is read only after E(s).
    auto plain_loop = [&]() {
      // (one step: the loads into `wr` and the reads from `rd` are declared
      // not to alias, so the reads need not wait for the loads in flight)
      auto step = [&](const u32x4* __restrict__ rd, u32x4* __restrict__ wr, bool load_next, int k_next) {
        if (load_next) issue(wr, k_next);
        compute(rd);
      };
      if (nk > 0) issue(lds[0], kt0 * KTE);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      for (int j = 0; j < nk; ++j) {
        step(lds[j & 1], lds[(j + 1) & 1], j + 1 < nk, (kt0 + j + 1) * KTE);
        wait_all_barrier();
      }
    };
    // The barrier between a slice's two MFMA sub-steps.  Iteration j (slice
    // j in stage j & 1, its sub-step-0 fragments already in registers):
    // sub-step 0's products; sub-step 1's reads; wait for this wave's loads
    // of slice j + 1 and its reads, barrier E(j + 1); loads of slice j + 2
    // into stage j & 1; sub-step 1's products, whose fragments crossed the
    // barrier in registers, so the wave has MFMAs to issue right after it
    // while the reads of slice j + 1's sub-step 0 follow.
    auto deferred_loop = [&]() {
      if constexpr (DEFER) {
        u32x4 fa[FM], fb[FN];
        // One iteration; `cur` holds slice j, `nxt` takes slice j + 1 (the
        // two stages declared not to alias, so that no read waits for the
        // loads in flight into the other stage).
        auto iter = [&](u32x4* __restrict__ cur, const u32x4* __restrict__ nxt, int j) {
          mma_frags(fa, fb);
          read_frags(cur, 1, fa, fb);
          wait_all_barrier();
          if (j + 2 < nk) issue(cur, (kt0 + j + 2) * KTE);
          mma_frags(fa, fb);
          if (j + 1 < nk) read_frags(nxt, 0, fa, fb);
        };
        if (nk > 0) issue(lds[0], kt0 * KTE);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (nk > 1) issue(lds[1], (kt0 + 1) * KTE);
        if (nk > 0) read_frags(lds[0], 0, fa, fb);
        // two iterations per trip (the one-iteration loop spills 32 bytes
        // per lane)
        for (int j = 0; j < nk; j += 2) {
          iter(lds[0], lds[1], j);
          if (j + 1 < nk) iter(lds[1], lds[0], j + 1);
        }
      }
    };
    if constexpr (DEFER) deferred_loop();
    else plain_loop();
    // the last barrier came after every read of the ring: it is free
  } else {
  // steps of KW slices; wave kw computes slice j * KW + kw of step j when
  // that slice is in range
  const int ns = (nk + KW - 1) / KW;
  u32x4 stg[NST][ACH + BCH];
  gload(stg[0], kt0 * KTE);
  if constexpr (NST >= 2) gload(stg[1], (kt0 + KW) * KTE);
  if constexpr (NST >= 3) gload(stg[2], (kt0 + 2 * KW) * KTE);
  if (ns > 0) lstore(stg[0], 0);
  __syncthreads();
  auto iter = [&](int j, auto S) {
    constexpr int s = decltype(S)::value;  // j % NST
    gload(stg[s], (kt0 + (j + NST) * KW) * KTE);
    if (KW == 1 || j * KW + kw < nk) compute(lds[j & 1]);
    if (j + 1 < ns) lstore(stg[(s + 1) % NST], (j + 1) & 1);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, (1 % NST)>;
  using I2 = std::integral_constant<int, (2 % NST)>;
  int j = 0;
  for (; j + NST <= ns; j += NST) {
    iter(j, I0{});
    if constexpr (NST >= 2) iter(j + 1, I1{});
    if constexpr (NST >= 3) iter(j + 2, I2{});
  }
  if (j < ns) iter(j, I0{});
  if constexpr (NST >= 3) {
    if (j + 1 < ns) iter(j + 1, I1{});
  }
  }

  if constexpr (KW > 1) {
    // The K shares' accumulators meet in LDS (the last iteration ended with
    // a barrier, so the ring is free); wave q then adds fragment row fm = q
    // over the shares in share order (fixed, so bit-stable) and finishes it.
    static_assert(KW == FM, "one fragment row per wave");
    static_assert(KW * FM * FN * 64 * 16 <= (int)sizeof(lds), "LDS holds every share");
    f32x4* red = reinterpret_cast<f32x4*>(&lds[0][0]);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) red[((kw * FM + fm) * FN + fn) * 64 + lane] = acc[fm][fn];
    __syncthreads();
    const int fm = kw;
    f32x4 sum[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      sum[fn] = red[(fm * FN + fn) * 64 + lane];
#pragma unroll
      for (int q = 1; q < KW; ++q) sum[fn] += red[((q * FM + fm) * FN + fn) * 64 + lane];
    }
    if (part >= 0) {  // same partial layout as below, written by fragment row
      const int t = unit / p.split;
      f32x4* dst = reinterpret_cast<f32x4*>(p.partial) + ((int64_t)t * p.split + part) * (FM * FN * 64) + lane;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) dst[(fm * FN + fn) * 64] = sum[fn];
      return;
    }
    float sq[1];
    epilogue_rows<BM, BN, WGM, WGN, TRI, 1>(p, bz, ti, tj, 0, fm, sum, sq);
    if (TRI && p.sumsq != nullptr)
      wave_sum_store((ti != tj ? 2.f : 1.f) * sq[0], sumsq_slot<BM, WGM, WGN>(p, L, 0, fm));
    return;
  }

  if (part >= 0) {  // partial sums of this K range, one f32x4 per thread and fragment
    // layout [split tile][wave][part][fragment][lane]: each wave writes, and
    // the reduce pass reads, one contiguous run per part
    const int t = unit / p.split;
    f32x4* dst = reinterpret_cast<f32x4*>(p.partial) +
                 (((int64_t)t * (WGM * WGN) + wave) * p.split + part) * (FM * FN * 64) + lane;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) dst[(fm * FN + fn) * 64] = acc[fm][fn];
    return;
  }
  // (the last K iteration ended with a barrier: the LDS ring is free)
  static_assert(KW > 1 || WGM * WGN * 16 * 68 * 4 <= (int)sizeof(lds), "staging fits the LDS ring");
  epilogue<BM, BN, WGM, WGN, TRI>(p, L, bz, ti, tj, acc, wave, reinterpret_cast<float*>(&lds[0][0]));
}

template <typename T, int BM, int BN, int WGM, int WGN, int BKB, int NST, bool TRI, int KW, bool AT, int NG>
__global__ void __launch_bounds__(WGM * WGN * KW * 64)
gemm_nt_kernel(const GemmGroups<NG> groups) {
  // The table is read in place from the kernel-argument segment (it is the
  // first argument): indexing the by-value argument with the block's group
  // would make the compiler copy the whole table to scratch memory.  Single
  // products on the smaller tiles read the by-value argument instead
  // (measured: about 1 us less per launch, which counts where those tiers
  // run); on 256 x 256 tiles the in-place reads are faster (the by-value
  // form left 12 bytes of scratch per lane in the triangle kernels).
  if constexpr (NG == 1 && BM < 256) {
    gemm_nt_block<T, BM, BN, WGM, WGN, BKB, NST, TRI, KW, AT>(groups.g[0], (int)blockIdx.x);
  } else {
    const GemmGroups<NG>& G = *(const GemmGroups<NG>*)__builtin_amdgcn_kernarg_segment_ptr();
    int gi = 0;
#pragma unroll
    for (int i = 1; i < NG; ++i) gi += (int)blockIdx.x >= G.bstart[i] ? 1 : 0;
    gemm_nt_block<T, BM, BN, WGM, WGN, BKB, NST, TRI, KW, AT>(G.g[gi], (int)blockIdx.x - G.bstart[gi]);
  }
}

// Second pass for split tiles.  Block (t, w) takes wave w's fragments of
// split tile t; its wave q handles fragment row fm = q: it adds the tile's
// parts in part order (fixed, so the result is bit-stable) and runs the
// epilogue of those fragments.  Splitting the work this way keeps many
// partial-sum loads in flight per lane (the pass is latency-bound).
template <typename T, int BM, int BN, int WGM, int WGN, bool TRI>
__global__ void __launch_bounds__(BM / WGM / 16 * 64)
gemm_nt_reduce_kernel(const GemmParams p) {
  constexpr int WG = WGM * WGN;
  constexpr int FM = BM / WGM / 16, FN = BN / WGN / 16;
  constexpr int FF = FM * FN * 64;  // f32x4 per wave and part
  const int t = blockIdx.x / WG, w = blockIdx.x % WG;
  const int fm = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t bz;
  int ti, tj;
  if (!tile_of<TRI>(p, p.nfull + t, bz, ti, tj)) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(p.partial) + ((int64_t)t * WG + w) * p.split * FF +
                     fm * FN * 64 + lane;
  f32x4 acc[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) acc[fn] = src[fn * 64];
  int sp = 1;
  for (; sp + 4 <= p.split; sp += 4) {
    f32x4 v[4][FN];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) v[u][fn] = src[(int64_t)(sp + u) * FF + fn * 64];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[fn] += v[u][fn];
  }
  for (; sp < p.split; ++sp)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fn] += src[(int64_t)sp * FF + fn * 64];
  float sq[1];
  epilogue_rows<BM, BN, WGM, WGN, TRI, 1>(p, bz, ti, tj, w, fm, acc, sq);
  if (TRI && p.sumsq != nullptr)
    wave_sum_store((ti != tj ? 2.f : 1.f) * sq[0], sumsq_slot<BM, WGM, WGN>(p, p.nfull + t, w, fm));
}

}  // namespace msign
