// Product kernel launches for a group table of NG entries (see launch.hpp).
#pragma once

#include "../../include/msign.h"
#include "launch.hpp"

#include <climits>
#include <cstring>

namespace msign {

static_assert(sizeof(GemmGroups<kMaxGroups>) <= 4096, "kernel arguments");

template <typename T, int BM, int BN, int WGM, int WGN, int BKB, int NST, bool TRI, int KW, bool AT, int NG>
hipError_t launch_cfg(const GemmParams* qs, const GroupPlan& l, hipStream_t st) {
  if (l.ng < 1 || l.ng > NG) return hipErrorInvalidValue;
  GemmGroups<NG> k;
  std::memset(&k, 0, sizeof(k));
  int64_t blocks = 0;
  for (int s = 0; s < NG; ++s) {
    if (s >= l.ng) {
      k.bstart[s] = INT32_MAX;
      continue;
    }
    const int i = l.order[s];
    GemmParams q = qs[i];
    const bool last = s == l.ng - 1;
    const int64_t tail = last ? l.tail : 0;
    q.tiles_m = l.tiles_m[i];
    q.tiles_n = l.tiles_n[i];
    q.tpm = l.tpm[i];
    q.nfull = (int32_t)(l.nt[i] - tail);
    q.split = last ? l.split : 1;
    k.g[s] = q;
    k.bstart[s] = (int32_t)blocks;
    blocks += q.nfull + tail * q.split;
  }
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  gemm_nt_kernel<T, BM, BN, WGM, WGN, BKB, NST, TRI, KW, AT, NG>
      <<<dim3((unsigned)blocks), WGM * WGN * KW * 64, 0, st>>>(k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || l.tail == 0) return e;
  gemm_nt_reduce_kernel<T, BM, BN, WGM, WGN, TRI>
      <<<dim3((unsigned)(l.tail * WGM * WGN)), BM / WGM / 16 * 64, 0, st>>>(k.g[l.ng - 1]);
  return hipGetLastError();
}

// Tile configurations per tier (256: 16 waves of 64 x 64, 128-byte K slices
// loaded straight into LDS; 128: 4 waves, 64-byte slices; 64: one tile
// shared along K by 4 waves, register prefetch).
template <typename T, int NG>
hipError_t launch_tri(const GemmParams* qs, const GroupPlan& l, hipStream_t st) {
  if (l.bm == 256) return launch_cfg<T, 256, 256, 4, 4, 128, 0, true, 1, false, NG>(qs, l, st);
  if (l.bm == 128) return launch_cfg<T, 128, 128, 2, 2, 64, 0, true, 1, false, NG>(qs, l, st);
  return launch_cfg<T, 64, 64, 1, 1, 64, 2, true, 4, false, NG>(qs, l, st);
}

// Rectangular products with P stored K-major (the iterate X, n x m, read
// as X^T).
template <typename T, int NG>
hipError_t launch_at(const GemmParams* qs, const GroupPlan& l, hipStream_t st) {
  if (l.bm == 256) return launch_cfg<T, 256, 256, 4, 4, 128, 0, false, 1, true, NG>(qs, l, st);
  if (l.bm == 128) return launch_cfg<T, 128, 128, 2, 2, 64, 0, false, 1, true, NG>(qs, l, st);
  return launch_cfg<T, 64, 64, 1, 1, 64, 2, false, 4, true, NG>(qs, l, st);
}

// Full-tile products with both operands row-major along K (single problems).
template <typename T>
hipError_t launch_dense(const GemmParams* qs, const GroupPlan& l, hipStream_t st) {
  if (l.bm == 256) return launch_cfg<T, 256, 256, 4, 4, 128, 0, false, 1, false, 1>(qs, l, st);
  if (l.bm == 128) return launch_cfg<T, 128, 128, 2, 2, 64, 0, false, 1, false, 1>(qs, l, st);
  return launch_cfg<T, 64, 64, 1, 1, 64, 2, false, 4, false, 1>(qs, l, st);
}

template <int NG>
hipError_t launch_products(int32_t cdt, bool tri, const GemmParams* qs, const GroupPlan& l, hipStream_t st) {
  switch (cdt) {
    case MSIGN_BF16: return tri ? launch_tri<bf16_t, NG>(qs, l, st) : launch_at<bf16_t, NG>(qs, l, st);
    case MSIGN_F16: return tri ? launch_tri<f16_t, NG>(qs, l, st) : launch_at<f16_t, NG>(qs, l, st);
    default: return tri ? launch_tri<float, NG>(qs, l, st) : launch_at<float, NG>(qs, l, st);
  }
}

}  // namespace msign
