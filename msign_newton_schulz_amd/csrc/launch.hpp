// Launch layout of one product (single or grouped) and the two launchers
// that instantiate the product kernels: one for a single problem (one-entry
// group table) and one for up to kMaxGroups problems.  Each launcher lives
// in a translation unit of its own so that the two sets of kernel
// instantiations compile in parallel.
#pragma once

#include "gemm_nt.hpp"

namespace msign {

// How one product launch is laid out: tile configuration, the tiles of each
// group, the order in which the groups' blocks are dealt (longest K first,
// so that the shortest tiles fill the last round), and the K split of the
// tiles past the last full round of resident blocks, all of them in the
// group dealt last.
struct GroupPlan {
  int bm;  // tile edge: 256, 128 or 64
  int ng;
  int order[kMaxGroups];  // launch position -> group
  int32_t tiles_m[kMaxGroups], tiles_n[kMaxGroups], tpm[kMaxGroups];
  int64_t nt[kMaxGroups];
  int64_t tail;  // split tiles, the last ones of group order[ng - 1]
  int32_t split;
  size_t partial_bytes;
};

// Launch the product kernel (and the reduce pass of a K-split tail) for the
// problems qs[0..l.ng) laid out by `l`: cdt is the operand dtype
// (MSIGN_BF16, MSIGN_F16 or MSIGN_F32), tri a triangle product (P Q^T
// symmetric, upper tiles mirrored), else a rectangular one with P stored
// K-major.  launch_products_single needs l.ng == 1.
hipError_t launch_products_single(int32_t cdt, bool tri, const GemmParams* qs, const GroupPlan& l,
                                  hipStream_t st);
hipError_t launch_products_grouped(int32_t cdt, bool tri, const GemmParams* qs, const GroupPlan& l,
                                   hipStream_t st);

// Full-tile product of one problem with both operands read along K: every
// tile of P Q^T is computed (no triangle), for measuring the triangle
// kernels against the plain product.  Outputs of a symmetric result should
// be given as transposed stores (the same matrix), which take the staged
// whole-line epilogue.
hipError_t launch_products_dense(int32_t cdt, const GemmParams* qs, const GroupPlan& l, hipStream_t st);

}  // namespace msign
