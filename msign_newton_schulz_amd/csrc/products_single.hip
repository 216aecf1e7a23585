// Product kernels for single problems (one-entry group table).
#include "launch_impl.hpp"

namespace msign {

hipError_t launch_products_single(int32_t cdt, bool tri, const GemmParams* qs, const GroupPlan& l,
                                  hipStream_t st) {
  return launch_products<1>(cdt, tri, qs, l, st);
}

}  // namespace msign
