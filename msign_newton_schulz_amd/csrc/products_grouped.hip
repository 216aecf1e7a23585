// Product kernels for grouped launches (up to kMaxGroups problems).
#include "launch_impl.hpp"

namespace msign {

hipError_t launch_products_grouped(int32_t cdt, bool tri, const GemmParams* qs, const GroupPlan& l,
                                   hipStream_t st) {
  return launch_products<kMaxGroups>(cdt, tri, qs, l, st);
}

}  // namespace msign
