// Full-tile product kernels (single problems, both operands read along K).
#include "launch_impl.hpp"

namespace msign {

hipError_t launch_products_dense(int32_t cdt, const GemmParams* qs, const GroupPlan& l, hipStream_t st) {
  if (l.ng != 1) return hipErrorInvalidValue;
  switch (cdt) {
    case MSIGN_BF16: return launch_dense<bf16_t>(qs, l, st);
    case MSIGN_F16: return launch_dense<f16_t>(qs, l, st);
    default: return launch_dense<float>(qs, l, st);
  }
}

}  // namespace msign
