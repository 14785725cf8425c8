// SGMV shrink/expand kernels instantiated for one storage type (bf16); split per type so the
// build compiles the types in parallel.
#include "sgmv_impl.hpp"
#include "shrink_lds.hpp"

namespace lmx {

hipError_t launch_shrink_bf16(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st) {
  if (plan.lds) return launch_shrink_lds_dt<DT_BF16>(a, plan, st);
  return launch_shrink_dt<DT_BF16>(a, plan, st);
}

hipError_t launch_shrink_sk_reduce_bf16(const ShrinkArgs& a, int bm, hipStream_t st) {
  return launch_shrink_sk_reduce_dt<DT_BF16>(a, bm, st);
}

hipError_t launch_expand_bf16(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  return launch_expand_dt<DT_BF16>(a, plan, st);
}

}  // namespace lmx
