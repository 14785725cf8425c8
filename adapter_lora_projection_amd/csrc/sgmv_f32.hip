// SGMV shrink/expand kernels instantiated for one storage type (f32); split per type so the
// build compiles the types in parallel.
#include "sgmv_impl.hpp"

namespace lmx {

hipError_t launch_shrink_f32(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st) {
  if (plan.lds) return hipErrorInvalidValue;  // 16-bit types only
  return launch_shrink_dt<DT_F32>(a, plan, st);
}

hipError_t launch_shrink_sk_reduce_f32(const ShrinkArgs& a, int bm, hipStream_t st) {
  return launch_shrink_sk_reduce_dt<DT_F32>(a, bm, st);
}

hipError_t launch_expand_f32(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  return launch_expand_dt<DT_F32>(a, plan, st);
}

}  // namespace lmx
