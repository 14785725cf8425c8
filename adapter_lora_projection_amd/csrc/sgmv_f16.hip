// SGMV shrink/expand kernels instantiated for one storage type (f16); split per type so the
// build compiles the types in parallel.
#include "sgmv_impl.hpp"
#include "shrink_gemv.hpp"
#include "shrink_lds.hpp"

namespace lmx {

hipError_t launch_shrink_f16(const ShrinkArgs& a, const ShrinkPlan& plan, hipStream_t st) {
  if (plan.gemv) return launch_shrink_gemv_dt<DT_F16>(a, plan, st);
  if (plan.lds) return launch_shrink_lds_dt<DT_F16>(a, plan, st);
  return launch_shrink_dt<DT_F16>(a, plan, st);
}

hipError_t launch_shrink_sk_reduce_f16(const ShrinkArgs& a, int bm, hipStream_t st) {
  return launch_shrink_sk_reduce_dt<DT_F16>(a, bm, st);
}

hipError_t launch_expand_f16(const ExpandArgs& a, const ExpandPlan& plan, hipStream_t st) {
  return launch_expand_dt<DT_F16>(a, plan, st);
}

hipError_t launch_pair_f16(const ShrinkArgs& s, const ExpandArgs& e, const PairArgs& pa,
                           bool kfull, bool aligned_y, hipStream_t st) {
  return launch_pair_dt<DT_F16>(s, e, pa, kfull, aligned_y, st);
}

}  // namespace lmx
