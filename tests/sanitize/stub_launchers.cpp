// Kernel-launcher stubs for the sanitizer build of libpkv's host code.
//
// The AddressSanitizer / UndefinedBehaviorSanitizer build compiles only the
// host translation units (planner, cost model, argument validation) with g++;
// the HIP kernels are not part of it.  Every launcher here reports a failed
// launch (PKV_EHIP), so an entry point that gets as far as a launch returns
// an error instead of running anything.  The CPU tests that run against this
// build exercise planning, policies, cost features and argument validation.
#include "pkv_internal.h"
#include "selfplan_args.h"

namespace pkv {

pkv_status launch_split(const pkv_problem&, int, int, const SplitArgs&, int, hipStream_t) {
  return PKV_EHIP;
}
pkv_status launch_merge(const pkv_problem&, const MergeArgs&, hipStream_t) { return PKV_EHIP; }
pkv_status launch_append(const AppendArgs&, int, hipStream_t) { return PKV_EHIP; }
pkv_status launch_plan_device(const pkv_problem&, const int32_t*, int32_t, int32_t*, int32_t*,
                              hipStream_t) {
  return PKV_EHIP;
}
// The allocation-free step's device array is not part of this build.
pkv_status noalloc_scratch_address(void**) { return PKV_EHIP; }

}  // namespace pkv
