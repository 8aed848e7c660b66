// Host-side helpers of the self-planned step shared by api.cpp and
// noalloc_api.cpp.  Not part of the public ABI (see include/pkv.h).
#pragma once

#include "pkv_internal.h"

namespace pkv {

// Self-planned step (api.cpp): the shared argument checks (problem, lengths
// pointer, split cap, batch <= kMaxLensRows, 32-bit task count, kernel
// shape) and the kernel arguments of its split and merge launches.
pkv_status check_selfplan_step(const pkv_problem* prob, const int32_t* seq_lens_dev,
                               int32_t max_splits);
SplitArgs selfplan_split_args(const pkv_problem* prob, const int32_t* seq_lens_dev,
                              int32_t max_splits, int32_t* work_counter_dev, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_table, float* st_m, float* st_l, float* st_o);
MergeArgs selfplan_merge_args(const pkv_problem* prob, const int32_t* seq_lens_dev,
                              int32_t max_splits, int32_t* work_counter_dev, const float* st_m,
                              const float* st_l, const float* st_o, void* out, float* lse);

// Device address of the allocation-free step's scratch array on the current
// device (noalloc.hip; looked up on the first call per device).
pkv_status noalloc_scratch_address(void** out);

}  // namespace pkv
