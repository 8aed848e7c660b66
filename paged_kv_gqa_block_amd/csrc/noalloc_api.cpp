// pkv_attend_noalloc: the self-planned decode step (split + merge) with its
// partial states in a library-owned device array (noalloc.hip) instead of
// caller buffers, so the call allocates nothing.  It serves callers that
// cannot allocate: code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc.
#include "launch_limits.h"
#include "pkv_internal.h"
#include "selfplan_args.h"

namespace pkv {
namespace {

size_t round_up_256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_noalloc_bytes(const pkv_problem* prob, int32_t max_splits) {
  if (check_problem(prob) != PKV_OK || max_splits < 1 || max_splits > 65535) return 0;
  const size_t slots = size_t(prob->batch) * prob->num_kv_heads * max_splits;
  const size_t g = size_t(prob->num_q_heads / prob->num_kv_heads);
  return 2 * round_up_256(slots * g * sizeof(float)) +
         round_up_256(slots * g * prob->head_dim * sizeof(float));
}

extern "C" pkv_status pkv_attend_noalloc(const pkv_problem* prob, const int32_t* seq_lens_dev,
                                         int32_t max_splits, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* block_table,
                                         void* out, float* lse, hipStream_t stream) {
  pkv_status st = check_selfplan_step(prob, seq_lens_dev, max_splits);
  if (st != PKV_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !out) return PKV_EINVAL;
  const size_t need = pkv_noalloc_bytes(prob, max_splits);
  if (need == 0) return PKV_EINVAL;
  if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ENOSPC;
  // One workgroup per possible task, so no task is ever claimed through a
  // counter: the scratch holds only the partial states, and nothing in it
  // has to start at zero (every state the merge reads was written by this
  // call's split launch).
  const int64_t upper = int64_t(prob->batch) * prob->num_kv_heads * max_splits;
  if (upper > kMaxGridGroups) return PKV_ERANGE;
  void* base = nullptr;
  st = noalloc_scratch_address(&base);
  if (st != PKV_OK) return st;
  const size_t slots = size_t(upper);
  const size_t g = size_t(prob->num_q_heads / prob->num_kv_heads);
  unsigned char* p = static_cast<unsigned char*>(base);
  float* st_m = reinterpret_cast<float*>(p);
  float* st_l = reinterpret_cast<float*>(p + round_up_256(slots * g * sizeof(float)));
  float* st_o = reinterpret_cast<float*>(p + 2 * round_up_256(slots * g * sizeof(float)));
  SplitArgs a = selfplan_split_args(prob, seq_lens_dev, max_splits, nullptr, q, k_pool, v_pool,
                                    block_table, st_m, st_l, st_o);
  a.num_items = static_cast<int32_t>(upper);
  st = launch_split(*prob, kModeLens, prob->kernel, a, static_cast<int>(upper), stream);
  if (st != PKV_OK) return st;
  MergeArgs m = selfplan_merge_args(prob, seq_lens_dev, max_splits, nullptr, st_m, st_l, st_o,
                                    out, lse);
  return launch_merge(*prob, m, stream);
}
