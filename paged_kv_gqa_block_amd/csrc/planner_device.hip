// Device-side planner: builds the compact-workqueue plan on the GPU from the
// device copy of the row lengths, in exactly the layout the host planner
// writes (include/pkv.h), so the split and merge kernels read either.
//
// Method: PersistentKV summary pages, "Methodology / 1. Native block-table
// decode engine", "Row-local bounds" (page counts and split ranges from each
// row's real length) and "Compact workqueue" (only non-empty
// (row, kv-head, split) intervals).  Split rule as in the host planner:
// pps = max(1, ceil(T_max / S)) pages shared by the batch, ceil(T_i / pps)
// splits for row i, tasks in (row, kv_head, split) order.
//
// One 1024-thread workgroup: a max-reduction for T_max, an exclusive scan of
// the per-row task counts for the row offsets, then every thread writes the
// tasks of its rows.  Rows whose length lies outside [0, max_pages * P] are
// planned as empty and counted in *bad_rows.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_workqueue_kernel(
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ plan, int32_t* bad_rows, int batch,
    int hkv, int splits, int group, int page_size, int max_pages) {
  __shared__ int s_scan[kPlanThreads];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  int32_t* row_len = plan + PKV_PLAN_HEADER_WORDS;
  int32_t* row_pages = row_len + batch;
  int32_t* row_nsplit = row_pages + batch;
  int32_t* row_task_off = row_nsplit + batch;
  const int off_tasks = (PKV_PLAN_HEADER_WORDS + 4 * batch + 1 + 3) & ~3;
  int32_t* tasks = plan + off_tasks;
  const int64_t cap = int64_t(max_pages) * page_size;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // Pass 1: lengths, pages, T_max.
  int t_max = 0, bad = 0;
  for (int i = tid; i < batch; i += kPlanThreads) {
    int n = seq_lens[i];
    if (n < 0 || n > cap) {  // planned as an empty row
      n = 0;
      ++bad;
    }
    const int t = (n + page_size - 1) / page_size;
    row_len[i] = n;
    row_pages[i] = t;
    t_max = max(t_max, t);
  }
  s_scan[tid] = t_max;
  if (bad) atomicAdd(&s_bad, bad);
  __syncthreads();
  for (int d = kPlanThreads / 2; d > 0; d >>= 1) {
    if (tid < d) s_scan[tid] = max(s_scan[tid], s_scan[tid + d]);
    __syncthreads();
  }
  t_max = s_scan[0];
  const int pps = max(1, (t_max + splits - 1) / splits);
  __syncthreads();

  // Pass 2: per-thread chunk of consecutive rows; exclusive scan of task counts.
  const int chunk = (batch + kPlanThreads - 1) / kPlanThreads;
  const int r0 = min(batch, tid * chunk), r1 = min(batch, r0 + chunk);
  int local = 0;
  for (int i = r0; i < r1; ++i) local += hkv * ((row_pages[i] + pps - 1) / pps);
  s_scan[tid] = local;
  __syncthreads();
  for (int d = 1; d < kPlanThreads; d <<= 1) {  // inclusive Hillis-Steele scan
    const int v = (tid >= d) ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  int off = s_scan[tid] - local;
  const int n_tasks = s_scan[kPlanThreads - 1];

  // Pass 3: row arrays and tasks {row, kv_head << 16 | split, page_begin, token_end}.
  for (int i = r0; i < r1; ++i) {
    const int t = row_pages[i];
    const int ns = (t + pps - 1) / pps;
    const int n = row_len[i];
    row_nsplit[i] = ns;
    row_task_off[i] = off;
    for (int g = 0; g < hkv; ++g)
      for (int s = 0; s < ns; ++s) {
        const int pb = s * pps, pe = min(pb + pps, t);
        int4* dst = reinterpret_cast<int4*>(tasks) + off;
        *dst = make_int4(i, (g << 16) | s, pb, min(pe * page_size, n));
        ++off;
      }
  }
  if (tid == 0) {
    row_task_off[batch] = n_tasks;
    plan[kMagic] = PKV_PLAN_MAGIC;
    plan[kPath] = PKV_WORKQUEUE;
    plan[kBatch] = batch;
    plan[kNumKvHeads] = hkv;
    plan[kSplits] = splits;
    plan[kPagesPerSplit] = pps;
    plan[kNumTasks] = n_tasks;
    plan[kNumBuckets] = 0;
    plan[kNumStateSlots] = n_tasks;
    plan[kNumEmptySlots] = 0;
    plan[kOffTasks] = off_tasks;
    plan[kOffBuckets] = off_tasks + kTaskWords * n_tasks;
    plan[kOffBucketRows] = off_tasks + kTaskWords * n_tasks;
    plan[kTotalWords] = off_tasks + kTaskWords * n_tasks;
    plan[kWordPageSize] = page_size;
    plan[kWordGroup] = group;
  }
  __syncthreads();
  if (tid == 0 && bad_rows) *bad_rows = s_bad;
}

}  // namespace

pkv_status launch_plan_device(const pkv_problem& p, const int32_t* seq_lens_dev, int32_t splits,
                              int32_t* plan_dev, int32_t* bad_rows_dev, hipStream_t s) {
  hipLaunchKernelGGL(plan_workqueue_kernel, dim3(1), dim3(kPlanThreads), 0, s, seq_lens_dev,
                     plan_dev, bad_rows_dev, p.batch, p.num_kv_heads, splits,
                     p.num_q_heads / p.num_kv_heads, p.page_size, p.max_pages_per_row);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // namespace pkv
