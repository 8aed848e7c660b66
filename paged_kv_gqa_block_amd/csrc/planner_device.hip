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
// the per-row task counts (wave scans plus one cross-wave step) for the row
// offsets, kept in LDS; then task j is written by thread j mod 1024, which
// finds its row by binary search over the offsets.  Batches of up to
// kMaxDevicePlanRows rows.  Rows whose length lies outside [0, max_pages * P] are
// planned as empty and counted in *bad_rows.  The word after the plan is the
// persistent split kernel's work counter, zeroed here.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

__device__ __forceinline__ int valid_len(int n, int64_t cap) { return (n < 0 || n > cap) ? -1 : n; }

__global__ __launch_bounds__(kPlanThreads) void plan_workqueue_kernel(
    const int32_t* __restrict__ seq_lens, int32_t* __restrict__ plan, int32_t* bad_rows, int batch,
    int hkv, int splits, int group, int page_size, int max_pages) {
  __shared__ int s_off[kMaxDevicePlanRows + 1];  // row task offsets
  __shared__ int s_wave[kPlanWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int32_t* row_len = plan + PKV_PLAN_HEADER_WORDS;
  int32_t* row_pages = row_len + batch;
  int32_t* row_nsplit = row_pages + batch;
  int32_t* row_task_off = row_nsplit + batch;
  const int off_tasks = (PKV_PLAN_HEADER_WORDS + 4 * batch + 1 + 3) & ~3;
  int4* tasks = reinterpret_cast<int4*>(plan + off_tasks);
  const int64_t cap = int64_t(max_pages) * page_size;

  // Pass 1: this thread's chunk of consecutive rows; T_max and bad rows.
  const int chunk = (batch + kPlanThreads - 1) / kPlanThreads;
  const int r0 = min(batch, tid * chunk), r1 = min(batch, r0 + chunk);
  int t_max = 0, bad = 0;
  for (int i = r0; i < r1; ++i) {
    const int n = valid_len(seq_lens[i], cap);
    bad += (n < 0);
    t_max = max(t_max, (max(n, 0) + page_size - 1) / page_size);
  }
  t_max = wave_max_i(t_max);
  if (lane == 0) s_wave[wave] = t_max;
  __syncthreads();
  t_max = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) t_max = max(t_max, s_wave[w]);
  const int pps = max(1, (t_max + splits - 1) / splits);
  __syncthreads();

  // Pass 2: exclusive scan of per-row task counts (Hkv * splits of the row).
  int local = 0;
  for (int i = r0; i < r1; ++i) {
    const int n = max(valid_len(seq_lens[i], cap), 0);
    local += hkv * (((n + page_size - 1) / page_size + pps - 1) / pps);
  }
  const int incl = wave_scan_i(local);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int base = 0, n_tasks = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    base += (w < wave) ? s_wave[w] : 0;
    n_tasks += s_wave[w];
  }
  int off = base + incl - local;
  for (int i = r0; i < r1; ++i) {
    const int n0 = valid_len(seq_lens[i], cap);
    const int n = max(n0, 0);
    const int t = (n + page_size - 1) / page_size;
    const int ns = (t + pps - 1) / pps;
    row_len[i] = n;
    row_pages[i] = t;
    row_nsplit[i] = ns;
    row_task_off[i] = off;
    s_off[i] = off;
    off += hkv * ns;
  }
  if (tid == 0) {
    s_off[batch] = n_tasks;
    row_task_off[batch] = n_tasks;
  }
  __syncthreads();

  // Pass 3: task j goes to the last row whose offset is <= j (rows with no
  // tasks share their successor's offset), found by binary search in LDS.
  for (int j = tid; j < n_tasks; j += kPlanThreads) {
    int lo = 0, hi = batch;  // s_off[lo] <= j < s_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= j) lo = mid;
      else hi = mid;
    }
    const int row = lo;
    const int n = max(valid_len(seq_lens[row], cap), 0);
    const int t = (n + page_size - 1) / page_size;
    const int ns = (t + pps - 1) / pps;
    const int k = j - s_off[row];
    const int g = k / ns, sp = k - g * ns;
    const int pb = sp * pps, pe = min(pb + pps, t);
    tasks[j] = make_int4(row, (g << 16) | sp, pb, min(pe * page_size, n));
  }
  if (tid == 0) {
    // Alignment words between row_task_off and the task list.
    for (int i = PKV_PLAN_HEADER_WORDS + 4 * batch + 1; i < off_tasks; ++i) plan[i] = 0;
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
    plan[off_tasks + kTaskWords * n_tasks] = 0;  // work counter of the persistent kernel
  }
  // Bad-row count: per-wave sums, one atomic-free combine.
  const int b = wave_sum_i(bad);
  __syncthreads();
  if (lane == 0) s_wave[wave] = b;
  __syncthreads();
  if (tid == 0 && bad_rows) {
    int total = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) total += s_wave[w];
    *bad_rows = total;
  }
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
