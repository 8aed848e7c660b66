// Internal declarations shared by the host planner, the API layer and the
// kernel launchers of libpkv.  Not part of the public ABI (see include/pkv.h).
#pragma once

#include <algorithm>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Word offsets inside the plan header (layout documented in pkv.h).
enum PlanWord : int {
  kMagic = 0,
  kPath = 1,
  kBatch = 2,
  kNumKvHeads = 3,
  kSplits = 4,
  kPagesPerSplit = 5,
  kNumTasks = 6,
  kNumBuckets = 7,
  kNumStateSlots = 8,
  kNumEmptySlots = 9,
  kOffTasks = 10,
  kOffBuckets = 11,
  kOffBucketRows = 12,
  kTotalWords = 13,
  kWordPageSize = 14,
  kWordGroup = 15,
};

constexpr int kBucketWords = 8;
constexpr int kTaskWords = 4;
constexpr int kPageSize = 16;
constexpr int kMaxGroup = 16;
constexpr int kMaxDevicePlanRows = 16384;  // batch limit of the device-side planner

// Counters of a plan, computed from the lengths without writing it (the
// host planner's counting pass; the cost model's features use it too).
struct PlanCounts {
  int64_t n_tasks;         // non-empty (row, kv head, split) tasks
  int64_t n_slots;         // partial-state slots of the split launches
  int64_t n_empty;         // slots holding only a neutral state
  int32_t n_buckets;       // bucket launches (exact or padded buckets)
  int32_t n_launches;      // kernel launches per step
  int32_t pps;             // WORKQUEUE split granule (pages)
  int32_t max_task_pages;  // pages of the longest task
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Smallest power of two >= t (0 for t = 0).
inline int32_t pow2_ceil(int32_t t) {
  int32_t p = 1;
  if (t == 0) return 0;
  while (p < t) p <<= 1;
  return p;
}

// Walks the buckets of a bucketed or padded plan in `order`:
// f(first, end, length_word, bucket_pages, pps, bucket_nsplit, max_row_pages)
// for the run order[first, end) of rows sharing one bucket key.
template <class F>
void for_each_bucket(const int32_t* lens, int32_t b, bool padded, int32_t page_size,
                     int32_t splits, const int32_t* order, F&& f) {
  for (int32_t k = 0; k < b;) {
    const int32_t t0 = static_cast<int32_t>(ceil_div(lens[order[k]], page_size));
    const int64_t key = padded ? pow2_ceil(t0) : lens[order[k]];
    int32_t e = k, max_pages = 0;
    while (e < b) {
      const int32_t r = order[e];
      const int32_t t = static_cast<int32_t>(ceil_div(lens[r], page_size));
      if ((padded ? pow2_ceil(t) : lens[r]) != key) break;
      max_pages = std::max(max_pages, t);
      ++e;
    }
    const int32_t pages = padded ? static_cast<int32_t>(key) : t0;
    const int32_t pps = static_cast<int32_t>(std::max<int64_t>(1, ceil_div(pages, splits)));
    const int32_t nsplit = static_cast<int32_t>(ceil_div(pages, pps));
    f(k, e, padded ? -1 : lens[order[k]], pages, pps, nsplit, max_pages);
    k = e;
  }
}

// Rows in bucket order: ascending key (the exact length, or for padded
// buckets the page count rounded up to a power of two), ties by row index.
void order_rows(const int32_t* lens, int32_t b, bool padded, int32_t page_size, int32_t* order);
// Counters of the plan pkv_plan would write; `order` (from order_rows) is
// read for BUCKETED and PADDED only.  Lengths must already be validated.
PlanCounts count_plan(const pkv_problem& p, const int32_t* lens, int32_t path, int32_t splits,
                      const int32_t* order);

// Which grid a split-kernel launch walks.
enum SplitMode : int {
  kModeWorkqueue = 0,
  kModeBucket = 1,
  kModeNoSplit = 2,
  kModePersistent = 3,  // persistent grid over a device-built plan
  kModeLens = 4,        // persistent grid, tasks derived from the lengths in-kernel
};
constexpr int kMaxLensRows = 1024;  // batch limit of the self-planned step

// Everything a split / no-split kernel needs; passed by value as a kernel
// argument.  Pointers are device pointers.
struct SplitArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* tasks;        // workqueue: tasks[n][4] {row, g<<16|s, page_begin, tok_end}
  int32_t* device_plan;        // persistent: device-built plan; its task count and the
                               // work counter at word [kTotalWords] are read on the device
  const int32_t* bucket_rows;  // bucket: rows of this bucket
  const int32_t* row_len;      // bucket: the plan's row lengths N_i
  float* st_m;
  float* st_l;
  float* st_o;
  void* out;    // no-split
  float* lse;   // no-split, may be null
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;      // G = Hq / Hkv, set by launch_split (no division on the device)
  int32_t max_pages;  // block-table row stride
  int32_t splits;     // bucket: S (slot stride)
  int32_t bucket_pps;
  int32_t bucket_nsplit;
  int32_t bucket_pages;
  int32_t bucket_len;   // bucket: the rows' common length N_b, or -1 when
                        // they differ (padded bucket: lengths from row_len)
  int32_t bucket_row0;  // bucket: its only row when it has one, else -1
  int32_t num_items;    // grid items (tasks, bucket slots or rows * Hkv)
  int32_t xcd_nsplit;   // workqueue: the split count every row shares when the
                        // XCD-affine launch order applies (launch_item), else 0
  float scale_log2;   // sm_scale * log2(e)
  int32_t num_rows;        // lens mode: B
  int32_t* work_counter;   // lens mode: task claim counter (zero between steps)
};

struct MergeArgs {
  const float* st_m;
  const float* st_l;
  const float* st_o;
  const int32_t* row_nsplit;    // workqueue
  const int32_t* row_task_off;  // workqueue
  const int32_t* bucket_rows;   // bucket: rows of this bucket
  void* out;
  float* lse;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;      // G = Hq / Hkv, set by launch_merge
  int32_t splits;     // bucket slot stride S
  int32_t num_rows;   // rows covered by this launch
  int32_t mode;       // kModeWorkqueue or kModeBucket
  int32_t bucket_row0;  // bucket: its only row when it has one, else -1
  int32_t* device_plan;  // device-planned step: the merge resets its work counter; else null
  int32_t uniform_nsplit;  // workqueue: the split count every row shares (> 0), else 0
  const int32_t* seq_lens;  // lens mode: device lengths (slots derived in-kernel)
  int32_t max_pages;        // lens mode: block-table row stride (length bound)
  int32_t* work_counter;    // lens mode: the split kernel's claim counter, reset here
};

struct AppendArgs {
  const void* k_new;  // [B][Hkv][d]
  const void* v_new;
  const int32_t* block_table;
  const int32_t* positions;  // [B]: slot to write; < 0 = inactive row
  void* k_pool;
  void* v_pool;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_pages;
};

// Kernel launchers (HIP translation units).  Return PKV_OK or PKV_EHIP.
pkv_status launch_split(const pkv_problem& prob, int mode, int kernel, const SplitArgs& args,
                        int grid, hipStream_t stream);
pkv_status launch_merge(const pkv_problem& prob, const MergeArgs& args, hipStream_t stream);
pkv_status launch_append(const AppendArgs& args, int batch, hipStream_t stream);
pkv_status launch_plan_device(const pkv_problem& prob, const int32_t* seq_lens_dev, int32_t splits,
                              int32_t* plan_dev, int32_t* bad_rows_dev, hipStream_t stream);

// Shape checks shared by plan / decode / merge.
pkv_status check_problem(const pkv_problem* prob);

}  // namespace pkv
