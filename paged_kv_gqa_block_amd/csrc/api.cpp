// Public entry points pkv_decode, pkv_merge, pkv_policy and pkv_status_str:
// argument validation on the host, then kernel launches on the caller's
// stream.  The planner entry points live in planner.cpp.
#include <algorithm>
#include <cmath>

#include "launch_limits.h"
#include "pkv_internal.h"
#include "selfplan_args.h"

using namespace pkv;

namespace {

// Checks that the plan in plan_host was made for this problem; returns its
// header words through `w`.
pkv_status check_plan(const pkv_problem* prob, const void* plan_host, const int32_t** w_out) {
  if (!plan_host) return PKV_EINVAL;
  const int32_t* w = static_cast<const int32_t*>(plan_host);
  if (w[kMagic] != PKV_PLAN_MAGIC) return PKV_EINVAL;
  if (w[kBatch] != prob->batch || w[kNumKvHeads] != prob->num_kv_heads ||
      w[kWordPageSize] != prob->page_size || w[kWordGroup] != prob->num_q_heads / prob->num_kv_heads)
    return PKV_ESHAPE;
  if (w[kPath] < PKV_BUCKETED || w[kPath] > PKV_PADDED) return PKV_EINVAL;
  *w_out = w;
  return PKV_OK;
}

constexpr float kLog2e = 1.4426950408889634f;

// Workgroups per CU of a persistent grid: the split kernel's resident count.
// Matrix cores: three for G <= 8 (held to 168 registers), two for G = 16.
// Vector ALU: two (one or two resident, by head size and group; a grid
// larger than the resident set only delays the surplus workgroups' first
// tasks).
int persistent_per_cu(const pkv_problem* p) {
  const bool mfma = p->kernel == PKV_KERNEL_MFMA || (p->kernel == PKV_KERNEL_AUTO && p->head_dim == 128);
  if (!mfma) return 2;
  return (p->num_q_heads / p->num_kv_heads <= 8) ? 3 : 2;
}

// Shapes the chosen split kernel covers: matrix cores d = 128, G <= 16;
// vector ALU d = 64 or 128, G <= 8; AUTO is matrix cores for d = 128.
pkv_status check_kernel_shape(const pkv_problem* p) {
  const int g = p->num_q_heads / p->num_kv_heads;
  const bool mfma = p->kernel == PKV_KERNEL_MFMA || (p->kernel == PKV_KERNEL_AUTO && p->head_dim == 128);
  if (mfma) return (p->head_dim == 128 && g <= kMaxGroup) ? PKV_OK : PKV_ESHAPE;
  return g <= 8 ? PKV_OK : PKV_ESHAPE;
}

}  // namespace

extern "C" pkv_status pkv_decode(const pkv_problem* prob, const void* plan_host,
                                 const void* plan_dev, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_table,
                                 const int32_t* seq_lens_dev, float* st_m, float* st_l,
                                 float* st_o, void* out, float* lse, hipStream_t stream) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  const int32_t* w = nullptr;
  st = check_plan(prob, plan_host, &w);
  if (st != PKV_OK) return st;
  (void)seq_lens_dev;  // every path takes the row lengths from the plan
  if (!plan_dev || !q || !k_pool || !v_pool || !block_table) return PKV_EINVAL;
  st = check_kernel_shape(prob);
  if (st != PKV_OK) return st;
  const int path = w[kPath];
  if (path == PKV_NOSPLIT) {
    if (!out) return PKV_EINVAL;
  } else if (w[kNumStateSlots] > 0 && (!st_m || !st_l || !st_o)) {
    return PKV_EINVAL;
  }

  SplitArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.st_m = st_m;
  a.st_l = st_l;
  a.st_o = st_o;
  a.out = out;
  a.lse = lse;
  a.num_q_heads = prob->num_q_heads;
  a.num_kv_heads = prob->num_kv_heads;
  a.max_pages = prob->max_pages_per_row;
  a.splits = w[kSplits];
  a.scale_log2 = prob->sm_scale * kLog2e;
  const int32_t* dev = static_cast<const int32_t*>(plan_dev);
  // The no-split kernel reads each row's length from the plan's row_len
  // array: the lengths pkv_plan validated, the same ones every other path
  // uses.
  a.seq_lens = dev + PKV_PLAN_HEADER_WORDS;

  if (path == PKV_WORKQUEUE) {
    const int n = w[kNumTasks];
    if (n == 0) return PKV_OK;
    if (n > kMaxGridGroups) return PKV_ERANGE;
    a.tasks = dev + w[kOffTasks];
    a.num_items = n;
    // XCD-affine launch order (launch_item in split_common.h) when every row
    // has the same split count u, the tasks are exactly B * Hkv * u and
    // B * Hkv is a multiple of 8.
    const int b = prob->batch;
    const int32_t* ns = w + PKV_PLAN_HEADER_WORDS + 2 * b;
    int32_t u = ns[0];
    for (int r = 1; r < b && u > 0; ++r)
      if (ns[r] != u) u = 0;
    const int64_t pairs = int64_t(b) * prob->num_kv_heads;
    a.xcd_nsplit = (u > 0 && pairs % 8 == 0 && pairs * u == n) ? u : 0;
    return launch_split(*prob, kModeWorkqueue, prob->kernel, a, n, stream);
  }
  if (path == PKV_NOSPLIT) {
    const int64_t n = int64_t(prob->batch) * prob->num_kv_heads;
    if (n > kMaxGridGroups) return PKV_ERANGE;
    a.num_items = static_cast<int32_t>(n);
    return launch_split(*prob, kModeNoSplit, prob->kernel, a, static_cast<int>(n), stream);
  }
  // BUCKETED / PADDED: one rectangular rows_b x Hkv x S launch per bucket.
  // Rows of a padded bucket differ in length: the kernel takes each row's
  // length from the plan's row_len array (bucket length word -1).
  a.row_len = dev + PKV_PLAN_HEADER_WORDS;
  const int32_t* bw = w + w[kOffBuckets];
  for (int k = 0; k < w[kNumBuckets]; ++k) {  // every launch size, before the first launch
    const int64_t rows = bw[kBucketWords * k + 4];
    if (rows > kMaxBucketRows || rows * prob->num_kv_heads * w[kSplits] > kMaxGridGroups)
      return PKV_ERANGE;
  }
  for (int k = 0; k < w[kNumBuckets]; ++k) {
    const int32_t* e = bw + kBucketWords * k;
    const int64_t items = int64_t(e[4]) * prob->num_kv_heads * w[kSplits];
    a.bucket_len = e[0];
    a.bucket_pages = e[1];
    a.bucket_pps = e[2];
    a.bucket_nsplit = e[3];
    a.bucket_rows = dev + w[kOffBucketRows] + e[5];
    a.bucket_row0 = (e[4] == 1) ? w[w[kOffBucketRows] + e[5]] : -1;
    a.num_items = static_cast<int32_t>(items);
    st = launch_split(*prob, kModeBucket, prob->kernel, a, static_cast<int>(items), stream);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_merge(const pkv_problem* prob, const void* plan_host,
                                const void* plan_dev, const float* st_m, const float* st_l,
                                const float* st_o, void* out, float* lse, hipStream_t stream) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  const int32_t* w = nullptr;
  st = check_plan(prob, plan_host, &w);
  if (st != PKV_OK) return st;
  const int path = w[kPath];
  if (path == PKV_NOSPLIT) return PKV_OK;
  if (!plan_dev || !out) return PKV_EINVAL;
  if (w[kNumStateSlots] > 0 && (!st_m || !st_l || !st_o)) return PKV_EINVAL;
  const int32_t* dev = static_cast<const int32_t*>(plan_dev);
  const int b = prob->batch;
  // One launch covers at most B rows x Hq heads (workqueue: exactly that).
  if (int64_t(b) * prob->num_q_heads > kMaxGridGroups) return PKV_ERANGE;

  MergeArgs a{};
  a.st_m = st_m;
  a.st_l = st_l;
  a.st_o = st_o;
  a.out = out;
  a.lse = lse;
  a.num_q_heads = prob->num_q_heads;
  a.num_kv_heads = prob->num_kv_heads;
  a.splits = w[kSplits];
  if (path == PKV_WORKQUEUE) {
    a.row_nsplit = dev + PKV_PLAN_HEADER_WORDS + 2 * b;
    a.row_task_off = dev + PKV_PLAN_HEADER_WORDS + 3 * b;
    a.num_rows = b;
    a.mode = kModeWorkqueue;
    a.bucket_row0 = -1;
    // When all rows share one split count, the merge derives each row's
    // first state slot from the row index (read from the host plan here).
    const int32_t* ns = w + PKV_PLAN_HEADER_WORDS + 2 * b;
    a.uniform_nsplit = ns[0];
    for (int r = 1; r < b && a.uniform_nsplit > 0; ++r)
      if (ns[r] != a.uniform_nsplit) a.uniform_nsplit = 0;
    return launch_merge(*prob, a, stream);
  }
  const int32_t* bw = w + w[kOffBuckets];
  for (int k = 0; k < w[kNumBuckets]; ++k) {
    const int32_t* e = bw + kBucketWords * k;
    a.bucket_rows = dev + w[kOffBucketRows] + e[5];
    a.bucket_row0 = (e[4] == 1) ? w[w[kOffBucketRows] + e[5]] : -1;
    a.num_rows = e[4];
    a.mode = kModeBucket;
    st = launch_merge(*prob, a, stream);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

// ---- device-planned workqueue step ----------------------------------------

namespace {

int32_t off_tasks_words(int32_t batch) {
  return (PKV_PLAN_HEADER_WORDS + 4 * batch + 1 + 3) & ~3;
}

}  // namespace

extern "C" pkv_status pkv_plan_device(const pkv_problem* prob, const int32_t* seq_lens_dev,
                                      int32_t max_splits, void* plan_dev, size_t plan_bytes,
                                      int32_t* bad_rows_dev, hipStream_t stream) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!seq_lens_dev || !plan_dev) return PKV_EINVAL;
  if (max_splits < 1 || max_splits > 65535) return PKV_EINVAL;
  if (prob->batch > kMaxDevicePlanRows) return PKV_ERANGE;
  // The kernel counts tasks and plan words in 32 bits: bound them by the
  // largest plan this problem can have (every row at its full split count).
  const size_t need = pkv_plan_bytes(prob, PKV_WORKQUEUE, max_splits);
  if (need / sizeof(int32_t) > size_t(INT32_MAX)) return PKV_ERANGE;
  if (plan_bytes < need) return PKV_ENOSPC;
  return launch_plan_device(*prob, seq_lens_dev, max_splits, static_cast<int32_t*>(plan_dev),
                            bad_rows_dev, stream);
}

extern "C" pkv_status pkv_decode_device(const pkv_problem* prob, const void* plan_dev,
                                        int32_t max_splits, const void* q, const void* k_pool,
                                        const void* v_pool, const int32_t* block_table,
                                        float* st_m, float* st_l, float* st_o,
                                        hipStream_t stream) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!plan_dev || !q || !k_pool || !v_pool || !block_table || !st_m || !st_l || !st_o)
    return PKV_EINVAL;
  if (max_splits < 1 || max_splits > 65535) return PKV_EINVAL;
  st = check_kernel_shape(prob);
  if (st != PKV_OK) return st;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return PKV_EHIP;
  const int32_t* plan = static_cast<const int32_t*>(plan_dev);
  SplitArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.st_m = st_m;
  a.st_l = st_l;
  a.st_o = st_o;
  a.num_q_heads = prob->num_q_heads;
  a.num_kv_heads = prob->num_kv_heads;
  a.max_pages = prob->max_pages_per_row;
  a.splits = max_splits;
  a.scale_log2 = prob->sm_scale * kLog2e;
  a.tasks = plan + off_tasks_words(prob->batch);
  // Task count and work counter (word [total_words], after the task list) are
  // located from the plan header on the device.
  a.device_plan = const_cast<int32_t*>(plan);
  a.bucket_row0 = -1;
  // As many workgroups as can be resident, never more than the largest task
  // count.
  const int per_cu = persistent_per_cu(prob);
  const int64_t upper = int64_t(prob->batch) * prob->num_kv_heads * max_splits;
  const int grid = static_cast<int>(std::min<int64_t>(upper, int64_t(per_cu) * cus));
  a.num_items = grid;
  return launch_split(*prob, kModePersistent, prob->kernel, a, grid, stream);
}

extern "C" pkv_status pkv_merge_device(const pkv_problem* prob, const void* plan_dev,
                                       const float* st_m, const float* st_l, const float* st_o,
                                       void* out, float* lse, hipStream_t stream) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!plan_dev || !st_m || !st_l || !st_o || !out) return PKV_EINVAL;
  const int32_t* plan = static_cast<const int32_t*>(plan_dev);
  const int b = prob->batch;
  MergeArgs a{};
  a.st_m = st_m;
  a.st_l = st_l;
  a.st_o = st_o;
  a.out = out;
  a.lse = lse;
  a.num_q_heads = prob->num_q_heads;
  a.num_kv_heads = prob->num_kv_heads;
  a.row_nsplit = plan + PKV_PLAN_HEADER_WORDS + 2 * b;
  a.row_task_off = plan + PKV_PLAN_HEADER_WORDS + 3 * b;
  a.num_rows = b;
  a.mode = kModeWorkqueue;
  a.bucket_row0 = -1;
  a.device_plan = const_cast<int32_t*>(plan);  // the merge resets the work counter
  return launch_merge(*prob, a, stream);
}

// ---- self-planned workqueue step --------------------------------------------

namespace pkv {

pkv_status check_selfplan_step(const pkv_problem* prob, const int32_t* seq_lens_dev,
                               int32_t max_splits) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!seq_lens_dev) return PKV_EINVAL;
  if (max_splits < 1 || max_splits > 65535) return PKV_EINVAL;
  if (prob->batch > kMaxLensRows) return PKV_ERANGE;
  // Task indices and slots are 32-bit: bound the largest task count.
  if (int64_t(prob->batch) * prob->num_kv_heads * max_splits > INT32_MAX) return PKV_ERANGE;
  return check_kernel_shape(prob);
}

SplitArgs selfplan_split_args(const pkv_problem* prob, const int32_t* seq_lens_dev,
                              int32_t max_splits, int32_t* work_counter_dev, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_table, float* st_m, float* st_l, float* st_o) {
  SplitArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens_dev;
  a.st_m = st_m;
  a.st_l = st_l;
  a.st_o = st_o;
  a.num_q_heads = prob->num_q_heads;
  a.num_kv_heads = prob->num_kv_heads;
  a.max_pages = prob->max_pages_per_row;
  a.splits = max_splits;
  a.scale_log2 = prob->sm_scale * kLog2e;
  a.bucket_row0 = -1;
  a.num_rows = prob->batch;
  a.work_counter = work_counter_dev;
  return a;
}

MergeArgs selfplan_merge_args(const pkv_problem* prob, const int32_t* seq_lens_dev,
                              int32_t max_splits, int32_t* work_counter_dev, const float* st_m,
                              const float* st_l, const float* st_o, void* out, float* lse) {
  MergeArgs a{};
  a.st_m = st_m;
  a.st_l = st_l;
  a.st_o = st_o;
  a.out = out;
  a.lse = lse;
  a.num_q_heads = prob->num_q_heads;
  a.num_kv_heads = prob->num_kv_heads;
  a.splits = max_splits;
  a.num_rows = prob->batch;
  a.mode = kModeLens;
  a.bucket_row0 = -1;
  a.seq_lens = seq_lens_dev;
  a.max_pages = prob->max_pages_per_row;
  a.work_counter = work_counter_dev;  // the merge resets the split kernel's counter
  return a;
}

}  // namespace pkv

extern "C" pkv_status pkv_decode_selfplan(const pkv_problem* prob, const int32_t* seq_lens_dev,
                                          int32_t max_splits, int32_t* work_counter_dev,
                                          const void* q, const void* k_pool, const void* v_pool,
                                          const int32_t* block_table, float* st_m, float* st_l,
                                          float* st_o, hipStream_t stream) {
  pkv_status st = check_selfplan_step(prob, seq_lens_dev, max_splits);
  if (st != PKV_OK) return st;
  if (!work_counter_dev) return PKV_EINVAL;
  if (!q || !k_pool || !v_pool || !block_table || !st_m || !st_l || !st_o) return PKV_EINVAL;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return PKV_EHIP;
  SplitArgs a = selfplan_split_args(prob, seq_lens_dev, max_splits, work_counter_dev, q, k_pool,
                                    v_pool, block_table, st_m, st_l, st_o);
  // The persistent grid of pkv_decode_device.
  const int per_cu = persistent_per_cu(prob);
  const int64_t upper = int64_t(prob->batch) * prob->num_kv_heads * max_splits;
  const int grid = static_cast<int>(std::min<int64_t>(upper, int64_t(per_cu) * cus));
  a.num_items = grid;
  return launch_split(*prob, kModeLens, prob->kernel, a, grid, stream);
}

extern "C" pkv_status pkv_merge_selfplan(const pkv_problem* prob, const int32_t* seq_lens_dev,
                                         int32_t max_splits, int32_t* work_counter_dev,
                                         const float* st_m, const float* st_l, const float* st_o,
                                         void* out, float* lse, hipStream_t stream) {
  pkv_status st = check_selfplan_step(prob, seq_lens_dev, max_splits);
  if (st != PKV_OK) return st;
  if (!work_counter_dev) return PKV_EINVAL;
  if (!st_m || !st_l || !st_o || !out) return PKV_EINVAL;
  MergeArgs a = selfplan_merge_args(prob, seq_lens_dev, max_splits, work_counter_dev, st_m, st_l,
                                    st_o, out, lse);
  return launch_merge(*prob, a, stream);
}

extern "C" pkv_status pkv_append_kv(const pkv_problem* prob, const void* k_new,
                                    const void* v_new, const int32_t* block_table,
                                    const int32_t* positions_dev, void* k_pool, void* v_pool,
                                    hipStream_t stream) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!k_new || !v_new || !block_table || !positions_dev || !k_pool || !v_pool)
    return PKV_EINVAL;
  // One workgroup per (row, KV head).
  if (int64_t(prob->batch) * prob->num_kv_heads > kMaxGridGroups) return PKV_ERANGE;
  AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_table = block_table;
  a.positions = positions_dev;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_kv_heads = prob->num_kv_heads;
  a.head_dim = prob->head_dim;
  a.max_pages = prob->max_pages_per_row;
  return launch_append(a, prob->batch, stream);
}

extern "C" pkv_status pkv_policy(const pkv_policy_table* table, int32_t batch, int32_t max_len,
                                 int32_t* path_out, int32_t* splits_out) {
  if (!table || !path_out || !splits_out || table->n_rules < 0) return PKV_EINVAL;
  if (table->n_rules > 0 && !table->rules) return PKV_EINVAL;
  for (int r = 0; r < table->n_rules; ++r) {
    const int32_t* e = table->rules + 6 * r;
    if (e[4] < PKV_BUCKETED || e[4] > PKV_PADDED || e[5] < 1) return PKV_EINVAL;
  }
  for (int r = 0; r < table->n_rules; ++r) {
    const int32_t* e = table->rules + 6 * r;
    if (e[0] <= batch && batch <= e[1] && e[2] <= max_len && max_len <= e[3]) {
      *path_out = e[4];
      *splits_out = e[5];
      return PKV_OK;
    }
  }
  return PKV_ERANGE;
}

extern "C" const char* pkv_status_str(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_ESHAPE: return "unsupported or mismatched shape";
    case PKV_EDTYPE: return "unsupported dtype";
    case PKV_ERANGE: return "value out of range";
    case PKV_ENOSPC: return "plan buffer too small";
    case PKV_EHIP: return "HIP call or kernel launch failed";
    default: return "unknown status";
  }
}
