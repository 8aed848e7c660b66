// Host planner: row-local split bounds, the compact workqueue, exact-length
// and power-of-two padded buckets, written into the plan buffer described in
// pkv.h.
//
// Follows the PersistentKV summary pages, "Methodology / 1. Native
// block-table decode engine": real per-row lengths set page counts and split
// ranges ("Row-local bounds"), the compact workqueue lists only non-empty
// (row, kv-head, split) intervals ("Compact workqueue"), and exact-length
// buckets are the alternative it replaces ("Results": launches per step).
// Where the pages leave the split rule open, the granule is
// ceil(T_max / S) pages shared by the whole batch for the workqueue, and
// ceil(T_b / S) per bucket for exact buckets.  Padded buckets group rows by
// their page count rounded up to a power of two (the coarse padding the
// pages' "Problem statement" contrasts with); the granule comes from the
// padded count, the split count of each row from its own pages.
#include <algorithm>
#include <cstring>
#include <numeric>

#include "pkv_internal.h"

namespace pkv {

pkv_status check_problem(const pkv_problem* p) {
  if (!p) return PKV_EINVAL;
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_pool_pages < 1 ||
      p->max_pages_per_row < 1)
    return PKV_EINVAL;
  if (p->num_q_heads % p->num_kv_heads != 0) return PKV_ESHAPE;
  if (p->num_q_heads / p->num_kv_heads > kMaxGroup) return PKV_ESHAPE;
  if (p->num_kv_heads > 32767) return PKV_ESHAPE;
  // Token indices (up to max_pages_per_row * 16, plus 15 when rounding up to
  // pages) are 32-bit in the kernels.
  if (p->max_pages_per_row > INT32_MAX / kPageSize) return PKV_ESHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return PKV_ESHAPE;
  if (p->page_size != kPageSize) return PKV_ESHAPE;
  if (p->dtype != PKV_F16 && p->dtype != PKV_BF16) return PKV_EDTYPE;
  if (p->kernel < PKV_KERNEL_AUTO || p->kernel > PKV_KERNEL_MFMA) return PKV_EINVAL;
  if (!(p->sm_scale == p->sm_scale)) return PKV_EINVAL;  // NaN scale
  return PKV_OK;
}

}  // namespace pkv

namespace pkv {

void order_rows(const int32_t* lens, int32_t b, bool padded, int32_t page_size, int32_t* order) {
  for (int32_t i = 0; i < b; ++i) order[i] = i;
  auto key = [&](int32_t r) -> int64_t {
    return padded ? pow2_ceil(static_cast<int32_t>(ceil_div(lens[r], page_size))) : lens[r];
  };
  // Ties broken by row index: the same order as a stable sort, without the
  // temporary buffer a stable sort may allocate.
  std::sort(order, order + b, [&](int32_t x, int32_t y) {
    const int64_t kx = key(x), ky = key(y);
    return kx < ky || (kx == ky && x < y);
  });
}

PlanCounts count_plan(const pkv_problem& p, const int32_t* lens, int32_t path, int32_t splits,
                      const int32_t* order) {
  PlanCounts c{};
  const int32_t b = p.batch, hkv = p.num_kv_heads, psz = p.page_size;
  int32_t t_max = 0;
  for (int32_t i = 0; i < b; ++i)
    t_max = std::max(t_max, static_cast<int32_t>(ceil_div(lens[i], psz)));
  if (path == PKV_WORKQUEUE) {
    c.pps = static_cast<int32_t>(std::max<int64_t>(1, ceil_div(t_max, splits)));
    for (int32_t i = 0; i < b; ++i) c.n_tasks += int64_t(hkv) * ceil_div(ceil_div(lens[i], psz), c.pps);
    c.n_slots = c.n_tasks;
    c.n_launches = 1 + (c.n_tasks > 0 ? 1 : 0);
    c.max_task_pages = std::min(c.pps, t_max);
  } else if (path == PKV_NOSPLIT) {
    for (int32_t i = 0; i < b; ++i) c.n_tasks += lens[i] > 0 ? hkv : 0;
    c.n_launches = 1;
    c.max_task_pages = t_max;
  } else {
    for_each_bucket(lens, b, path == PKV_PADDED, psz, splits, order,
                    [&](int32_t first, int32_t end, int32_t, int32_t, int32_t pps, int32_t,
                        int32_t max_pages) {
                      for (int32_t j = first; j < end; ++j) {
                        const int64_t ns = ceil_div(ceil_div(lens[order[j]], psz), pps);
                        c.n_tasks += hkv * ns;
                        c.n_empty += hkv * (splits - ns);
                      }
                      c.n_slots += int64_t(end - first) * hkv * splits;
                      c.max_task_pages = std::max(c.max_task_pages, std::min(pps, max_pages));
                      ++c.n_buckets;
                    });
    c.n_launches = 2 * c.n_buckets;
  }
  return c;
}

}  // namespace pkv

using namespace pkv;

namespace {

size_t words_upper_bound(const pkv_problem* p, int32_t path, int32_t splits) {
  const int64_t b = p->batch, hkv = p->num_kv_heads;
  const int64_t per_row = (path == PKV_NOSPLIT) ? 1 : splits;
  int64_t w = PKV_PLAN_HEADER_WORDS + 4 * b + 1;
  w = (w + 3) & ~int64_t(3);  // tasks start 16-byte aligned
  w += kTaskWords * hkv * b * per_row;
  w += kBucketWords * b + b;
  return static_cast<size_t>(w);
}

}  // namespace

extern "C" size_t pkv_plan_bytes(const pkv_problem* prob, int32_t path, int32_t max_splits) {
  if (check_problem(prob) != PKV_OK) return 0;
  if (path < PKV_BUCKETED || path > PKV_PADDED) return 0;
  if (max_splits < 1 || max_splits > 65535) return 0;
  return words_upper_bound(prob, path, max_splits) * sizeof(int32_t);
}

extern "C" pkv_status pkv_plan(const pkv_problem* prob, const int32_t* seq_lens_host,
                               int32_t path, int32_t max_splits, void* plan_host,
                               void* plan_dev, size_t plan_bytes, pkv_plan_info* info_out,
                               hipStream_t stream) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!seq_lens_host || !plan_host) return PKV_EINVAL;
  if (path < PKV_BUCKETED || path > PKV_PADDED) return PKV_EINVAL;
  if (max_splits < 1 || max_splits > 65535) return PKV_EINVAL;
  const int b = prob->batch, hkv = prob->num_kv_heads, psz = prob->page_size;
  const int64_t cap_tokens = int64_t(prob->max_pages_per_row) * psz;
  for (int i = 0; i < b; ++i)
    if (seq_lens_host[i] < 0 || seq_lens_host[i] > cap_tokens) return PKV_ERANGE;
  const size_t need = words_upper_bound(prob, path, max_splits) * sizeof(int32_t);
  if (plan_bytes < need) return PKV_ENOSPC;

  int32_t* w = static_cast<int32_t*>(plan_host);
  int32_t* row_len = w + PKV_PLAN_HEADER_WORDS;
  int32_t* row_pages = row_len + b;
  int32_t* row_nsplit = row_pages + b;
  int32_t* row_task_off = row_nsplit + b;
  int64_t off_tasks = (PKV_PLAN_HEADER_WORDS + 4 * int64_t(b) + 1 + 3) & ~int64_t(3);
  int32_t* tasks = w + off_tasks;
  // Alignment words between row_task_off and the task list.
  for (int64_t i = PKV_PLAN_HEADER_WORDS + 4 * int64_t(b) + 1; i < off_tasks; ++i) w[i] = 0;

  for (int i = 0; i < b; ++i) {
    row_len[i] = seq_lens_host[i];
    row_pages[i] = static_cast<int32_t>(ceil_div(seq_lens_host[i], psz));
  }

  // Bucketed and padded plans order the rows by bucket key.  The order is
  // built in the last B words the plan may use, then moved to its place in
  // the plan (bucket_rows) once the task count fixes that place; the library
  // allocates no memory of its own.
  const bool bucketed = (path == PKV_BUCKETED || path == PKV_PADDED);
  const int64_t upper = static_cast<int64_t>(words_upper_bound(prob, path, max_splits));
  int32_t* order = nullptr;
  if (bucketed) {
    order = w + upper - b;
    order_rows(seq_lens_host, b, path == PKV_PADDED, psz, order);
  }
  const PlanCounts c = count_plan(*prob, seq_lens_host, path, max_splits, order);
  if (c.n_slots > INT32_MAX || c.n_tasks > INT32_MAX) return PKV_ERANGE;
  const int64_t off_buckets = off_tasks + kTaskWords * c.n_tasks;
  const int64_t off_brows = off_buckets + kBucketWords * int64_t(c.n_buckets);
  const int64_t total = off_brows + (bucketed ? b : 0);
  if (total > INT32_MAX) return PKV_ERANGE;  // header offsets are 32-bit words
  if (bucketed) {
    std::memmove(w + off_brows, order, size_t(b) * sizeof(int32_t));
    order = w + off_brows;  // tasks and buckets are written below this point
  }

  int64_t n_tasks = 0;
  // Word 3 is the task's token end min(pe * P, N_row), from which the
  // kernels get both the page end and the real tokens of the last page.
  auto push_task = [&](int row, int g, int s, int pb, int pe) {
    int32_t* t = tasks + kTaskWords * n_tasks;
    t[0] = row;
    t[1] = (g << 16) | s;
    t[2] = pb;
    t[3] = static_cast<int32_t>(std::min<int64_t>(int64_t(pe) * psz, seq_lens_host[row]));
    ++n_tasks;
  };

  if (path == PKV_WORKQUEUE) {
    for (int i = 0; i < b; ++i) {
      row_nsplit[i] = static_cast<int32_t>(ceil_div(row_pages[i], c.pps));
      row_task_off[i] = static_cast<int32_t>(n_tasks);
      for (int g = 0; g < hkv; ++g)
        for (int s = 0; s < row_nsplit[i]; ++s)
          push_task(i, g, s, s * c.pps, std::min((s + 1) * c.pps, row_pages[i]));
    }
    row_task_off[b] = static_cast<int32_t>(n_tasks);
  } else if (bucketed) {
    int32_t* bw = w + off_buckets;
    int32_t k = 0;
    for_each_bucket(seq_lens_host, b, path == PKV_PADDED, psz, max_splits, order,
                    [&](int32_t first, int32_t end, int32_t len_word, int32_t pages, int32_t pps,
                        int32_t nsplit, int32_t) {
                      for (int32_t j = first; j < end; ++j) {
                        const int row = order[j];
                        // Row-local bound: the row's own pages set its split count.
                        row_nsplit[row] = static_cast<int32_t>(ceil_div(row_pages[row], pps));
                        row_task_off[row] = static_cast<int32_t>(n_tasks);
                        for (int g = 0; g < hkv; ++g)
                          for (int s = 0; s < row_nsplit[row]; ++s)
                            push_task(row, g, s, s * pps, std::min((s + 1) * pps, row_pages[row]));
                      }
                      int32_t* e = bw + kBucketWords * k++;
                      e[0] = len_word;
                      e[1] = pages;
                      e[2] = pps;
                      e[3] = nsplit;
                      e[4] = end - first;
                      e[5] = first;
                      e[6] = 0;
                      e[7] = 0;
                    });
    row_task_off[b] = static_cast<int32_t>(n_tasks);
  } else {  // PKV_NOSPLIT
    for (int i = 0; i < b; ++i) {
      row_nsplit[i] = row_pages[i] ? 1 : 0;
      row_task_off[i] = static_cast<int32_t>(n_tasks);
      if (row_pages[i])
        for (int g = 0; g < hkv; ++g) push_task(i, g, 0, 0, row_pages[i]);
    }
    row_task_off[b] = static_cast<int32_t>(n_tasks);
  }
  if (n_tasks != c.n_tasks) return PKV_EINVAL;  // counting and writing disagree: a bug

  w[kMagic] = PKV_PLAN_MAGIC;
  w[kPath] = path;
  w[kBatch] = b;
  w[kNumKvHeads] = hkv;
  w[kSplits] = max_splits;
  w[kPagesPerSplit] = path == PKV_WORKQUEUE ? c.pps : 0;
  w[kNumTasks] = static_cast<int32_t>(n_tasks);
  w[kNumBuckets] = c.n_buckets;
  w[kNumStateSlots] = static_cast<int32_t>(c.n_slots);
  w[kNumEmptySlots] = static_cast<int32_t>(c.n_empty);
  w[kOffTasks] = static_cast<int32_t>(off_tasks);
  w[kOffBuckets] = static_cast<int32_t>(off_buckets);
  w[kOffBucketRows] = static_cast<int32_t>(off_brows);
  w[kTotalWords] = static_cast<int32_t>(total);
  w[kWordPageSize] = psz;
  w[kWordGroup] = prob->num_q_heads / hkv;

  if (info_out) {
    pkv_status s2 = pkv_plan_get_info(prob, plan_host, info_out);
    if (s2 != PKV_OK) return s2;
  }
  if (plan_dev) {
    if (hipMemcpyAsync(plan_dev, plan_host, size_t(total) * sizeof(int32_t),
                       hipMemcpyHostToDevice, stream) != hipSuccess)
      return PKV_EHIP;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_plan_get_info(const pkv_problem* prob, const void* plan_host,
                                        pkv_plan_info* info) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!plan_host || !info) return PKV_EINVAL;
  const int32_t* w = static_cast<const int32_t*>(plan_host);
  if (w[kMagic] != PKV_PLAN_MAGIC) return PKV_EINVAL;
  if (w[kBatch] != prob->batch || w[kNumKvHeads] != prob->num_kv_heads ||
      w[kWordPageSize] != prob->page_size || w[kWordGroup] != prob->num_q_heads / prob->num_kv_heads)
    return PKV_ESHAPE;
  const int32_t path = w[kPath];
  const int64_t g = prob->num_q_heads / prob->num_kv_heads;
  const int32_t* row_len = w + PKV_PLAN_HEADER_WORDS;
  int64_t tokens = 0;
  for (int i = 0; i < prob->batch; ++i) tokens += row_len[i];
  std::memset(info, 0, sizeof(*info));
  info->path = path;
  info->n_tasks = w[kNumTasks];
  info->n_buckets = w[kNumBuckets];
  info->n_state_slots = w[kNumStateSlots];
  info->n_empty_slots = w[kNumEmptySlots];
  info->splits = w[kSplits];
  info->pages_per_split = w[kPagesPerSplit];
  if (path == PKV_WORKQUEUE)
    info->n_launches = 1 + (w[kNumTasks] > 0 ? 1 : 0);
  else if (path == PKV_BUCKETED || path == PKV_PADDED)
    info->n_launches = 2 * w[kNumBuckets];
  else
    info->n_launches = 1;
  info->kv_bytes = tokens * prob->num_kv_heads * prob->head_dim * 2 * 2;
  info->merge_state_bytes = 2 * int64_t(w[kNumStateSlots]) * g * (prob->head_dim + 2) * 4;
  info->plan_bytes = int64_t(w[kTotalWords]) * 4;
  const int32_t* tasks = w + w[kOffTasks];
  for (int32_t j = 0; j < w[kNumTasks]; ++j) {
    const int32_t pages = (tasks[kTaskWords * j + 3] + prob->page_size - 1) / prob->page_size -
                          tasks[kTaskWords * j + 2];
    info->max_task_pages = std::max(info->max_task_pages, pages);
  }
  return PKV_OK;
}
