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
#include <vector>

#include "pkv_internal.h"

namespace pkv {
namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Smallest power of two >= t (0 for t = 0).
inline int32_t pow2_ceil(int32_t t) {
  int32_t p = 1;
  if (t == 0) return 0;
  while (p < t) p <<= 1;
  return p;
}

}  // namespace

pkv_status check_problem(const pkv_problem* p) {
  if (!p) return PKV_EINVAL;
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_pool_pages < 1 ||
      p->max_pages_per_row < 1)
    return PKV_EINVAL;
  if (p->num_q_heads % p->num_kv_heads != 0) return PKV_ESHAPE;
  if (p->num_q_heads / p->num_kv_heads > kMaxGroup) return PKV_ESHAPE;
  if (p->num_kv_heads > 32767) return PKV_ESHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return PKV_ESHAPE;
  if (p->page_size != kPageSize) return PKV_ESHAPE;
  if (p->dtype != PKV_F16 && p->dtype != PKV_BF16) return PKV_EDTYPE;
  if (p->kernel < PKV_KERNEL_AUTO || p->kernel > PKV_KERNEL_MFMA) return PKV_EINVAL;
  if (!(p->sm_scale == p->sm_scale)) return PKV_EINVAL;  // NaN scale
  return PKV_OK;
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

  int32_t t_max = 0;
  for (int i = 0; i < b; ++i) {
    row_len[i] = seq_lens_host[i];
    row_pages[i] = static_cast<int32_t>(ceil_div(seq_lens_host[i], psz));
    t_max = std::max(t_max, row_pages[i]);
  }

  int64_t n_tasks = 0, n_slots = 0, n_empty = 0;
  int32_t pps_global = 0;
  int32_t n_buckets = 0;
  std::vector<int32_t> order;

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
    pps_global = static_cast<int32_t>(std::max<int64_t>(1, ceil_div(t_max, max_splits)));
    for (int i = 0; i < b; ++i) {
      row_nsplit[i] = static_cast<int32_t>(ceil_div(row_pages[i], pps_global));
      row_task_off[i] = static_cast<int32_t>(n_tasks);
      for (int g = 0; g < hkv; ++g)
        for (int s = 0; s < row_nsplit[i]; ++s)
          push_task(i, g, s, s * pps_global, std::min((s + 1) * pps_global, row_pages[i]));
    }
    row_task_off[b] = static_cast<int32_t>(n_tasks);
    n_slots = n_tasks;
  } else if (path == PKV_BUCKETED || path == PKV_PADDED) {
    const bool padded = (path == PKV_PADDED);
    // Bucket key: the exact length, or the padded page count.
    std::vector<int64_t> key(b);
    for (int i = 0; i < b; ++i) key[i] = padded ? pow2_ceil(row_pages[i]) : seq_lens_host[i];
    order.resize(b);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return key[x] < key[y]; });
    // Buckets and their rows are appended after the task list once its
    // length is known; collect them first.
    struct Bucket { int32_t len, pages, pps, nsplit, n_rows, first; };
    std::vector<Bucket> bks;
    for (int k = 0; k < b;) {
      int e = k;
      while (e < b && key[order[e]] == key[order[k]]) ++e;
      Bucket bk;
      bk.len = padded ? -1 : seq_lens_host[order[k]];
      bk.pages = padded ? static_cast<int32_t>(key[order[k]]) : row_pages[order[k]];
      bk.pps = static_cast<int32_t>(std::max<int64_t>(1, ceil_div(bk.pages, max_splits)));
      bk.nsplit = static_cast<int32_t>(ceil_div(bk.pages, bk.pps));
      bk.n_rows = e - k;
      bk.first = k;
      bks.push_back(bk);
      for (int j = k; j < e; ++j) {
        const int row = order[j];
        // Row-local bound: the row's own pages set its split count.
        row_nsplit[row] = static_cast<int32_t>(ceil_div(row_pages[row], bk.pps));
        for (int g = 0; g < hkv; ++g)
          for (int s = 0; s < row_nsplit[row]; ++s)
            push_task(row, g, s, s * bk.pps, std::min((s + 1) * bk.pps, row_pages[row]));
        n_empty += int64_t(hkv) * (max_splits - row_nsplit[row]);
      }
      n_slots += int64_t(bk.n_rows) * hkv * max_splits;
      k = e;
    }
    n_buckets = static_cast<int32_t>(bks.size());
    // row_task_off: first task of each row in task order (rows appear in
    // bucket order, so offsets are not monotone in the row index).
    int64_t t = 0;
    for (int j = 0; j < b; ++j) {
      row_task_off[order[j]] = static_cast<int32_t>(t);
      t += int64_t(hkv) * row_nsplit[order[j]];
    }
    row_task_off[b] = static_cast<int32_t>(t);
    int32_t* bw = tasks + kTaskWords * n_tasks;
    for (int k = 0; k < n_buckets; ++k) {
      int32_t* e = bw + kBucketWords * k;
      e[0] = bks[k].len;
      e[1] = bks[k].pages;
      e[2] = bks[k].pps;
      e[3] = bks[k].nsplit;
      e[4] = bks[k].n_rows;
      e[5] = bks[k].first;
      e[6] = 0;
      e[7] = 0;
    }
    int32_t* brows = bw + kBucketWords * n_buckets;
    for (int j = 0; j < b; ++j) brows[j] = order[j];
  } else {  // PKV_NOSPLIT
    for (int i = 0; i < b; ++i) {
      row_nsplit[i] = row_pages[i] ? 1 : 0;
      row_task_off[i] = static_cast<int32_t>(n_tasks);
      if (row_pages[i])
        for (int g = 0; g < hkv; ++g) push_task(i, g, 0, 0, row_pages[i]);
    }
    row_task_off[b] = static_cast<int32_t>(n_tasks);
  }
  if (n_slots > INT32_MAX) return PKV_ERANGE;

  const int64_t off_buckets = off_tasks + kTaskWords * n_tasks;
  const int64_t off_brows = off_buckets + kBucketWords * int64_t(n_buckets);
  const int64_t total = off_brows + (n_buckets > 0 ? b : 0);

  w[kMagic] = PKV_PLAN_MAGIC;
  w[kPath] = path;
  w[kBatch] = b;
  w[kNumKvHeads] = hkv;
  w[kSplits] = max_splits;
  w[kPagesPerSplit] = pps_global;
  w[kNumTasks] = static_cast<int32_t>(n_tasks);
  w[kNumBuckets] = n_buckets;
  w[kNumStateSlots] = static_cast<int32_t>(n_slots);
  w[kNumEmptySlots] = static_cast<int32_t>(n_empty);
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
  return PKV_OK;
}
