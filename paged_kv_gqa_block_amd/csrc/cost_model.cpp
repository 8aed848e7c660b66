// Learned cost model for the path choice: plan features of a candidate
// (path, split cap) in natural units and a per-path linear model of the step
// time, fitted to measured step times.  The PersistentKV summary pages leave
// such a model as future work ("Significado y Reivindicaciones" / "Direcciones
// Futuras", es page; "2. Calibrated adaptive policy" uses hand-calibrated
// thresholds instead).  Host code only; it allocates nothing (bucket orders
// use the caller's scratch, per-CU sums the stack).
#include <algorithm>
#include <cstdint>
#include <cmath>

#include "pkv_internal.h"

using namespace pkv;

namespace {

constexpr int kMaxCus = 1024;
// Tasks per CU of the balanced workqueue candidates of pkv_policy_default.
constexpr int32_t kNumBalanced = 2;
constexpr int32_t kBalancedPerCu[kNumBalanced] = {1, 2};

// Per-CU load of one launch: grid item j goes to CU j mod num_cus (the
// round-robin spread of a launch's workgroups); max() is the largest sum of
// pages over the CUs.  The items of one (row, KV head) are a run of
// consecutive grid items, all of `pps` pages except the last (`last` pages),
// possibly followed by empty bucket slots.  A run is added in O(1): whole
// turns around the CUs go to a common offset, the rest to a difference array
// over the CUs, and the last item's shortfall to a point correction; max()
// then costs O(num_cus).  The sums are exactly those of adding the items one
// by one.
struct CuLoad {
  int64_t diff[kMaxCus + 1];
  int64_t point[kMaxCus];
  int64_t base;  // pages added to every CU
  int32_t cus;
  int32_t k;     // CU of the next grid item
  int64_t j;     // grid items so far
  void start(int32_t n) {
    cus = n;
    k = 0;
    j = 0;
    base = 0;
    std::fill(diff, diff + n + 1, 0);
    std::fill(point, point + n, 0);
  }
  // `n` items of `pps` pages at CUs k, k+1, ... (mod cus), the last one of
  // `last` pages (n >= 1, last <= pps), then `advance` - n empty items.
  void add_run(int64_t n, int64_t pps, int64_t last, int64_t advance) {
    base += (n / cus) * pps;
    const int64_t r = n % cus;
    if (r > 0) {
      const int64_t end = k + r;
      diff[k] += pps;
      if (end <= cus) {
        diff[end] -= pps;
      } else {
        diff[cus] -= pps;
        diff[0] += pps;
        diff[end - cus] -= pps;
      }
    }
    point[(k + n - 1) % cus] -= pps - last;
    k = static_cast<int32_t>((k + advance) % cus);
    j += advance;
  }
  // One item of `pages` pages.
  void add(int64_t pages) { add_run(1, pages, pages, 1); }
  int64_t max() const {
    int64_t run = 0, best = INT64_MIN;
    for (int32_t c = 0; c < cus; ++c) {
      run += diff[c];
      best = std::max(best, base + run + point[c]);
    }
    return best;
  }
};

pkv_status features(const pkv_problem* prob, const int32_t* lens, int32_t path, int32_t splits,
                    int32_t num_cus, int32_t* scratch, float* f) {
  const int32_t b = prob->batch, hkv = prob->num_kv_heads, psz = prob->page_size;
  const int64_t cap = int64_t(prob->max_pages_per_row) * psz;
  for (int32_t i = 0; i < b; ++i)
    if (lens[i] < 0 || lens[i] > cap) return PKV_ERANGE;
  const bool bucketed = (path == PKV_BUCKETED || path == PKV_PADDED);
  if (bucketed) {
    if (!scratch) return PKV_EINVAL;
    order_rows(lens, b, path == PKV_PADDED, psz, scratch);
  }
  const PlanCounts c = count_plan(*prob, lens, path, splits, bucketed ? scratch : nullptr);

  // Grid items in launch order with their pages (0 for an empty slot).
  CuLoad load;  // 16 KiB on the stack
  int64_t crit = 0, items = 0;
  load.start(num_cus);
  if (path == PKV_WORKQUEUE) {
    for (int32_t i = 0; i < b; ++i) {
      const int64_t t = ceil_div(lens[i], psz);
      const int64_t ns = ceil_div(t, c.pps);
      if (ns == 0) continue;
      const int64_t last = t - (ns - 1) * c.pps;
      for (int32_t g = 0; g < hkv; ++g) load.add_run(ns, c.pps, last, ns);
    }
    items = load.j;
    crit = load.max();
  } else if (path == PKV_NOSPLIT) {
    for (int32_t i = 0; i < b; ++i)
      for (int32_t g = 0; g < hkv; ++g) load.add(ceil_div(lens[i], psz));
    items = load.j;
    crit = load.max();
  } else {
    for_each_bucket(lens, b, path == PKV_PADDED, psz, splits, scratch,
                    [&](int32_t first, int32_t end, int32_t, int32_t, int32_t pps, int32_t,
                        int32_t) {
                      load.start(num_cus);
                      for (int32_t r = first; r < end; ++r) {
                        const int64_t t = ceil_div(lens[scratch[r]], psz);
                        const int64_t ns = std::min<int64_t>(ceil_div(t, pps), splits);
                        for (int32_t g = 0; g < hkv; ++g) {
                          if (ns == 0) {  // every slot of the row is empty
                            load.add_run(1, 0, 0, splits);
                          } else {
                            load.add_run(ns, pps, std::min<int64_t>(pps, t - (ns - 1) * pps),
                                         splits);
                          }
                        }
                      }
                      items += load.j;
                      crit += load.max();
                    });
  }
  int64_t tokens = 0;
  for (int32_t i = 0; i < b; ++i) tokens += lens[i];
  const int64_t g = prob->num_q_heads / hkv;
  f[0] = 1.f;
  f[1] = float(c.n_launches);
  f[2] = float(double(tokens) * hkv * prob->head_dim * 2 * 2 / 1e6);
  f[3] = float(2.0 * double(c.n_slots) * g * (prob->head_dim + 2) * 4 / 1e6);
  f[4] = float(crit);
  f[5] = float(double(items) / 1e3);
  f[6] = float(double(c.n_tasks) / 1e3);
  f[7] = float(double(c.max_task_pages) / 1e2);
  return PKV_OK;
}

bool valid_cus(int32_t n) { return n >= 1 && n <= kMaxCus; }

// Largest split cap S in [1, max_splits] whose compact workqueue holds at
// most per_cu * num_cus tasks, or 0 when even S = 1 holds more.  The task
// count of S (count_plan: Hkv * sum_i ceil(T_i / ceil(T_max / S))) never
// decreases as S grows, so the cap is found by bisection.  Lengths must be
// valid.
int32_t balanced_splits(const pkv_problem& p, const int32_t* lens, int32_t num_cus,
                        int32_t per_cu, int32_t max_splits) {
  const int64_t budget = int64_t(per_cu) * num_cus;
  auto tasks = [&](int32_t s) { return count_plan(p, lens, PKV_WORKQUEUE, s, nullptr).n_tasks; };
  if (tasks(1) > budget) return 0;
  int32_t lo = 1, hi = max_splits;  // tasks(lo) <= budget
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo + 1) / 2;
    if (tasks(mid) <= budget) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The model's step time of candidate (path, s) in microseconds.
pkv_status predict(const pkv_problem* prob, const pkv_cost_model* model, const int32_t* lens,
                   int32_t path, int32_t s, int32_t* scratch, double* y) {
  float f[PKV_COST_FEATURES];
  const pkv_status st = features(prob, lens, path, path == PKV_NOSPLIT ? 1 : s, model->num_cus,
                                 scratch, f);
  if (st != PKV_OK) return st;
  const float* w = model->weights + PKV_COST_FEATURES * path;
  *y = 0.0;
  for (int j = 0; j < PKV_COST_FEATURES; ++j) *y += double(w[j]) * f[j];
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_balanced_splits(const pkv_problem* prob, const int32_t* seq_lens_host,
                                          int32_t num_cus, int32_t per_cu, int32_t max_splits,
                                          int32_t* splits_out) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!seq_lens_host || !splits_out) return PKV_EINVAL;
  if (!valid_cus(num_cus) || per_cu < 1 || per_cu > 64 || max_splits < 1 || max_splits > 65535)
    return PKV_EINVAL;
  const int64_t cap = int64_t(prob->max_pages_per_row) * prob->page_size;
  for (int32_t i = 0; i < prob->batch; ++i)
    if (seq_lens_host[i] < 0 || seq_lens_host[i] > cap) return PKV_ERANGE;
  *splits_out = balanced_splits(*prob, seq_lens_host, num_cus, per_cu, max_splits);
  return PKV_OK;
}

extern "C" pkv_status pkv_cost_features(const pkv_problem* prob, const int32_t* seq_lens_host,
                                        int32_t path, int32_t max_splits, int32_t num_cus,
                                        int32_t* scratch_host, float* features_out) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!seq_lens_host || !features_out) return PKV_EINVAL;
  if (path < PKV_BUCKETED || path > PKV_PADDED) return PKV_EINVAL;
  if (max_splits < 1 || max_splits > 65535 || !valid_cus(num_cus)) return PKV_EINVAL;
  return features(prob, seq_lens_host, path, path == PKV_NOSPLIT ? 1 : max_splits, num_cus,
                  scratch_host, features_out);
}

extern "C" pkv_status pkv_policy_model(const pkv_problem* prob, const pkv_cost_model* model,
                                       const int32_t* seq_lens_host, int32_t* scratch_host,
                                       int32_t* path_out, int32_t* splits_out,
                                       float* predicted_us_out) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!model || !seq_lens_host || !path_out || !splits_out) return PKV_EINVAL;
  if (model->n_candidates < 1 || !model->candidates || !model->weights ||
      !valid_cus(model->num_cus))
    return PKV_EINVAL;
  for (int32_t k = 0; k < model->n_candidates; ++k) {
    const int32_t path = model->candidates[2 * k], s = model->candidates[2 * k + 1];
    if (path < PKV_BUCKETED || path > PKV_PADDED || s < 1 || s > 65535) return PKV_EINVAL;
  }
  double best = INFINITY;
  int32_t best_path = 0, best_s = 0;
  for (int32_t k = 0; k < model->n_candidates; ++k) {
    const int32_t path = model->candidates[2 * k], s = model->candidates[2 * k + 1];
    double y = 0.0;
    st = predict(prob, model, seq_lens_host, path, s, scratch_host, &y);
    if (st != PKV_OK) return st;
    if (y < best) {  // the first candidate wins a tie
      best = y;
      best_path = path;
      best_s = s;
    }
  }
  *path_out = best_path;
  *splits_out = best_s;
  if (predicted_us_out) *predicted_us_out = float(best);
  return PKV_OK;
}

extern "C" pkv_status pkv_policy_default(const pkv_policy_table* table,
                                         const pkv_cost_model* model, const pkv_problem* prob,
                                         const int32_t* seq_lens_host, int32_t* scratch_host,
                                         int32_t* path_out, int32_t* splits_out) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!table || !model || !seq_lens_host || !path_out || !splits_out) return PKV_EINVAL;
  const int64_t cap = int64_t(prob->max_pages_per_row) * prob->page_size;
  int32_t n_max = 0;
  for (int32_t i = 0; i < prob->batch; ++i) {
    if (seq_lens_host[i] < 0 || seq_lens_host[i] > cap) return PKV_ERANGE;
    n_max = std::max(n_max, seq_lens_host[i]);
  }
  // One row: its length is N_max, so the (B, N_max) table sees the whole
  // workload.  Several rows: the length mix decides the load balance, which
  // the model's per-CU feature sees and the table's key does not.
  if (prob->batch == 1) return pkv_policy(table, 1, n_max, path_out, splits_out);
  // The model's candidates, then the CU-balanced workqueue caps
  // (kBalancedPerCu tasks per CU, at most the model's largest workqueue cap)
  // that are not among them; the first of equal predictions wins.
  if (model->n_candidates < 1 || !model->candidates || !model->weights ||
      !valid_cus(model->num_cus))
    return PKV_EINVAL;
  int32_t s_max = 0;
  for (int32_t k = 0; k < model->n_candidates; ++k) {
    const int32_t path = model->candidates[2 * k], s = model->candidates[2 * k + 1];
    if (path < PKV_BUCKETED || path > PKV_PADDED || s < 1 || s > 65535) return PKV_EINVAL;
    if (path == PKV_WORKQUEUE) s_max = std::max(s_max, s);
  }
  double best = INFINITY;
  int32_t best_path = 0, best_s = 0;
  for (int32_t k = 0; k < model->n_candidates; ++k) {
    const int32_t path = model->candidates[2 * k], s = model->candidates[2 * k + 1];
    double y = 0.0;
    st = predict(prob, model, seq_lens_host, path, s, scratch_host, &y);
    if (st != PKV_OK) return st;
    if (y < best) {
      best = y;
      best_path = path;
      best_s = s;
    }
  }
  int32_t bal[kNumBalanced];
  for (int32_t i = 0; i < kNumBalanced; ++i)
    bal[i] = s_max > 0 ? balanced_splits(*prob, seq_lens_host, model->num_cus,
                                         kBalancedPerCu[i], s_max)
                       : 0;
  for (int32_t i = 0; i < kNumBalanced; ++i) {
    const int32_t s = bal[i];
    bool listed = (s == 0);  // 0: no cap keeps the tasks within the budget
    for (int32_t k = 0; k < model->n_candidates; ++k)
      listed |= model->candidates[2 * k] == PKV_WORKQUEUE && model->candidates[2 * k + 1] == s;
    for (int32_t j = 0; j < i; ++j) listed |= bal[j] == s;
    if (listed) continue;
    double y = 0.0;
    st = predict(prob, model, seq_lens_host, PKV_WORKQUEUE, s, scratch_host, &y);
    if (st != PKV_OK) return st;
    if (y < best) {
      best = y;
      best_path = PKV_WORKQUEUE;
      best_s = s;
    }
  }
  *path_out = best_path;
  *splits_out = best_s;
  return PKV_OK;
}
