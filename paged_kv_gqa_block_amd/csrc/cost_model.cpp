// Learned cost model for the path choice: plan features of a candidate
// (path, split cap) and a per-path linear model of log2 of the step time,
// fitted by least squares to measured step times.  The PersistentKV summary
// pages leave such a model as future work ("Conclusion"; "2. Calibrated
// adaptive policy" uses hand-calibrated thresholds instead).  Host code only;
// it allocates nothing (bucket orders use the caller's scratch).
#include <algorithm>
#include <cmath>

#include "pkv_internal.h"

using namespace pkv;

namespace {

double log2_at_least_1(double x) { return std::log2(std::max(1.0, x)); }

pkv_status features(const pkv_problem* prob, const int32_t* lens, int32_t path, int32_t splits,
                    int32_t* scratch, float* f) {
  const int32_t b = prob->batch, hkv = prob->num_kv_heads;
  const int64_t cap = int64_t(prob->max_pages_per_row) * prob->page_size;
  int64_t sum = 0;
  int32_t n_max = 0;
  for (int32_t i = 0; i < b; ++i) {
    if (lens[i] < 0 || lens[i] > cap) return PKV_ERANGE;
    sum += lens[i];
    n_max = std::max(n_max, lens[i]);
  }
  const bool bucketed = (path == PKV_BUCKETED || path == PKV_PADDED);
  if (bucketed) {
    if (!scratch) return PKV_EINVAL;
    order_rows(lens, b, path == PKV_PADDED, prob->page_size, scratch);
  }
  const PlanCounts c = count_plan(*prob, lens, path, splits, bucketed ? scratch : nullptr);
  const int64_t g = prob->num_q_heads / hkv;
  const double items = path == PKV_WORKQUEUE ? double(c.n_tasks)
                       : path == PKV_NOSPLIT ? double(b) * hkv
                                             : double(c.n_slots);
  const double state_bytes = 2.0 * double(c.n_slots) * g * (prob->head_dim + 2) * 4;
  const double kv_bytes = double(sum) * hkv * prob->head_dim * 2 * 2;
  f[0] = 1.f;
  f[1] = float(log2_at_least_1(b));
  f[2] = float(log2_at_least_1(n_max));
  f[3] = float(log2_at_least_1(double(sum) / b));
  f[4] = float(log2_at_least_1(path == PKV_NOSPLIT ? 1 : splits));
  f[5] = float(log2_at_least_1(double(c.n_tasks)));
  f[6] = float(c.n_launches);
  f[7] = float(log2_at_least_1(items));
  f[8] = float(std::log2(1.0 + state_bytes));
  f[9] = float(log2_at_least_1(kv_bytes));
  f[10] = float(log2_at_least_1(c.max_task_pages));
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_cost_features(const pkv_problem* prob, const int32_t* seq_lens_host,
                                        int32_t path, int32_t max_splits, int32_t* scratch_host,
                                        float* features_out) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!seq_lens_host || !features_out) return PKV_EINVAL;
  if (path < PKV_BUCKETED || path > PKV_PADDED) return PKV_EINVAL;
  if (max_splits < 1 || max_splits > 65535) return PKV_EINVAL;
  return features(prob, seq_lens_host, path, max_splits, scratch_host, features_out);
}

extern "C" pkv_status pkv_policy_model(const pkv_problem* prob, const pkv_cost_model* model,
                                       const int32_t* seq_lens_host, int32_t* scratch_host,
                                       int32_t* path_out, int32_t* splits_out,
                                       float* predicted_us_out) {
  pkv_status st = check_problem(prob);
  if (st != PKV_OK) return st;
  if (!model || !seq_lens_host || !path_out || !splits_out) return PKV_EINVAL;
  if (model->n_candidates < 1 || !model->candidates || !model->weights) return PKV_EINVAL;
  for (int32_t k = 0; k < model->n_candidates; ++k) {
    const int32_t path = model->candidates[2 * k], s = model->candidates[2 * k + 1];
    if (path < PKV_BUCKETED || path > PKV_PADDED || s < 1 || s > 65535) return PKV_EINVAL;
  }
  double best = INFINITY;
  int32_t best_k = -1;
  float f[PKV_COST_FEATURES];
  for (int32_t k = 0; k < model->n_candidates; ++k) {
    const int32_t path = model->candidates[2 * k], s = model->candidates[2 * k + 1];
    st = features(prob, seq_lens_host, path, s, scratch_host, f);
    if (st != PKV_OK) return st;
    const float* w = model->weights + PKV_COST_FEATURES * path;
    double y = 0.0;
    for (int j = 0; j < PKV_COST_FEATURES; ++j) y += double(w[j]) * f[j];
    if (y < best) {  // first candidate wins ties
      best = y;
      best_k = k;
    }
  }
  *path_out = model->candidates[2 * best_k];
  *splits_out = model->candidates[2 * best_k + 1];
  if (predicted_us_out) *predicted_us_out = float(std::exp2(best));
  return PKV_OK;
}
