// Merge kernel (gfx950): exact combination of a row's partial online-softmax
// states into the normalised output and its log-sum-exp.
//
// Method: PersistentKV summary pages, "Methodology / 1. Native block-table
// decode engine", "Sequence splitting" bullet: a separate merge kernel
// combines the split states exactly.  For one (row, query head) with states
// (m_s, l_s, o_s): M = max m_s, w_s = exp(m_s - M), L = sum w_s l_s,
// out = sum w_s o_s / L, lse = M + ln L.  Neutral states (m = -inf) weigh 0;
// a row with only neutral states gets out = 0 and lse = -inf.
//
// One 256-thread workgroup per (row, query head).  Thread t owns output
// chunk t % (d/4) (four floats) and split group t / (d/4); the split groups
// walk the row's states with a stride, so every state load of the row is
// issued up front.  Each thread keeps an online-rescaled partial (max, sum,
// 4 outputs); split groups are then combined through LDS.
#include "device_common.h"
#include "launch_limits.h"
#include "lens_plan.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// The scalars a merge workgroup needs before its first state load.
struct MergeHot {
  const float* st_m;
  const float* st_l;
  const float* st_o;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t splits;
  int32_t bucket_row0;
  int32_t uniform_nsplit;
  int32_t mode;
  int32_t num_rows;
};

template <int D, bool BF16>
__device__ __forceinline__ void merge_body(const MergeHot& hot, const MergeArgs& a) {
  constexpr int CH = D / 4;    // float4 chunks per output row
  constexpr int SG = 256 / CH; // split groups
  constexpr int U = 4;         // states loaded per thread per round
  const int t = threadIdx.x;
  const int ch = t % CH;
  const int sg = t / CH;
  // Item = (row index, query head), KV head fastest within a row: item j of
  // a row is query head hh = j / Hkv of KV head g = j % Hkv.  Workgroups go to
  // the 8 XCDs round-robin, so with Hq and Hkv multiples of 8 the merge of a
  // KV head runs on the XCD where a bucket launch ran all of that head's
  // splits (split_common.h), and reads their states from that XCD's L2.
  const int item = blockIdx.x;
  const int ri = item / hot.num_q_heads;
  const int j = item - ri * hot.num_q_heads;
  const int hkv = hot.num_kv_heads;
  const int G = hot.group;
  const int g = j % hkv;
  const int hh = j / hkv;
  const int h = g * G + hh;
  int row, nsplit;
  int64_t base;  // first state slot of this (row, kv head)
  __shared__ int s_red[4];
  if (hot.mode == kModeLens) {
    // Self-planned workqueue: the row's split count and first slot follow
    // from the device lengths (the split kernel derived the same tasks).
    row = ri;
    int64_t first;
    lens_row_slots<256>(a.seq_lens, hot.num_rows, hkv, hot.splits, int64_t(a.max_pages) * 16, row,
                        s_red, &nsplit, &first);
    base = first + int64_t(g) * nsplit;
  } else if (hot.mode == kModeWorkqueue && hot.uniform_nsplit > 0) {
    // Every row has the same split count, so the row's first slot follows
    // from its index and the plan's row arrays need not be read (one
    // dependent memory round trip less).
    row = ri;
    nsplit = hot.uniform_nsplit;
    base = (int64_t(row) * hkv + g) * nsplit;
  } else if (hot.mode == kModeWorkqueue) {
    row = ri;
    nsplit = a.row_nsplit[row];
    base = int64_t(a.row_task_off[row]) + int64_t(g) * nsplit;
  } else {
    row = (hot.bucket_row0 >= 0) ? hot.bucket_row0 : a.bucket_rows[ri];
    nsplit = hot.splits;
    base = (int64_t(row) * hkv + g) * hot.splits;
  }

  __shared__ float s_m[SG], s_l[SG];
  __shared__ float4 s_o[SG][CH];
  float mloc = kNegInf, lloc = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = sg; s0 < nsplit; s0 += SG * U) {
    float ms[U], ls[U];
    float4 os[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * SG;
      if (s < nsplit) {
        const int64_t e = (base + s) * G + hh;
        ms[u] = hot.st_m[e];
        ls[u] = hot.st_l[e];
        os[u] = reinterpret_cast<const float4*>(hot.st_o + e * D)[ch];
      } else {
        ms[u] = kNegInf;
        ls[u] = 0.f;
        os[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ms[u] == kNegInf) continue;  // neutral state
      const float mn = fmaxf(mloc, ms[u]);
      const float a1 = (mloc == kNegInf) ? 0.f : __expf(mloc - mn);
      const float a2 = __expf(ms[u] - mn);
      lloc = lloc * a1 + ls[u] * a2;
      acc.x = acc.x * a1 + os[u].x * a2;
      acc.y = acc.y * a1 + os[u].y * a2;
      acc.z = acc.z * a1 + os[u].z * a2;
      acc.w = acc.w * a1 + os[u].w * a2;
      mloc = mn;
    }
  }
  if (ch == 0) {
    s_m[sg] = mloc;
    s_l[sg] = lloc;
  }
  s_o[sg][ch] = acc;
  __syncthreads();
  // The split kernel has finished (stream order): reset the persistent
  // kernel's work counter for the next step on this plan.  Done after the
  // state loads, so that their addresses wait on no other argument.
  if (item == 0 && t == 0) {
    if (a.device_plan) a.device_plan[a.device_plan[kTotalWords]] = 0;
    if (a.work_counter) *a.work_counter = 0;
  }
  if (t >= CH) return;

  float mx = kNegInf;
#pragma unroll
  for (int k = 0; k < SG; ++k) mx = fmaxf(mx, s_m[k]);
  float lsum = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (mx != kNegInf) {
#pragma unroll
    for (int k = 0; k < SG; ++k) {
      const float mk = s_m[k];
      const float wk = (mk == kNegInf) ? 0.f : __expf(mk - mx);
      lsum = fmaf(wk, s_l[k], lsum);
      const float4 v = s_o[k][t];
      o.x = fmaf(wk, v.x, o.x);
      o.y = fmaf(wk, v.y, o.y);
      o.z = fmaf(wk, v.z, o.z);
      o.w = fmaf(wk, v.w, o.w);
    }
  }
  const int64_t qh = int64_t(row) * hot.num_q_heads + h;
  const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
  uint16_t* out = static_cast<uint16_t*>(a.out) + qh * D + 4 * t;
  const uint32_t lo = Elem<BF16>::from_float(o.x * inv) |
                      (uint32_t(Elem<BF16>::from_float(o.y * inv)) << 16);
  const uint32_t hi = Elem<BF16>::from_float(o.z * inv) |
                      (uint32_t(Elem<BF16>::from_float(o.w * inv)) << 16);
  *reinterpret_cast<uint2*>(out) = make_uint2(lo, hi);
  if (a.lse && t == 0) a.lse[qh] = (lsum > 0.f) ? mx + __logf(lsum) : kNegInf;
}

// The merge kernel.  The scalars the first state loads depend on (MergeHot)
// are its leading parameters, which this file's kernel-argument preloading
// puts into SGPRs at wave launch: a field read from the argument segment
// instead costs a memory round trip (about 0.6 us on MI355X, the segment being
// written for every launch), and loaded where first used the fields arrived
// in three such round trips one after the other.  The remaining fields of `a`
// (output, lse, plan arrays, counters) are needed later.  Measured on MI355X
// (same-box A/B): 0.3-1.0 us less per step than the lazily loaded arguments
// on every workload with a merge, up to 1.5 us at B = 64.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(const float* st_m, const float* st_l,
                                                    const float* st_o, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t group,
                                                    int32_t splits, int32_t bucket_row0,
                                                    int32_t uniform_nsplit, int32_t mode,
                                                    int32_t num_rows, MergeArgs a) {
  merge_body<D, BF16>(MergeHot{st_m, st_l, st_o, num_q_heads, num_kv_heads, group, splits,
                               bucket_row0, uniform_nsplit, mode, num_rows},
                      a);
}

template <int D, bool BF16>
void launch_merge_kernel(const MergeArgs& a, int64_t items, hipStream_t s) {
  hipLaunchKernelGGL((merge_kernel<D, BF16>), dim3(static_cast<uint32_t>(items)), dim3(256), 0,
                     s, a.st_m, a.st_l, a.st_o, a.num_q_heads, a.num_kv_heads, a.group, a.splits,
                     a.bucket_row0, a.uniform_nsplit, a.mode, a.num_rows, a);
}

}  // namespace

pkv_status launch_merge(const pkv_problem& p, const MergeArgs& args, hipStream_t s) {
  MergeArgs a = args;
  a.group = p.num_q_heads / p.num_kv_heads;
  const int64_t items = int64_t(a.num_rows) * p.num_q_heads;
  if (items == 0) return PKV_OK;
  if (items > kMaxGridGroups) return PKV_ERANGE;
  const bool bf = p.dtype == PKV_BF16;
  if (p.head_dim == 128) {
    if (bf) launch_merge_kernel<128, true>(a, items, s);
    else launch_merge_kernel<128, false>(a, items, s);
  } else {
    if (bf) launch_merge_kernel<64, true>(a, items, s);
    else launch_merge_kernel<64, false>(a, items, s);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

pkv_status launch_split_valu(const pkv_problem& p, int mode, const SplitArgs& a, int grid,
                             hipStream_t s);
pkv_status launch_split_mfma(const pkv_problem& p, int mode, const SplitArgs& a, int grid,
                             hipStream_t s);

// Chooses the split-kernel arithmetic.  AUTO takes the matrix-core kernel
// wherever it applies (d = 128, any G <= 16) -- on MI355X it is faster than the
// vector-ALU kernel on every measured workload -- and the vector-ALU kernel for
// d = 64 (G <= 8).  Every grid mode exists in both kernels.
pkv_status launch_split(const pkv_problem& p, int mode, int kernel, const SplitArgs& args,
                        int grid, hipStream_t s) {
  if (grid <= 0) return PKV_OK;
  SplitArgs a = args;
  a.group = p.num_q_heads / p.num_kv_heads;
  if (kernel == PKV_KERNEL_MFMA || (kernel == PKV_KERNEL_AUTO && p.head_dim == 128))
    return launch_split_mfma(p, mode, a, grid, s);
  return launch_split_valu(p, mode, a, grid, s);
}

}  // namespace pkv
