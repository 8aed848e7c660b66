// Self-planned workqueue: the compact workqueue of the device lengths,
// derived inside the split and merge kernels instead of by a planner launch.
//
// Method: PersistentKV summary pages, "Methodology / 1. Native block-table
// decode engine", "Row-local bounds" and "Compact workqueue".  The split rule
// is the workqueue planners' (host and device): pps = max(1, ceil(T_max / S))
// pages shared by the batch, ceil(T_i / pps) splits for row i, tasks in
// (row, kv_head, split) order, so task t and its state slot t are exactly
// those of the planned workqueue.  Rows whose length lies outside
// [0, max_pages * 16] are treated as empty.
#pragma once

#include "device_common.h"
#include "pkv_internal.h"
#include "split_common.h"

namespace pkv {

__device__ __forceinline__ int lens_valid(int n, int64_t cap) { return (n < 0 || n > cap) ? 0 : n; }

// Every workgroup of the split kernel builds the row offsets of the task list
// in LDS: s_len[r] = N_r (invalid lengths as 0), s_off[r] = first task of row
// r, s_off[B] = task count.  NT threads, each owning up to kMaxLensRows / NT
// consecutive rows; s_red holds one int per wave.  Returns pps, and in
// *ns_max the split count of the longest row.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ int lens_plan_in_lds(const int32_t* __restrict__ seq_lens, int b,
                                                int hkv, int splits, int64_t cap, int* s_len,
                                                int* s_off, int* s_red, int* ns_max) {
  constexpr int kPer = kMaxLensRows / NT;
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = tid * kPer;
  int n[kPer];
  int t_max = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    n[i] = (r0 + i < b) ? lens_valid(seq_lens[r0 + i], cap) : 0;
    t_max = max(t_max, (n[i] + 15) >> 4);
  }
  t_max = wave_max_i(t_max);
  if (lane == 0) s_red[wave] = t_max;
  __syncthreads();
  t_max = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t_max = max(t_max, s_red[w]);
  const int pps = max(1, (t_max + splits - 1) / splits);
  *ns_max = (t_max + pps - 1) / pps;
  int local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) local += hkv * ((((n[i] + 15) >> 4) + pps - 1) / pps);
  const int incl = wave_scan_i(local);
  __syncthreads();  // every wave has read s_red
  if (lane == 63) s_red[wave] = incl;
  __syncthreads();
  int off = incl - local, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    off += (w < wave) ? s_red[w] : 0;
    total += s_red[w];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (r0 + i < b) {
      s_len[r0 + i] = n[i];
      s_off[r0 + i] = off;
      off += hkv * ((((n[i] + 15) >> 4) + pps - 1) / pps);
    }
  }
  if (tid == 0) s_off[b] = total;
  __syncthreads();
  return pps;
}

// Task t (< s_off[B]) of the self-planned workqueue; its state slot is t.
// t is workgroup-uniform, so every value read from LDS, and every quotient,
// is too: each is moved to a scalar register (the task then costs no vector
// registers, as a task record loaded from memory does not).
__device__ __forceinline__ Task lens_task(int t, const int* s_len, const int* s_off, int b,
                                          int hkv, int pps) {
  int lo = 0, hi = b;  // s_off[lo] <= t < s_off[hi]; rows without tasks are skipped
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(s_off[mid]) <= t) lo = mid;
    else hi = mid;
  }
  Task tk;
  tk.row = lo;
  const int n = __builtin_amdgcn_readfirstlane(s_len[lo]);
  const int off0 = __builtin_amdgcn_readfirstlane(s_off[lo]);
  const int off1 = __builtin_amdgcn_readfirstlane(s_off[lo + 1]);
  const int pages = (n + 15) >> 4;
  const int ns = __builtin_amdgcn_readfirstlane((off1 - off0) / hkv);
  const int k = t - off0;
  tk.g = __builtin_amdgcn_readfirstlane(k / ns);
  const int s = k - tk.g * ns;
  tk.page_begin = s * pps;
  const int pe = min(tk.page_begin + pps, pages);
  tk.tok_end = min(pe * 16, n);
  tk.slot = t;
  tk.empty = false;
  return tk;
}

// Self-planned persistent grid: the claim protocol of persistent_plan_loop
// over the workqueue of the device lengths, rebuilt in LDS by every
// workgroup (O(B) work, B <= kMaxLensRows); the counter is the caller's.
template <int NT, typename RunTask>
__device__ __forceinline__ void lens_loop(const SplitArgs& a, RunTask run) {
  __shared__ int s_len[kMaxLensRows];
  __shared__ int s_off[kMaxLensRows + 1];
  __shared__ int s_red[NT / 64];
  __shared__ int s_task;
  const int b = a.num_rows, hkv = a.num_kv_heads;
  int ns_max;
  const int pps = __builtin_amdgcn_readfirstlane(lens_plan_in_lds<NT>(
      a.seq_lens, b, hkv, a.splits, int64_t(a.max_pages) * 16, s_len, s_off, s_red, &ns_max));
  ns_max = __builtin_amdgcn_readfirstlane(ns_max);
  const int n_tasks = __builtin_amdgcn_readfirstlane(s_off[b]);
  const int grid = static_cast<int>(gridDim.x);
  int t = static_cast<int>(blockIdx.x);
  // When the grid covers every task (one task per workgroup) and every row
  // has the longest row's split count, with B * Hkv a multiple of 8, the
  // first task follows the XCD-affine order of launch_item (split_common.h):
  // a bijection on [0, n_tasks) that runs each (row, KV head)'s splits on
  // the XCD of its merge.
  if (t < n_tasks && n_tasks <= grid && ns_max > 0 && (b * hkv) % 8 == 0 &&
      n_tasks == b * hkv * ns_max) {
    const int k = t >> 3;
    const int q = k / ns_max;
    t = ((q << 3) + (t & 7)) * ns_max + (k - q * ns_max);
  }
  while (t < n_tasks) {
    run(lens_task(t, s_len, s_off, b, hkv, pps));
    if (n_tasks <= grid) break;
    __syncthreads();
    if (threadIdx.x == 0) s_task = grid + atomicAdd(a.work_counter, 1);
    __syncthreads();
    t = __builtin_amdgcn_readfirstlane(s_task);
  }
}

// Merge side: the split count of `row` and its first state slot
// (Hkv * sum of the earlier rows' split counts), from the device lengths.
// NT threads stride over the rows; s_red holds one int per wave.  Every
// thread gets the result.
template <int NT>
__device__ __forceinline__ void lens_row_slots(const int32_t* __restrict__ seq_lens, int b,
                                               int hkv, int splits, int64_t cap, int row,
                                               int* s_red, int* nsplit_out,
                                               int64_t* first_slot_out) {
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int t_max = 0;
  for (int r = tid; r < b; r += NT) t_max = max(t_max, (lens_valid(seq_lens[r], cap) + 15) >> 4);
  t_max = wave_max_i(t_max);
  if (lane == 0) s_red[wave] = t_max;
  __syncthreads();
  t_max = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t_max = max(t_max, s_red[w]);
  const int pps = max(1, (t_max + splits - 1) / splits);
  int before = 0;
  for (int r = tid; r < row; r += NT)
    before += (((lens_valid(seq_lens[r], cap) + 15) >> 4) + pps - 1) / pps;
  before = wave_sum_i(before);
  __syncthreads();  // every wave has read s_red
  if (lane == 0) s_red[wave] = before;
  __syncthreads();
  int64_t sum = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += s_red[w];
  *nsplit_out = (((lens_valid(seq_lens[row], cap) + 15) >> 4) + pps - 1) / pps;
  *first_slot_out = sum * hkv;
}

}  // namespace pkv
