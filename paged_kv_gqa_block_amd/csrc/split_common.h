// Pieces shared by the two split / no-split kernels (vector-ALU and
// matrix-core): task decoding for the three grid modes, the empty-task
// outputs, and the final combine of the waves' partial states.
#pragma once

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

// One workgroup's work: row, KV head, first page and one-past-last real token
// of the page range, and the partial-state slot (split modes).
struct Task {
  int row;
  int g;
  int page_begin;
  int tok_end;  // min(page_end * 16, N_row); page_end = ceil(tok_end / 16)
  int64_t slot;
  bool empty;   // bucket slot past the bucket's split count
};

template <int MODE>
__device__ __forceinline__ Task decode_task(const SplitArgs& a, int item) {
  Task t;
  const int hkv = a.num_kv_heads;
  t.empty = false;
  t.slot = 0;
  if constexpr (MODE == kModeWorkqueue) {
    const int4 w = reinterpret_cast<const int4*>(a.tasks)[item];
    t.row = w.x;
    t.g = w.y >> 16;
    t.page_begin = w.z;
    t.tok_end = w.w;
    t.slot = item;
  } else if constexpr (MODE == kModeBucket) {
    // Three-dimensional grid (KV head, split slot, row of the bucket): the
    // task comes from the block index without the integer divisions (a few
    // dozen scalar instructions each) that a 1-D index would need.
    (void)item;
    t.g = blockIdx.x;
    const int s = blockIdx.y;
    t.row = (a.bucket_row0 >= 0) ? a.bucket_row0 : a.bucket_rows[blockIdx.z];
    t.slot = (int64_t(t.row) * hkv + t.g) * a.splits + s;
    // Exact bucket: the rows share length, pages and split count.  Padded
    // bucket: the row's own length bounds its splits (row-local bounds).
    int n = a.bucket_len, pages = a.bucket_pages, nsplit = a.bucket_nsplit;
    if (n < 0) {
      n = a.row_len[t.row];
      pages = (n + 15) >> 4;
      nsplit = (pages + a.bucket_pps - 1) / a.bucket_pps;
    }
    t.empty = s >= nsplit;
    t.page_begin = s * a.bucket_pps;
    const int pe = min(t.page_begin + a.bucket_pps, pages);
    t.tok_end = min(pe * 16, n);
  } else {
    t.row = item / hkv;
    t.g = item - t.row * hkv;
    t.page_begin = 0;
    t.tok_end = -1;  // filled in from seq_lens by the caller
  }
  return t;
}

// Task index of this workgroup in a one-workgroup-per-item launch.  A
// workqueue launch whose rows all have ns splits, with B * Hkv a multiple of 8
// (a.xcd_nsplit = ns, checked on the host), deals whole (row, KV head) pairs
// to the 8 XCDs: block j (XCD j mod 8) runs task p * ns + (j / 8) mod ns of
// pair p = 8 * ((j / 8) / ns) + j mod 8.  This is a bijection on the tasks,
// and every split of pair p runs on XCD p mod 8, where the merge of that KV
// head runs (merge.hip).  Other launches run task j.
template <int MODE>
__device__ __forceinline__ int launch_item(const SplitArgs& a) {
  const int j = static_cast<int>(blockIdx.x);
  if constexpr (MODE == kModeWorkqueue) {
    const int ns = a.xcd_nsplit;
    if (ns > 0) {
      const int k = j >> 3;
      const int q = k / ns;
      return ((q << 3) + (j & 7)) * ns + (k - q * ns);
    }
  }
  return j;
}

// Grid of one bucket launch: (KV head, split slot, row of the bucket), KV
// head fastest.  Workgroups are dealt to the 8 XCDs round-robin in launch
// order, so with Hkv a multiple of 8 every split of one KV head runs on one
// XCD; the merge puts that head's query heads on the same XCD (merge.hip),
// where its L2 still holds the states.  The host keeps the row count within
// kMaxBucketRows.
inline dim3 bucket_grid(const SplitArgs& a, int items) {
  const int per_row = a.splits * a.num_kv_heads;
  return dim3(static_cast<uint32_t>(a.num_kv_heads), static_cast<uint32_t>(a.splits),
              static_cast<uint32_t>(items / per_row));
}

// Persistent grid over a device-built workqueue plan: workgroup w first runs
// task w; further tasks (grid + k for the k-th claim) come from a
// device-scope counter, zeroed by the device planner and reset by the device
// merge, so they go to whichever workgroups are running.  A workgroup exits
// once its task index passes the task count (or at once after its first task
// when the grid covers every task), and none ever waits on another.
// run(Task) processes one task and may reuse LDS: the barrier before each
// claim orders it against the next task.
template <typename RunTask>
__device__ __forceinline__ void persistent_plan_loop(const SplitArgs& a, RunTask run) {
  __shared__ int s_task;
  const int n_tasks = a.device_plan[kNumTasks];
  const int grid = static_cast<int>(gridDim.x);
  int32_t* counter = a.device_plan + a.device_plan[kTotalWords];
  int t = static_cast<int>(blockIdx.x);
  while (t < n_tasks) {
    run(decode_task<kModeWorkqueue>(a, t));
    if (n_tasks <= grid) break;
    __syncthreads();  // LDS (and s_task) are reused by the next task
    if (threadIdx.x == 0) s_task = grid + atomicAdd(counter, 1);
    __syncthreads();
    t = s_task;
  }
}

// Neutral state (-inf, 0, 0) of an empty bucket slot.
template <int NW>
__device__ __forceinline__ void write_neutral(const SplitArgs& a, const Task& t, int G, int D) {
  for (int e = threadIdx.x; e < G * D; e += NW * 64) a.st_o[t.slot * G * D + e] = 0.f;
  if (threadIdx.x < G) {
    a.st_m[t.slot * G + threadIdx.x] = kNegInf;
    a.st_l[t.slot * G + threadIdx.x] = 0.f;
  }
}

// Output of an empty row on the no-split path: out = 0, lse = -inf.
template <int NW>
__device__ __forceinline__ void write_empty_row(const SplitArgs& a, const Task& t, int G, int D) {
  uint16_t* out =
      static_cast<uint16_t*>(a.out) + (int64_t(t.row) * a.num_q_heads + t.g * G) * D;
  for (int e = threadIdx.x; e < G * D; e += NW * 64) out[e] = 0;
  if (a.lse && threadIdx.x < G)
    a.lse[int64_t(t.row) * a.num_q_heads + t.g * G + threadIdx.x] = kNegInf;
}

// Combine the NW waves' states (max in log2 units, sum, unnormalised output,
// already in LDS) and write either the task's partial state or, on the
// no-split path, the normalised output and lse.  Must follow a barrier.
// Each thread combines four consecutive output elements of one head (one
// 16-byte LDS read per wave, one 16-byte state store); per element the
// arithmetic and its order are those of a one-element loop.  sm_o must be
// 16-byte aligned.
template <int D, int GP, int NW, bool BF16, int MODE>
__device__ __forceinline__ void combine_waves_and_store(const SplitArgs& a, const Task& t, int G,
                                                        const float (&sm_m)[NW][GP],
                                                        const float (&sm_l)[NW][GP],
                                                        const float (&sm_o)[NW][GP][D]) {
  constexpr int C4 = D / 4;  // 16-byte chunks per head
  for (int e = threadIdx.x; e < G * C4; e += NW * 64) {
    const int h = e / C4;
    const int c4 = e - h * C4;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm_m[w][h]);
    float lsum = 0.f;
    float4 osum = make_float4(0.f, 0.f, 0.f, 0.f);
    if (mx != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm_m[w][h];
        const float wt = (mw == kNegInf) ? 0.f : fast_exp2(mw - mx);
        lsum = fmaf(wt, sm_l[w][h], lsum);
        const float4 o = reinterpret_cast<const float4*>(sm_o[w][h])[c4];
        osum.x = fmaf(wt, o.x, osum.x);
        osum.y = fmaf(wt, o.y, osum.y);
        osum.z = fmaf(wt, o.z, osum.z);
        osum.w = fmaf(wt, o.w, osum.w);
      }
    }
    if constexpr (MODE == kModeNoSplit) {
      const int64_t qh = int64_t(t.row) * a.num_q_heads + t.g * G + h;
      const bool pos = lsum > 0.f;
      const uint32_t lo = uint32_t(Elem<BF16>::from_float(pos ? osum.x / lsum : 0.f)) |
                          (uint32_t(Elem<BF16>::from_float(pos ? osum.y / lsum : 0.f)) << 16);
      const uint32_t hi = uint32_t(Elem<BF16>::from_float(pos ? osum.z / lsum : 0.f)) |
                          (uint32_t(Elem<BF16>::from_float(pos ? osum.w / lsum : 0.f)) << 16);
      reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + qh * D)[c4] = make_uint2(lo, hi);
      if (c4 == 0 && a.lse) a.lse[qh] = pos ? mx * kLn2 + __logf(lsum) : kNegInf;
    } else {
      reinterpret_cast<float4*>(a.st_o + (t.slot * G + h) * D)[c4] = osum;
      if (c4 == 0) {
        a.st_m[t.slot * G + h] = (mx == kNegInf) ? kNegInf : mx * kLn2;
        a.st_l[t.slot * G + h] = lsum;
      }
    }
  }
}

// Block-table entries of 64 of a wave's pages: lane j holds the pool page of
// the wave's page k0 + j (its pages are first, first + NW, ...).  Entries past
// the task's pages are read only while inside the table row, and never used.
template <int NW>
__device__ __forceinline__ int load_page_ids(const int32_t* bt_row, int max_pages, int first,
                                             int k0, int lane) {
  const int idx = first + (k0 + lane) * NW;
  return (idx < max_pages) ? bt_row[idx] : 0;
}

}  // namespace pkv
