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
// One wave per (row, query head); 4 waves per workgroup.  Lane s first owns
// split s (weights and the sum L via wave reductions), then lanes own output
// elements and accumulate the weighted o_s, loading the per-split weight
// through a wave broadcast.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) x = fmaxf(x, shfl_xor(x, sh));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) x += shfl_xor(x, sh);
  return x;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int EPL = D / 64;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);  // (row index, q head)
  if (item >= a.num_rows * a.num_q_heads) return;
  const int ri = item / a.num_q_heads;
  const int h = item - ri * a.num_q_heads;
  const int hkv = a.num_kv_heads;
  const int G = a.num_q_heads / hkv;
  const int g = h / G;
  const int hh = h - g * G;
  int row, nsplit;
  int64_t base;  // first state slot of this (row, kv head)
  if (a.mode == kModeWorkqueue) {
    row = ri;
    nsplit = a.row_nsplit[row];
    base = int64_t(a.row_task_off[row]) + int64_t(g) * nsplit;
  } else {
    row = a.bucket_rows[ri];
    nsplit = a.splits;
    base = (int64_t(row) * hkv + g) * a.splits;
  }

  // Pass 1: global max over the splits.
  float mx = kNegInf;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int s = s0 + lane;
    if (s < nsplit) mx = fmaxf(mx, a.st_m[(base + s) * G + hh]);
  }
  mx = wave_max(mx);

  float acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
  float lsum = 0.f;
  if (mx != kNegInf) {
    for (int s0 = 0; s0 < nsplit; s0 += 64) {
      const int s = s0 + lane;
      float w = 0.f;
      if (s < nsplit) {
        const float ms = a.st_m[(base + s) * G + hh];
        w = (ms == kNegInf) ? 0.f : __expf(ms - mx);
        lsum = fmaf(w, a.st_l[(base + s) * G + hh], lsum);
      }
      const int cnt = min(64, nsplit - s0);
      for (int k = 0; k < cnt; ++k) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
        if (wk == 0.f) continue;  // wave-uniform skip of neutral / negligible states
        const float* op = a.st_o + ((base + s0 + k) * G + hh) * D + lane * EPL;
#pragma unroll
        for (int j = 0; j < EPL; ++j) acc[j] = fmaf(wk, op[j], acc[j]);
      }
    }
    lsum = wave_sum(lsum);
  }
  const int64_t qh = int64_t(row) * a.num_q_heads + h;
  uint16_t* out = static_cast<uint16_t*>(a.out) + qh * D + lane * EPL;
  const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) out[j] = Elem<BF16>::from_float(acc[j] * inv);
  if (a.lse && lane == 0) a.lse[qh] = (lsum > 0.f) ? mx + __logf(lsum) : kNegInf;
}

}  // namespace

pkv_status launch_merge(const pkv_problem& p, const MergeArgs& a, hipStream_t s) {
  const int items = a.num_rows * p.num_q_heads;
  if (items == 0) return PKV_OK;
  const dim3 grid((items + 3) / 4), block(256);
  const bool bf = p.dtype == PKV_BF16;
  if (p.head_dim == 128) {
    if (bf) hipLaunchKernelGGL((merge_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (bf) hipLaunchKernelGGL((merge_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

// Chooses the split-kernel arithmetic.  AUTO currently means the vector-ALU
// kernel; the matrix-core kernel is selected explicitly.
pkv_status launch_split_valu(const pkv_problem& p, int mode, const SplitArgs& a, int grid,
                             hipStream_t s);

pkv_status launch_split(const pkv_problem& p, int mode, int kernel, const SplitArgs& a, int grid,
                        hipStream_t s) {
  if (grid <= 0) return PKV_OK;
  if (kernel == PKV_KERNEL_MFMA) return PKV_ESHAPE;
  return launch_split_valu(p, mode, a, grid, s);
}

}  // namespace pkv
