// KV append kernel (gfx950): store the step's new key and value of every row
// in the paged pools, through the block table, before attention runs.
//
// Token position p of row i lives in pool page block_table[i][p / P] at slot
// p % P -- the addressing the split kernels read (PersistentKV summary pages,
// "Methodology / 1. Native block-table decode engine", Layout: pages are used
// in place through the block table).  The pages do not describe the append;
// it is the input-side step that lets a decode loop run end to end.
//
// One 64-lane workgroup per (row, KV head): lanes 0..d/8-1 copy the key and
// lanes 32..32+d/8-1 the value, 16 bytes each.  Rows with a negative position
// are inactive; positions at or past the block table's capacity are skipped.
#include "device_common.h"
#include "launch_limits.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int item = blockIdx.x;
  const int row = item / a.num_kv_heads;
  const int g = item - row * a.num_kv_heads;
  const int p = a.positions[row];
  if (p < 0 || p >= a.max_pages * 16) return;
  const int lane = threadIdx.x;
  const int c = lane & 31;
  if (c >= a.head_dim / 8) return;
  const bool is_v = lane >= 32;
  const int page = a.block_table[int64_t(row) * a.max_pages + (p >> 4)];
  const int64_t src = (int64_t(row) * a.num_kv_heads + g) * a.head_dim + 8 * c;
  const int64_t dst = ((int64_t(page) * a.num_kv_heads + g) * 16 + (p & 15)) * a.head_dim + 8 * c;
  const uint16_t* s = static_cast<const uint16_t*>(is_v ? a.v_new : a.k_new) + src;
  uint16_t* d = static_cast<uint16_t*>(is_v ? a.v_pool : a.k_pool) + dst;
  *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
}

}  // namespace

pkv_status launch_append(const AppendArgs& a, int batch, hipStream_t s) {
  const int64_t grid = int64_t(batch) * a.num_kv_heads;
  if (grid <= 0) return PKV_OK;
  if (grid > kMaxGridGroups) return PKV_ERANGE;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<uint32_t>(grid)), dim3(64), 0, s, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // namespace pkv
