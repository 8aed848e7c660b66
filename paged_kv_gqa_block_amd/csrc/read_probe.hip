// Read-only bandwidth probe (libpkv_probe.so): streams every page chunk the
// split kernel would read for a plan's tasks, with nothing else in the loop.
// Interface and purpose in include/pkv_probe.h.
#include <cstdint>

#include <hip/hip_runtime.h>

#include "pkv.h"
#include "pkv_probe.h"

namespace {

constexpr int kWaves = 4;
constexpr int kDepth = 2;  // pages of loads a wave keeps in flight

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal (streaming) cache policy.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One workgroup per task; wave w reads the task's pages w, w + 4, ... two at a
// time.  U = 16-byte loads per lane per page chunk (4 for d = 128, 2 for 64).
template <int U>
__global__ __launch_bounds__(kWaves * 64) void probe_read_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int32_t* __restrict__ bt,
    int max_pages, int hkv, const int4* __restrict__ tasks, uint32_t* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int4 task = tasks[blockIdx.x];
  const int row = task.x, g = task.y >> 16;
  const int pb = task.z, pe = (task.w + 15) >> 4;
  const int32_t* bt_row = bt + int64_t(row) * max_pages;
  uint32_t acc = 0;
  for (int p0 = pb + wave * kDepth; p0 < pe; p0 += kWaves * kDepth) {
    uint4 buf[kDepth][2 * U];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int p = min(p0 + d, pe - 1);
      const int64_t base = (int64_t(bt_row[p]) * hkv + g) * (64 * U);
#pragma unroll
      for (int i = 0; i < U; ++i) {  // streaming (non-temporal) loads, as the split kernels
        buf[d][i] = load_stream(k + base + i * 64 + lane);
        buf[d][U + i] = load_stream(v + base + i * 64 + lane);
      }
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
#pragma unroll
      for (int i = 0; i < 2 * U; ++i) acc += buf[d][i].x ^ buf[d][i].y ^ buf[d][i].z ^ buf[d][i].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // keeps the loads; practically never true
}

// Direct-to-LDS variant: the same tasks' pages for head_dim 128, moved by
// gfx950's buffer loads that write LDS instead of registers.  Wave w of NW
// keeps a ring of R page slices (K 4 KiB + V 4 KiB each) in LDS: slot j mod R
// receives page j, and it is reloaded with page j + R once page j has been
// waited for (and, with CONSUME, read back from LDS).  No register holds page
// data in flight, so R pages per wave cost LDS, not VGPRs.  The sink gets one
// checksum per (task, wave, lane): the sum over the wave's pages of the xor of
// the four words that lane read from each 16-byte chunk of K and V (CONSUME),
// or 0.
typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N vector-memory operations of this wave are in flight
// (in-order completion: every older load has landed).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int NW, int R, bool CONSUME>
__global__ __launch_bounds__(NW * 64) void probe_lds_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const int32_t* __restrict__ bt,
    int max_pages, int hkv, const int4* __restrict__ tasks, uint32_t* sink) {
  static_assert(8 * R <= 63, "the vector-memory counter holds at most 63 loads");
  __shared__ u32x4 ring[NW][R][512];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int4 task = tasks[blockIdx.x];
  const int row = task.x, g = task.y >> 16;
  const int pb = task.z, tok_end = task.w;
  const int pe = (tok_end + 15) >> 4;
  const int32_t* bt_row = bt + int64_t(row) * max_pages;
  const int first = pb + wave;
  const int cnt = (pe > first) ? (pe - first + NW - 1) / NW : 0;  // pages of this wave
  const int64_t page_stride = int64_t(hkv) * 16 * 128;
  const uint16_t* kbase = k + int64_t(g) * 16 * 128;
  const uint16_t* vbase = v + int64_t(g) * 16 * 128;
  uint32_t acc = 0;
  for (int kc = 0; kc < cnt; kc += 64) {
    const int cnt_c = min(64, cnt - kc);
    const int idx = first + (kc + lane) * NW;
    const int pids = (lane < cnt_c && idx < max_pages) ? bt_row[idx] : 0;
    // Page j (< cnt_c) of this chunk into slot j mod R; the buffer bounds
    // stop at the page's last real token (bytes past it read as zero).
    auto issue = [&](int j) {
      const int pid = __builtin_amdgcn_readlane(pids, j);
      const int valid = min(16, tok_end - (first + (kc + j) * NW) * 16);
      const int nbytes = valid * 256;
      const auto kr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(kbase + int64_t(pid) * page_stride), (short)0, nbytes, 0x00020000);
      const auto vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(vbase + int64_t(pid) * page_stride), (short)0, nbytes, 0x00020000);
      u32x4* slot = &ring[wave][j % R][0];
#pragma unroll
      for (int i = 0; i < 4; ++i)  // aux 2: the streaming (non-temporal) policy
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(slot + i * 64), 16,
                                                 lane * 16 + i * 1024, 0, 0, 2);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(slot + 256 + i * 64), 16,
                                                 lane * 16 + i * 1024, 0, 0, 2);
    };
    const int pre = min(R, cnt_c);
    for (int j = 0; j < pre; ++j) issue(j);
    for (int j = 0; j < cnt_c; ++j) {
      // Eight loads per page: page j has landed once at most 8 * (pages
      // issued after it) loads remain.
      if (j + R - 1 < cnt_c)
        wait_vmem<8 * (R - 1)>();
      else
        wait_vmem<0>();
      if constexpr (CONSUME) {
        // The compiler does not track which LDS-bound load a read depends
        // on (it would wait for all of them), so the read is written out,
        // with its own wait, and the wait above orders it after page j.
        const uint32_t addr = static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>(&ring[wave][j % R][lane]));
        u32x4 a0, a1, a2, a3, b0, b1, b2, b3;
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %8 offset:1024\n\t"
            "ds_read_b128 %2, %8 offset:2048\n\t"
            "ds_read_b128 %3, %8 offset:3072\n\t"
            "ds_read_b128 %4, %8 offset:4096\n\t"
            "ds_read_b128 %5, %8 offset:5120\n\t"
            "ds_read_b128 %6, %8 offset:6144\n\t"
            "ds_read_b128 %7, %8 offset:7168\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1), "=&v"(b2),
              "=&v"(b3)
            : "v"(addr)
            : "memory");
        acc += (a0.x ^ a0.y ^ a0.z ^ a0.w) + (a1.x ^ a1.y ^ a1.z ^ a1.w) +
               (a2.x ^ a2.y ^ a2.z ^ a2.w) + (a3.x ^ a3.y ^ a3.z ^ a3.w) +
               (b0.x ^ b0.y ^ b0.z ^ b0.w) + (b1.x ^ b1.y ^ b1.z ^ b1.w) +
               (b2.x ^ b2.y ^ b2.z ^ b2.w) + (b3.x ^ b3.y ^ b3.z ^ b3.w);
      }
      if (j + R < cnt_c) issue(j + R);
    }
    wait_vmem<0>();
  }
  sink[(int64_t(blockIdx.x) * NW + wave) * 64 + lane] = acc;
}

// Contiguous streaming read: workgroup b reads bytes [b * chunk, (b + 1) *
// chunk) of p, 256 threads x 16 bytes per load, U loads in flight per thread.
template <int U>
__global__ __launch_bounds__(256) void probe_stream_kernel(const uint8_t* __restrict__ p,
                                                           int32_t chunk, uint32_t* sink) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p + int64_t(blockIdx.x) * chunk), (short)0, chunk, 0x00020000);
  uint32_t acc = 0;
  const int t = threadIdx.x;
  for (int off = 0; off < chunk; off += 4096 * U) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off + u * 4096 + t * 16, 0, 2);
#pragma unroll
    for (int u = 0; u < U; ++u) acc += x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // keeps the loads; practically never true
}

// One wave that sleeps until `ticks` of the device's constant-rate clock
// have passed since it started (at most kMaxSleepRounds sleeps of 127 x 64
// cycles, so it always ends), then returns.  Enqueued before a timed window,
// it keeps the device busy while the host enqueues the window's launches.
constexpr int kMaxSleepRounds = 20000;
__global__ void probe_sleep_kernel(uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < kMaxSleepRounds; ++i) {
    if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(127);
  }
}

// A kernel with (almost) no work: thread 0 of workgroup 0 copies flag[0] to
// flag[1] when flag is given.  Launched after a split kernel with the merge's
// grid it isolates the cost of a dependent launch.
__global__ void probe_empty_kernel(uint32_t* flag) {
  if (flag && blockIdx.x == 0 && threadIdx.x == 0) flag[1] = flag[0];
}

}  // namespace

extern "C" int pkv_probe_read(const void* k_pool, const void* v_pool, const int32_t* block_table,
                              int32_t max_pages_per_row, int32_t num_kv_heads, int32_t head_dim,
                              const void* plan_host, const void* plan_dev, uint32_t* sink,
                              hipStream_t stream) {
  if (!k_pool || !v_pool || !block_table || !plan_host || !plan_dev || !sink) return -1;
  if ((head_dim != 64 && head_dim != 128) || num_kv_heads < 1 || max_pages_per_row < 1) return -1;
  const int32_t* w = static_cast<const int32_t*>(plan_host);
  if (w[0] != PKV_PLAN_MAGIC || w[3] != num_kv_heads || w[14] != 16) return -1;
  const int n_tasks = w[6];
  if (n_tasks == 0) return 0;
  const int4* tasks = reinterpret_cast<const int4*>(static_cast<const int32_t*>(plan_dev) + w[10]);
  const uint4* k = static_cast<const uint4*>(k_pool);
  const uint4* v = static_cast<const uint4*>(v_pool);
  if (head_dim == 128)
    hipLaunchKernelGGL(probe_read_kernel<4>, dim3(n_tasks), dim3(kWaves * 64), 0, stream, k, v,
                       block_table, max_pages_per_row, num_kv_heads, tasks, sink);
  else
    hipLaunchKernelGGL(probe_read_kernel<2>, dim3(n_tasks), dim3(kWaves * 64), 0, stream, k, v,
                       block_table, max_pages_per_row, num_kv_heads, tasks, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

#define PKV_PROBE_LDS_CASE(NW, R, C)                                                          \
  if (waves == NW && depth == R && c == C) {                                                  \
    hipLaunchKernelGGL((probe_lds_kernel<NW, R, C>), dim3(n_tasks), dim3(NW * 64), 0, stream, \
                       static_cast<const uint16_t*>(k_pool), static_cast<const uint16_t*>(v_pool), \
                       block_table, max_pages_per_row, num_kv_heads, tasks, sink);             \
    return hipGetLastError() == hipSuccess ? 0 : -6;                                          \
  }

extern "C" int pkv_probe_read_lds(const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, int32_t max_pages_per_row,
                                  int32_t num_kv_heads, int32_t head_dim, const void* plan_host,
                                  const void* plan_dev, int32_t waves, int32_t depth,
                                  int32_t consume, uint32_t* sink, hipStream_t stream) {
  if (!k_pool || !v_pool || !block_table || !plan_host || !plan_dev || !sink) return -1;
  if (head_dim != 128 || num_kv_heads < 1 || max_pages_per_row < 1) return -1;
  const int32_t* w = static_cast<const int32_t*>(plan_host);
  if (w[0] != PKV_PLAN_MAGIC || w[3] != num_kv_heads || w[14] != 16) return -1;
  const int n_tasks = w[6];
  if (n_tasks == 0) return 0;
  const int4* tasks = reinterpret_cast<const int4*>(static_cast<const int32_t*>(plan_dev) + w[10]);
  const bool c = consume != 0;
  PKV_PROBE_LDS_CASE(4, 2, true) PKV_PROBE_LDS_CASE(4, 4, true)
  PKV_PROBE_LDS_CASE(8, 2, true) PKV_PROBE_LDS_CASE(2, 7, true)
  PKV_PROBE_LDS_CASE(4, 2, false) PKV_PROBE_LDS_CASE(4, 4, false)
  PKV_PROBE_LDS_CASE(8, 2, false) PKV_PROBE_LDS_CASE(2, 7, false)
  return -1;
}

extern "C" int pkv_probe_stream(const void* buf, int64_t bytes, int32_t grid,
                                int32_t loads_in_flight, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || grid < 1 || bytes <= 0) return -1;
  const int u = loads_in_flight;
  if (u != 4 && u != 8) return -1;
  if (bytes % (int64_t(grid) * 4096 * u) != 0 || bytes / grid > INT32_MAX) return -1;
  const int32_t chunk = static_cast<int32_t>(bytes / grid);
  const uint8_t* p = static_cast<const uint8_t*>(buf);
  if (u == 4)
    hipLaunchKernelGGL(probe_stream_kernel<4>, dim3(grid), dim3(256), 0, stream, p, chunk, sink);
  else
    hipLaunchKernelGGL(probe_stream_kernel<8>, dim3(grid), dim3(256), 0, stream, p, chunk, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int pkv_probe_empty(int32_t grid, int32_t threads, uint32_t* flag,
                               hipStream_t stream) {
  if (grid < 1 || threads < 1 || threads > 1024) return -1;
  hipLaunchKernelGGL(probe_empty_kernel, dim3(grid), dim3(threads), 0, stream, flag);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int pkv_probe_sleep(int32_t microseconds, hipStream_t stream) {
  if (microseconds < 0 || microseconds > 50000) return -1;
  static int khz = 0;  // rate of the clock s_memrealtime reads (device 0's, as every MI355X's)
  if (khz == 0) {
    int dev = 0, rate = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        rate <= 0)
      return -6;
    khz = rate;
  }
  const uint64_t ticks = uint64_t(microseconds) * uint64_t(khz) / 1000u;
  hipLaunchKernelGGL(probe_sleep_kernel, dim3(1), dim3(64), 0, stream, ticks);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
