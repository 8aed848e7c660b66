/*
 * pkv_probe.h -- read-only bandwidth probe for the paged KV pools
 * (libpkv_probe.so).  Measurement tool, not part of the decode path.
 *
 * pkv_probe_read streams, for every task of a plan made by pkv_plan, the
 * K and V pool chunks that the split kernel reads for that task: for task
 * (row, kv_head, page_begin, token_end) the pages
 * block_table[row][page_begin .. ceil(token_end / P)) of head kv_head, whole
 * pages of P * head_dim elements, with no arithmetic beyond folding the loaded
 * words into one register.  The loads carry the non-temporal (streaming)
 * cache policy, as the split kernel's KV loads do.  Timing it gives the HBM rate that this exact
 * access pattern (random 16-token pages of one KV head, as laid out in the
 * [pages][Hkv][P][d] pools) reaches on the device, the practical ceiling of
 * the split kernel for that workload.  The method's access pattern is the
 * one of the PersistentKV summary pages, "Methodology / 1. Native block-table
 * decode engine" (pages read in place through the block table).
 *
 * Arguments: k_pool, v_pool: device pools [num_pool_pages][Hkv][P][head_dim]
 * of 2-byte elements; block_table: device [B][max_pages_per_row] int32;
 * plan_dev: device copy of a plan buffer (layout in pkv.h); plan_host: the
 * same plan on the host (task count and offsets are read from it); sink:
 * device buffer of at least one uint32 per task, written only in a case that
 * never happens for finite data (it keeps the loads alive).  head_dim 64 or
 * 128, page_size 16.  All pointers are caller-owned; the call is
 * asynchronous on `stream`.  Block-table entries are not checked on the
 * device.  Returns 0, -1 for a null pointer or unsupported shape, -6 when the
 * launch fails.
 */
#ifndef PKV_PROBE_H_
#define PKV_PROBE_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int pkv_probe_read(const void* k_pool, const void* v_pool, const int32_t* block_table,
                   int32_t max_pages_per_row, int32_t num_kv_heads, int32_t head_dim,
                   const void* plan_host, const void* plan_dev, uint32_t* sink,
                   hipStream_t stream);

/*
 * pkv_probe_read_lds: the same pages as pkv_probe_read (head_dim 128 only),
 * moved by gfx950's buffer loads that write LDS directly.  Each of `waves`
 * waves per workgroup keeps a ring of `depth` page slices (K 4 KiB + V 4 KiB)
 * in LDS, so deep prefetch costs LDS (waves * depth * 8 KiB per workgroup)
 * instead of registers.  With consume != 0 each page is read back from LDS
 * before its slot is reloaded and folded into sink[(task * waves + wave) * 64
 * + lane]: the sum, over that wave's pages (page_begin + wave, + waves, ...),
 * of the xor of the four 32-bit words the lane read from each of the page's
 * eight 16-byte chunks (K then V, chunk i at byte offset i * 1024 + lane * 16
 * of the 4 KiB slice); with consume == 0 that entry is 0.  sink holds at
 * least n_tasks * waves * 64 uint32.  Supported (waves, depth): (4, 2),
 * (4, 4), (8, 2), (2, 7).  Other arguments and the return codes as for
 * pkv_probe_read.
 */
int pkv_probe_read_lds(const void* k_pool, const void* v_pool, const int32_t* block_table,
                       int32_t max_pages_per_row, int32_t num_kv_heads, int32_t head_dim,
                       const void* plan_host, const void* plan_dev, int32_t waves,
                       int32_t depth, int32_t consume, uint32_t* sink, hipStream_t stream);

/*
 * pkv_probe_stream: a contiguous streaming read of `bytes` bytes of device
 * memory at `buf` (the rate HBM gives a plain sequential reader of the same
 * byte count, with no block table): `grid` workgroups of 256 threads each read
 * one contiguous chunk of bytes / grid, 16-byte non-temporal loads,
 * loads_in_flight (4 or 8) per thread.  bytes must be a multiple of
 * grid * 4096 * loads_in_flight, and bytes / grid below 2^31.  sink: at least
 * `grid` uint32, written only in a case that never happens for finite data.
 * Returns 0, -1 for bad arguments, -6 when the launch fails.
 */
int pkv_probe_stream(const void* buf, int64_t bytes, int32_t grid, int32_t loads_in_flight,
                     uint32_t* sink, hipStream_t stream);

/*
 * pkv_probe_empty: a kernel of `grid` workgroups of `threads` threads that
 * does nothing but, when flag is not NULL, copy flag[0] to flag[1] (one
 * thread).  Launched after a split kernel with the merge's grid, it measures
 * what a dependent launch costs by itself.  Returns 0, -1 for bad sizes, -6
 * when the launch fails.
 */
int pkv_probe_empty(int32_t grid, int32_t threads, uint32_t* flag, hipStream_t stream);

/*
 * pkv_probe_sleep: one wave that waits `microseconds` (0..50000) of the
 * device's constant-rate clock (hipDeviceAttributeWallClockRate) and ends;
 * it always ends, after at most a bounded number of sleep rounds.  Enqueued
 * just before the start event of a timed window, it keeps the device busy
 * while the host enqueues the window's launches, so the window measures the
 * launches and not the host's first submission.  Returns 0, -1 for a bad
 * duration, -6 when the clock rate cannot be read or the launch fails.
 */
int pkv_probe_sleep(int32_t microseconds, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H_ */
