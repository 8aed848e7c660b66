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

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H_ */
