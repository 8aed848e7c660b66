/*
 * pkv.h -- C ABI of the paged grouped-query decode-attention engine for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the decode step of "PersistentKV: Page-Aware Decode
 * Scheduling for Long-Context LLM Serving on Commodity GPUs" as summarised on
 * its gist.science pages, section "Methodology / 1. Native block-table decode
 * engine":
 *   - GQA: G = Hq / Hkv query heads share one KV head (query head h reads KV
 *     head h / G);
 *   - Layout: the engine reads K and V pages in place through a block table
 *     and never repacks them into contiguous tensors;
 *   - Sequence splitting: each row's sequence is cut into S disjoint ranges,
 *     each emitting a partial online-softmax state, and a separate merge
 *     kernel combines those states exactly;
 *   - Row-local bounds: real per-row lengths N_i (not padded ones) set the
 *     page counts and split ranges; empty splits write a neutral state and
 *     exit early;
 *   - Compact workqueue: a 1-D grid over only the non-empty
 *     (row, kv-head, split) intervals, instead of one launch pair per exact
 *     length bucket (or per padded length bucket, the coarse alternative of
 *     the "Problem statement" section).
 * Section "2. Calibrated adaptive policy" picks the execution path from the
 * batch size B and the longest context N_max with calibrated thresholds.
 *
 * Call order for one decode step of one layer:
 *     pkv_policy -> pkv_plan -> pkv_decode -> pkv_merge (no merge for NOSPLIT)
 *
 * Conventions shared by every entry point:
 *   - Ownership: every buffer is owned by the caller.  The library allocates
 *     no device or host memory and keeps no global state; all functions are
 *     re-entrant.
 *   - Streams: GPU work is enqueued asynchronously on the given stream; the
 *     library never synchronises.  A NULL stream is the default stream.
 *   - Errors: a negative pkv_status is returned and nothing is enqueued,
 *     except for PKV_EHIP from a launch that failed after earlier launches
 *     of the same call (bucketed and padded plans launch once per bucket).
 *     Arguments are validated on the host before any launch.  Block-table
 *     entries are not read on the host: an entry outside [0, num_pool_pages)
 *     among a row's first ceil(N_i / P) entries is undefined behaviour.
 *   - Layouts (all row-major, contiguous, element type = problem dtype
 *     unless stated):
 *       q, out          [B][Hq][d]
 *       k_pool, v_pool  [num_pool_pages][Hkv][P][d]   (one KV head's page is
 *                                                       one contiguous P*d run)
 *       block_table     int32 [B][max_pages_per_row]; entry j of row i is the
 *                       pool page holding tokens [j*P, (j+1)*P) of row i
 *       seq_lens        int32 [B], 0 <= N_i <= max_pages_per_row * P
 *       lse             float32 [B][Hq], natural-log sum of exp of the scaled
 *                       scores (-inf for an empty row)
 *       st_m, st_l      float32 [n_state_slots][G]    running max and sum of
 *                                                      exp(score - max)
 *       st_o            float32 [n_state_slots][G][d] unnormalised output
 *     A score is sm_scale * <q_h, k_t>.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_EINVAL = -1, /* null pointer, bad enum, non-positive size            */
  PKV_ESHAPE = -2, /* unsupported shape: Hq % Hkv, d, P, G, plan mismatch  */
  PKV_EDTYPE = -3, /* unsupported dtype                                    */
  PKV_ERANGE = -4, /* a length or split count out of range; no policy rule */
  PKV_ENOSPC = -5, /* plan buffer too small                                */
  PKV_EHIP = -6    /* a HIP call or kernel launch failed                   */
};

enum { PKV_F16 = 0, PKV_BF16 = 1 };

/* Execution paths (policy output, plan input). */
enum {
  PKV_BUCKETED = 0,  /* exact-length buckets: per bucket one rectangular
                        rows x Hkv x S split grid and one merge launch      */
  PKV_WORKQUEUE = 1, /* compact 1-D workqueue of non-empty tasks + 1 merge  */
  PKV_NOSPLIT = 2,   /* one single-pass launch, one workgroup per
                        (row, kv head), writes the normalised output        */
  PKV_PADDED = 3     /* power-of-two padded buckets: rows grouped by their
                        page count rounded up to a power of two, one
                        rows x Hkv x S split grid and one merge launch per
                        bucket, split granule from the padded length, but
                        every row keeps its row-local bound (the pages'
                        "Row-local bounds": splits past the row's real pages
                        write neutral state and read no KV)                */
};

/* Split-kernel arithmetic.  MFMA (matrix cores): head_dim 128, G <= 16.
 * VALU (vector ALU): head_dim 64 or 128, G <= 8.  AUTO, the faster one
 * measured on MI355X: MFMA for head_dim 128, VALU for head_dim 64 (so G <= 8
 * there).  pkv_decode returns PKV_ESHAPE for any other combination. */
enum { PKV_KERNEL_AUTO = 0, PKV_KERNEL_VALU = 1, PKV_KERNEL_MFMA = 2 };

typedef struct pkv_problem {
  int32_t batch;             /* B >= 1                                        */
  int32_t num_q_heads;       /* Hq >= 1                                       */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0, G = Hq/Hkv <= 16     */
  int32_t head_dim;          /* d: 64 or 128                                  */
  int32_t page_size;         /* P: 16 tokens per page                         */
  int32_t num_pool_pages;    /* pages in each of the K and V pools, >= 1      */
  int32_t max_pages_per_row; /* block-table row stride, 1 .. 2^27 - 1 (token
                                indices stay within 32 bits)                 */
  int32_t dtype;             /* PKV_F16 or PKV_BF16 (q, pools and out)        */
  float sm_scale;            /* softmax scale, e.g. 1/sqrt(d)                 */
  int32_t kernel;            /* PKV_KERNEL_*                                  */
} pkv_problem;

/* Workload counters of one plan (the scheduler-derived counters of the
 * pages' evaluation: tasks, launches per step, merge-state traffic). */
typedef struct pkv_plan_info {
  int32_t path;
  int32_t n_tasks;          /* non-empty (row, kv head, split) tasks        */
  int32_t n_buckets;        /* buckets (BUCKETED, PADDED), else 0           */
  int32_t n_launches;       /* kernel launches per step (split + merge)     */
  int32_t n_state_slots;    /* partial-state slots written by the split     */
  int32_t n_empty_slots;    /* slots that only hold a neutral state         */
  int32_t splits;           /* S, the split cap per row                     */
  int32_t pages_per_split;  /* WORKQUEUE granule (pages), else 0            */
  int64_t kv_bytes;         /* bytes of real KV tokens: sum N_i*Hkv*d*2*e   */
  int64_t merge_state_bytes;/* 2 * slots * G * (d + 2) * 4: written + read  */
  int64_t plan_bytes;       /* bytes of the plan buffer actually used       */
  int32_t max_task_pages;   /* pages of the longest task                    */
} pkv_plan_info;

/* Ordered policy rules, first match wins.  Row r is
 *   rules[6*r .. 6*r+5] = { b_lo, b_hi, nmax_lo, nmax_hi, path, splits }
 * and matches when b_lo <= B <= b_hi and nmax_lo <= N_max <= nmax_hi. */
typedef struct pkv_policy_table {
  int32_t n_rules;
  const int32_t* rules;
} pkv_policy_table;

/*
 * Plan buffer (int32 words, written by pkv_plan; callers may read it):
 *   [0]  magic 0x31564B50 ("PKV1")     [1]  path
 *   [2]  batch                          [3]  num_kv_heads
 *   [4]  splits S                       [5]  pages_per_split (WORKQUEUE)
 *   [6]  n_tasks                        [7]  n_buckets
 *   [8]  n_state_slots                  [9]  n_empty_slots
 *   [10] word offset of tasks           [11] word offset of buckets
 *   [12] word offset of bucket rows     [13] total words used
 *   [14] page_size                      [15] group G
 *   [16 ..]            row_len[B]       (N_i)
 *   [16+B ..]          row_pages[B]     (T_i = ceil(N_i / P))
 *   [16+2B ..]         row_nsplit[B]
 *   [16+3B ..]         row_task_off[B+1] (first task of each row in task
 *                      order; entry B = n_tasks)
 *   (0 to 3 zero words, so that the task list starts 16-byte aligned)
 *   tasks[n_tasks][4]  { row, (kv_head << 16) | split, page_begin, token_end }
 *                      with token_end = min(page_end * P, N_row) (so
 *                      page_end = ceil(token_end / P)), starting at word
 *                      [10], a multiple of 4
 *                      ordered (row, kv_head, split) for WORKQUEUE and
 *                      NOSPLIT, bucket by bucket for BUCKETED and PADDED;
 *                      WORKQUEUE: the state slot of task j is j
 *   buckets[n_buckets][8] { length, pages, pages_per_split, nsplit, n_rows,
 *                           first index into bucket rows, 0, 0 }
 *                      BUCKETED: ascending length; PADDED: length = -1 (rows
 *                      keep their own), pages = the padded page count
 *                      (0 or a power of two), ascending, nsplit = the
 *                      padded length's split count (a row's own count is
 *                      row_nsplit).  State slot of (row, kv_head, split) in
 *                      both: (row * Hkv + kv_head) * S + split
 *   bucket_rows[B]     rows of every bucket, bucket-major, ascending inside
 * Split s of a row covers pages [page_begin, page_end) and tokens
 * [page_begin * P, min(page_end * P, N_i)).
 */
#define PKV_PLAN_MAGIC 0x31564B50
#define PKV_PLAN_HEADER_WORDS 16

/* Upper bound, in bytes, of the plan buffer for this problem, path and
 * split cap.  Returns 0 on invalid arguments. */
size_t pkv_plan_bytes(const pkv_problem* prob, int32_t path, int32_t max_splits);

/*
 * Build the plan on the host from the host copy of the row lengths, write it
 * to plan_host and, when plan_dev is not NULL, enqueue one host-to-device
 * copy of the used bytes on `stream` (plan_host should then be pinned and
 * must stay unchanged until the copy has run).  Split rules (row-local
 * bounds, see the header comment):
 *   WORKQUEUE: pps = max(1, ceil(T_max / S)) pages, shared by the batch; row i
 *              gets ceil(T_i / pps) splits; tasks only for non-empty splits.
 *   BUCKETED:  rows grouped by exact length; bucket b uses
 *              pps_b = max(1, ceil(T_b / S)) and ceil(T_b / pps_b) splits;
 *              its grid has rows_b * Hkv * S slots, the rest neutral.
 *   PADDED:    rows grouped by T_i rounded up to a power of two (0 stays 0);
 *              bucket b uses pps_b = max(1, ceil(T_pad / S)) pages; row i
 *              gets ceil(T_i / pps_b) splits (row-local bound), the last
 *              ending at T_i; its grid has rows_b * Hkv * S slots, the rest
 *              neutral.
 *   NOSPLIT:   one task per (row, kv head) of every non-empty row.
 * The whole buffer of pkv_plan_bytes bytes is working memory: bucketed and
 * padded plans order their rows in its last B words before moving the order
 * into place, so words past the used length are unspecified afterwards.
 * Errors: PKV_EINVAL (null pointer, max_splits < 1 or > 65535, bad path),
 * PKV_ESHAPE (problem shape), PKV_ERANGE (N_i < 0 or N_i > max_pages_per_row*P,
 * or more than 2^31 - 1 tasks, state slots or plan words), PKV_ENOSPC (plan_bytes too
 * small), PKV_EHIP (the copy failed to enqueue).  info_out may be NULL.
 */
pkv_status pkv_plan(const pkv_problem* prob, const int32_t* seq_lens_host, int32_t path,
                    int32_t max_splits, void* plan_host, void* plan_dev, size_t plan_bytes,
                    pkv_plan_info* info_out, hipStream_t stream);

/* Counters of an existing plan (reads plan_host only). */
pkv_status pkv_plan_get_info(const pkv_problem* prob, const void* plan_host,
                             pkv_plan_info* info_out);

/*
 * Split decode (the engine's first kernel, or the whole step for NOSPLIT).
 * plan_host is read for launch shapes; plan_dev (the device copy of the same
 * plan, already enqueued on `stream`) is read by the kernels.
 *   WORKQUEUE / BUCKETED / PADDED: writes st_m, st_l, st_o for all n_state_slots
 *     slots (neutral (-inf, 0, 0) for empty slots); out and lse are unused.
 *   NOSPLIT: writes out (and lse when not NULL) for every row; st_* unused
 *     and may be NULL.  Rows with N_i = 0 get out = 0, lse = -inf.
 * Tokens past N_i in a row's last page, and pool pages not referenced by the
 * first T_i table entries of a row, are never used (they may hold NaN).
 * Every path takes the row lengths N_i from the plan (the lengths pkv_plan
 * validated); seq_lens_dev is not read and may be NULL.
 * Errors: PKV_EINVAL, PKV_ESHAPE (shape or plan/problem mismatch),
 * PKV_EDTYPE, PKV_ERANGE (a launch of more than 2^24 - 1 workgroups: tasks,
 * B * Hkv for NOSPLIT, or rows_b * Hkv * S for one bucket; or a bucket of
 * more than 65535 rows, the limit of its launch's third grid dimension),
 * PKV_EHIP.
 */
pkv_status pkv_decode(const pkv_problem* prob, const void* plan_host, const void* plan_dev,
                      const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens_dev, float* st_m,
                      float* st_l, float* st_o, void* out, float* lse, hipStream_t stream);

/*
 * Merge (the engine's second kernel): for each (row, q head) combine the
 * row's partial states exactly: M = max_s m_s, w_s = exp(m_s - M),
 * L = sum_s w_s l_s, out = sum_s w_s o_s / L rounded to nearest-even into the
 * problem dtype, lse = M + ln L.  All-neutral rows give out = 0, lse = -inf.
 * WORKQUEUE: one launch; BUCKETED / PADDED: one launch per bucket;
 * NOSPLIT: no-op.
 * lse may be NULL.  Errors as pkv_decode; PKV_ERANGE when a launch's rows
 * times Hq exceed 2^24 - 1 workgroups.
 */
pkv_status pkv_merge(const pkv_problem* prob, const void* plan_host, const void* plan_dev,
                     const float* st_m, const float* st_l, const float* st_o, void* out,
                     float* lse, hipStream_t stream);

/*
 * Learned cost model (an alternative to the threshold table; the pages leave
 * a learned model as future work: es page, "Significado y
 * Reivindicaciones" / "Direcciones Futuras").  For a candidate
 * (path, split cap) the features f[0..PKV_COST_FEATURES) of its plan are
 *   f0 = 1
 *   f1 = kernel launches per step
 *   f2 = real-KV megabytes, sum N_i * Hkv * d * 2 * 2 / 1e6
 *   f3 = merge-state megabytes, 2 * n_state_slots * G * (d + 2) * 4 / 1e6
 *   f4 = per-CU critical pages: for each split launch, grid item j (the
 *        launch's workgroups in grid order: tasks for WORKQUEUE, (row, kv
 *        head) for NOSPLIT, (bucket row, kv head, split slot) for the bucket
 *        paths, empty slots counting 0 pages) is charged to CU j mod num_cus;
 *        f4 sums over the launches the largest page total of one CU
 *   f5 = grid items of all split launches / 1000
 *   f6 = non-empty tasks / 1000
 *   f7 = pages of the largest task / 100 (WORKQUEUE: min(granule, T_max);
 *        bucket paths: the largest min(granule, longest row) over the
 *        buckets; NOSPLIT: T_max)
 * with the counters pkv_plan would report, and the model predicts the step
 * time in microseconds as sum_j weights[path][j] * f_j.  pkv_policy_model
 * returns the candidate with the smallest prediction (the first one on a
 * tie) and, when predicted_us_out is not NULL, that prediction.
 * The weights hold for one split kernel: the caller passes the weights fitted
 * for the kernel pkv_decode will run on this problem (the shipped model has
 * one set for the matrix-core kernel at G <= 8, one for its G > 8 variant
 * and one for the vector-ALU kernel).
 * num_cus (1..1024): the device's compute units the model was fitted with.
 * scratch_host: B int32 of caller memory, used for bucket orders (may be
 * NULL when no candidate is BUCKETED or PADDED).  NOSPLIT candidates ignore
 * their split cap.  Host only, nothing is enqueued; cost O(B + tasks) per
 * candidate.  Errors: PKV_EINVAL (null pointer, empty model, num_cus out of
 * range, a candidate with an unknown path or a split cap outside
 * [1, 65535]), PKV_ESHAPE, PKV_EDTYPE, PKV_ERANGE (a length outside
 * [0, max_pages_per_row * P]).
 */
#define PKV_COST_FEATURES 8

typedef struct pkv_cost_model {
  int32_t n_candidates;
  const int32_t* candidates; /* [n_candidates][2] = { path, split cap }       */
  const float* weights;      /* [4][PKV_COST_FEATURES], one row per path id   */
  int32_t num_cus;           /* compute units used for feature f4             */
} pkv_cost_model;

pkv_status pkv_cost_features(const pkv_problem* prob, const int32_t* seq_lens_host, int32_t path,
                             int32_t max_splits, int32_t num_cus, int32_t* scratch_host,
                             float* features_out);
pkv_status pkv_policy_model(const pkv_problem* prob, const pkv_cost_model* model,
                            const int32_t* seq_lens_host, int32_t* scratch_host,
                            int32_t* path_out, int32_t* splits_out, float* predicted_us_out);

/*
 * Device-planned workqueue step (no host round trip, graph-capturable).
 *
 * pkv_plan_device builds the WORKQUEUE plan on the GPU from the device copy
 * of the row lengths, in the same layout (and with the same contents, for
 * valid lengths) as pkv_plan(..., PKV_WORKQUEUE, ...).  plan_bytes must be at
 * least pkv_plan_bytes(prob, PKV_WORKQUEUE, max_splits); batch <= 16384,
 * and that size in 32-bit words at most 2^31 - 1 (else PKV_ERANGE).
 * Lengths cannot be
 * checked on the host: a row whose length lies outside
 * [0, max_pages_per_row * P] is planned as an empty row, and the number of
 * such rows is written to *bad_rows_dev when it is not NULL.
 *
 * pkv_decode_device runs the split kernel as a persistent grid (about as
 * many workgroups as fit on the device at once, at most B * Hkv *
 * max_splits): workgroup w runs task w, and further tasks are claimed
 * through a work counter kept in plan word [total_words] (just past the task
 * list; pkv_plan_bytes leaves room for it).  pkv_plan_device zeroes the
 * counter and pkv_merge_device resets it, so every pkv_decode_device must
 * follow a pkv_plan_device or a pkv_merge_device on the same plan; calls
 * that overlap on one plan race.  It writes st_m, st_l, st_o exactly as
 * pkv_decode does for the WORKQUEUE path (slot = task index); the state
 * buffers must hold B * Hkv * max_splits slots.  The split kernel is chosen
 * and the shape checked as for pkv_decode (PKV_ESHAPE where no kernel covers
 * it).
 *
 * pkv_merge_device combines the states into out / lse (lse may be NULL) using
 * the device plan's row arrays.  The three calls are ordered on `stream`.
 * Errors as pkv_plan / pkv_decode / pkv_merge.
 */
pkv_status pkv_plan_device(const pkv_problem* prob, const int32_t* seq_lens_dev,
                           int32_t max_splits, void* plan_dev, size_t plan_bytes,
                           int32_t* bad_rows_dev, hipStream_t stream);
pkv_status pkv_decode_device(const pkv_problem* prob, const void* plan_dev, int32_t max_splits,
                             const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, float* st_m, float* st_l, float* st_o,
                             hipStream_t stream);
pkv_status pkv_merge_device(const pkv_problem* prob, const void* plan_dev, const float* st_m,
                            const float* st_l, const float* st_o, void* out, float* lse,
                            hipStream_t stream);

/*
 * Self-planned workqueue step: the device-planned step without a plan (two
 * launches, no planner kernel, no plan buffer).  Same method ("Row-local
 * bounds", "Compact workqueue") and the same tasks, slots and results as
 * pkv_plan_device + pkv_decode_device + pkv_merge_device: every workgroup of
 * the split kernel derives the workqueue of the device lengths in its own
 * LDS (O(B) work per workgroup), and every merge workgroup derives its row's
 * split count and first slot the same way.
 *   seq_lens_dev: int32 [B] on the device, read by both calls; a length
 *     outside [0, max_pages_per_row * P] is treated as an empty row (out 0,
 *     lse -inf).  It must not change between the two calls.
 *   work_counter_dev: one int32 of device memory, owned by the caller, zero
 *     before the first pkv_decode_selfplan (for instance hipMemset once at
 *     allocation).  The split kernel claims tasks through it and
 *     pkv_merge_selfplan sets it back to zero, so every pkv_decode_selfplan
 *     must be followed by its pkv_merge_selfplan before the counter is used
 *     again; calls that overlap on one counter race.
 *   st_m, st_l, st_o: as pkv_decode_device (B * Hkv * max_splits slots).
 * batch <= 1024 and B * Hkv * max_splits <= 2^31 - 1 (else PKV_ERANGE);
 * the split kernel is chosen and the shape checked as for pkv_decode.
 * Errors: PKV_EINVAL, PKV_ESHAPE, PKV_EDTYPE, PKV_ERANGE, PKV_EHIP.
 */
pkv_status pkv_decode_selfplan(const pkv_problem* prob, const int32_t* seq_lens_dev,
                               int32_t max_splits, int32_t* work_counter_dev, const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_table, float* st_m, float* st_l, float* st_o,
                               hipStream_t stream);
pkv_status pkv_merge_selfplan(const pkv_problem* prob, const int32_t* seq_lens_dev,
                              int32_t max_splits, int32_t* work_counter_dev, const float* st_m,
                              const float* st_l, const float* st_o, void* out, float* lse,
                              hipStream_t stream);

/*
 * KV append: store the step's new key and value of every row in the paged
 * pools before attention (the input side of a decode step; not described on
 * the pages).  k_new, v_new: [B][Hkv][d] in the problem dtype.  positions_dev:
 * int32 [B], the token position to write for each row (its length before the
 * step); row i's token p goes to pool page block_table[i][p / P], slot p % P.
 * A negative position marks an inactive row; positions at or past
 * max_pages_per_row * P are skipped.  The block-table entry of the written
 * page must be a valid pool page (undefined behaviour otherwise, as for
 * pkv_decode).  Errors: PKV_EINVAL, PKV_ESHAPE, PKV_EDTYPE, PKV_ERANGE
 * (B * Hkv above 2^24 - 1), PKV_EHIP.
 */
pkv_status pkv_append_kv(const pkv_problem* prob, const void* k_new, const void* v_new,
                         const int32_t* block_table, const int32_t* positions_dev, void* k_pool,
                         void* v_pool, hipStream_t stream);

/*
 * Calibrated path choice: first rule of `table` matching (batch, max_len).
 * Writes the rule's path and split cap.  Errors: PKV_EINVAL (null pointer,
 * negative n_rules, a rule with an unknown path or splits < 1),
 * PKV_ERANGE (no rule matches; outputs untouched).
 */
pkv_status pkv_policy(const pkv_policy_table* table, int32_t batch, int32_t max_len,
                      int32_t* path_out, int32_t* splits_out);

/*
 * Default path choice of the engine: for B = 1 the calibrated table's rule
 * for (1, N_1) (pkv_policy: the one row's length fixes the workload); for
 * B >= 2 the learned cost model's choice (the smallest prediction, as
 * pkv_policy_model) among its candidates and the CU-balanced workqueue caps
 * (pkv_balanced_splits with per_cu = 1 and 2, bounded by the largest
 * WORKQUEUE split cap among the candidates; a cap already listed, or 0, is
 * not added, and on equal predictions the listed candidate wins), because
 * with several rows the length mix, not only (B, N_max), decides how evenly
 * the split launch loads the CUs.  The pages
 * calibrate thresholds on (B, N_max) ("Metodologia / 2. Politica Adaptativa
 * Calibrada", es page) and name a learned cost model as the next step
 * ("Significado y Reivindicaciones" / "Direcciones Futuras"); this policy
 * keeps the first where it sees the whole workload and takes the second
 * elsewhere.  Host only.  scratch_host as for pkv_policy_model.
 * Errors: PKV_EINVAL (null pointer, or as pkv_policy / pkv_policy_model),
 * PKV_ESHAPE, PKV_EDTYPE, PKV_ERANGE (a length outside
 * [0, max_pages_per_row * P], or no table rule matches at B = 1).
 */
pkv_status pkv_policy_default(const pkv_policy_table* table, const pkv_cost_model* model,
                              const pkv_problem* prob, const int32_t* seq_lens_host,
                              int32_t* scratch_host, int32_t* path_out, int32_t* splits_out);

/*
 * CU-balanced split cap of the compact workqueue: the largest S in
 * [1, max_splits] whose WORKQUEUE plan (pkv_plan's task count, Hkv * sum_i
 * ceil(T_i / ceil(T_max / S))) holds at most per_cu * num_cus tasks, so that
 * one launch deals every CU at most about per_cu tasks of near-equal size;
 * *splits_out = 0 when even S = 1 holds more.  The split rule of the pages
 * ("Row-local bounds", "Compact workqueue") is unchanged: S, the split cap
 * a policy chooses, only sets the granule, and the default policy scores
 * this cap beside its listed candidates.  Host only, O(B log max_splits).
 * num_cus 1..1024, per_cu 1..64, max_splits 1..65535.  Errors: PKV_EINVAL
 * (null pointer, an argument out of range), PKV_ESHAPE, PKV_EDTYPE,
 * PKV_ERANGE (a length outside [0, max_pages_per_row * P]).
 */
pkv_status pkv_balanced_splits(const pkv_problem* prob, const int32_t* seq_lens_host,
                               int32_t num_cus, int32_t per_cu, int32_t max_splits,
                               int32_t* splits_out);

/*
 * Decode step that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It is pkv_decode_selfplan followed by
 * pkv_merge_selfplan (the same self-planned workqueue, the same two kernels,
 * results bit-identical to that pair) with two differences:
 *   - the partial states live in a device array owned by the library,
 *     PKV_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 *     until the process ends; pkv_noalloc_bytes(prob, max_splits) states how
 *     much of it a call needs (B * Hkv * max_splits slots of G * (d + 2)
 *     floats), and a call needing more fails with PKV_ENOSPC;
 *   - the split launch has one workgroup per possible task (B * Hkv *
 *     max_splits, at most 2^24 - 1, else PKV_ERANGE), so no claim counter is
 *     used and nothing in the array has to start at zero.
 * The caller passes the inputs (as pkv_decode_selfplan) and the outputs out
 * [B][Hq][d] and lse [B][Hq] (lse may be NULL).  Every call on one GPU uses
 * that GPU's one array, which keeps the last call's contents: calls that
 * overlap on one GPU (on different streams, or from different threads
 * without ordering) race.  The first call on a device looks up the array's
 * device address (hipGetSymbolAddress) with that device current; no call
 * allocates.  Errors: as pkv_decode_selfplan, plus PKV_ENOSPC.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

size_t pkv_noalloc_bytes(const pkv_problem* prob, int32_t max_splits);
pkv_status pkv_attend_noalloc(const pkv_problem* prob, const int32_t* seq_lens_dev,
                              int32_t max_splits, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table, void* out,
                              float* lse, hipStream_t stream);

/* Static description of a status code; never NULL. */
const char* pkv_status_str(pkv_status status);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
