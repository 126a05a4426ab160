/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) multi-head latent attention
 * (MLA) decode library, libmla_decode.so: one query token per sequence, or
 * several (mla_decode_plan_multi).
 *
 * The operation.  For every sequence b of a batch and every query head h
 * (16 heads share one latent KV head):
 *
 *   s_t       = sm_scale * < q[b,h,0:576], c_t[0:576] >
 *   out[b,h,:] = sum_t softmax(s)_t * c_t[0:512]
 *
 * where c_t is the dequantised 576-wide cache row of token t (512 latent +
 * 64 rope columns) and V is the first 512 columns of the same row.  This is
 * the decode step of the amd-mixed-mla submissions: submission 599694
 * ("overhead elimination"), function `_bmm` and kernel `_flash_fp8_single`;
 * submission 727205 ("v25: LEAN"), kernels `mla_s1` (split-K stage 1) and
 * `mla_rd` (stage 2 merge); submission 700955 ("locked baseline dispatch"),
 * kernels `mla_attn_v71` / `reduce_lse_v71`.
 *
 * Cache formats (one per handle):
 *   MLA_KV_BF16      rows of 576 bf16 (1152 bytes).
 *   MLA_KV_FP8_E4M3  rows of 576 OCP e4m3fn codes (576 bytes); value = code x
 *                    kv_scale, kv_scale one fp32 for the whole tensor, read
 *                    from device memory (599694, `_flash_fp8_single`).
 *   MLA_KV_MXFP4     rows of 288 bytes of e2m1 nibbles (element 2i in the low
 *                    nibble of byte i) plus, in a separate array, one e8m0
 *                    scale byte per 32 elements (18 per row, row stride >= 18);
 *                    value = e2m1 x 2^(e-127) (700955, `mla_attn_v71`).
 *
 * Addressing.  With page_size == 1 the rows of sequence b are
 * kv[kv_indptr[b] .. kv_indptr[b+1]).  With page_size > 1 (a power of two),
 * kv is viewed as pages of page_size rows; kv_indptr counts pages, the pages
 * of sequence b are kv_page_indices[kv_indptr[b] .. kv_indptr[b+1]) and its
 * last page holds kv_last_page_len[b] (1..page_size) valid tokens; logical
 * token j lives in row page*page_size + j%page_size.  A sequence of length 0
 * produces a zero output.
 *
 * Execution.  Each workgroup of the split kernel streams one token range
 * ("work item") of one sequence with an online softmax and writes either the
 * output (the item is the whole sequence) or a normalised partial and its
 * log-sum-exp; the partials of every split sequence are merged by their
 * log-sum-exp weights (727205 `mla_rd`, 700955 `reduce_lse_v71`, 599694
 * `_flash_fp8_split_s2`).  For sequences of different lengths the planner
 * cuts the batch into bins of about equal work, one per resident workgroup,
 * and a workgroup runs the items of its bin in turn (a sequence may span
 * bins).  The merge is a second kernel launch, except for a bf16 cache
 * whose plan's items differ in length (at most 12 per sequence): there the
 * item of a sequence that finishes last merges its partials, so each call is
 * one launch.  fp8 and MXFP4 plans hand their partials to the merge kernel
 * as bf16, which measured faster than merging them inside the split kernel.
 * No merge runs when no sequence is split.  The completion counters of that merge belong to the plan: runs of
 * one handle must not overlap (on any streams).  A plan may be made while
 * runs of the previous plan are still executing: it builds the work list on
 * the host and uploads it, without waiting, into the other of the handle's
 * two plan buffers (a decode loop re-plans every step as its sequences
 * grow).
 *
 * Ownership.  The caller owns every tensor, the workspace and the stream.  A
 * handle owns only its plan (a small device work list, allocated by
 * mla_decode_plan and freed by mla_decode_destroy).  All pointers passed to mla_decode_run are device
 * pointers unless the name ends in _host.
 *
 * Errors.  Every call validates its arguments on the host before touching the
 * GPU and returns a status; nothing is launched when a call fails, no
 * exception crosses the ABI and the process is never terminated.  Launch
 * failures map to MLA_ERR_HIP; faults inside a kernel surface at the caller's
 * next synchronisation.  mla_decode_last_error() gives a per-handle message.
 *
 * Threading.  A handle may be used from one host thread at a time.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_KV_BF16 = 0,
  MLA_KV_FP8_E4M3 = 1,
  MLA_KV_MXFP4 = 2
} mla_kv_dtype;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,          /* null pointer, bad size, inconsistent indptr ... */
  MLA_ERR_UNSUPPORTED = 2,          /* shape or option this library does not implement */
  MLA_ERR_NOT_PLANNED = 3,          /* run before a successful plan */
  MLA_ERR_WORKSPACE_TOO_SMALL = 4,  /* workspace_bytes below the planned size */
  MLA_ERR_HIP = 5                   /* a HIP runtime call failed */
} mla_status;

typedef struct mla_decode_s* mla_decode_t;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int mla_decode_version(void);

/* Human-readable name of a status code (static storage). */
const char* mla_status_string(mla_status s);

/*
 * Create a handle.  Supported: num_heads 16, qk_dim 576, v_dim 512 (the
 * shape of the amd-mixed-mla task, 727205 module constants), any finite
 * sm_scale > 0 (the task uses 1/sqrt(576)), page_size a power of two in
 * [1, 1024].  `device` is the HIP device ordinal the handle will run on; it
 * is not touched until mla_decode_plan.  *out is set to NULL on failure.
 */
mla_status mla_decode_create(mla_decode_t* out, int device, int num_heads, int qk_dim, int v_dim,
                             float sm_scale, mla_kv_dtype kv_dtype, int page_size);

/*
 * Plan a batch: splits every sequence into work items (token ranges, whole
 * tiles of the format's split kernel -- 128 tokens for fp8 and MXFP4, 64 for
 * bf16 -- except at a sequence's end or under split_override, which cuts at
 * 32-token boundaries) sized against the device's compute-unit count and
 * the stage-1 kernel's residency (up to 256 items for one long sequence),
 * uploads the work list to the device and reports the workspace size the
 * run needs (bytes; may be 0).  The upload goes from pinned host memory on a
 * stream of the handle, ordered after the runs that read the buffer it
 * overwrites; the host does not wait for it (except to reuse a host buffer
 * whose upload from two plans ago is still queued), and the first run of the
 * plan on each stream waits for it on the device.  The first plan of a
 * handle (and one that needs a larger buffer) allocates device and pinned
 * host memory.  This is the host planner of 700955 ("locked baseline
 * dispatch"), `_compute_custom_splits` (split counts from the batch and the
 * compute units), rebuilt around the stage-1 kernel's measured residency.  kv_indptr_host has batch+1 entries (tokens if
 * page_size == 1, pages otherwise; non-decreasing, starting anywhere >= 0);
 * kv_last_page_len_host has batch entries when page_size > 1 and is ignored
 * (may be NULL) otherwise.  split_override > 0 forces that many items per
 * non-empty sequence (at most one per 32 tokens); 0 lets the planner choose.
 * The plan stays valid until the next plan or destroy; the device copies of
 * kv_indptr / kv_last_page_len passed to run must hold the same values (the
 * work list carries each sequence's kv_indptr entry as planned, and the
 * kernels address the cache through it).
 */
mla_status mla_decode_plan(mla_decode_t h, int batch, const int32_t* kv_indptr_host,
                           const int32_t* kv_last_page_len_host, int split_override,
                           size_t* workspace_bytes);

/*
 * The planner alone, on the host, for inspection and testing (no handle, no
 * GPU).  Same inputs as mla_decode_plan plus the cache format (items are
 * whole tiles of its split kernel: 64 tokens for bf16, 128 otherwise) and
 * the device figures it would read (compute units, resident stage-1
 * workgroups per unit).  Writes up to
 * max_items work items as rows of five int32 (sequence, first token, end
 * token, partial slot or -1 when the item is the whole sequence or -2 for the
 * item that writes an empty sequence's zero output, and the workgroup that
 * runs it) in launch order, and the number of items, partial slots and the
 * workspace bytes.  A ragged batch is cut into bins of about equal work, one
 * per resident workgroup, whose items one workgroup runs in turn; otherwise
 * each item has a workgroup of its own.
 * Returns MLA_ERR_INVALID_ARG when max_items is too small (num_items still
 * set).
 */
mla_status mla_decode_plan_preview(int batch, const int32_t* kv_indptr_host,
                                   const int32_t* kv_last_page_len_host, int page_size,
                                   mla_kv_dtype kv_dtype, int split_override, int num_cus,
                                   int blocks_per_cu, int32_t* items_out, int max_items,
                                   int* num_items, int* num_slots, size_t* workspace_bytes);

/*
 * Multi-token decode: a plan for several query tokens per sequence (draft
 * tokens being verified, or a chunk of new tokens).  The submissions call
 * aiter's decode with one query token per sequence (qo_indptr = 0, 1, ..,
 * batch and a maximum query length of 1: 599694 "overhead elimination", its
 * aiter path; 727205 "v25: LEAN", its metadata call); this takes the same
 * qo_indptr argument with longer query runs.
 *   qo_indptr_host  int32 [batch+1], qo_indptr[0] = 0, non-decreasing; sequence
 *                   b has q_b = qo_indptr[b+1] - qo_indptr[b] query tokens,
 *                   0 <= q_b <= its cache length n_b, at least one in all.
 * Query token j of sequence b is row r = qo_indptr[b] + j of q
 * [qo_indptr[batch], 16, 576] and of out [qo_indptr[batch], 16, 512].  It is
 * the token at position n_b - q_b + j of its sequence, whose cache already
 * holds the rows of all its query tokens, and it attends causally: to cache
 * tokens 0 .. n_b - q_b + j.  A sequence with q_b = 0 produces no row.  The
 * other arguments, the run call and the errors are those of mla_decode_plan;
 * with q_b = 1 everywhere the plan is the single-token plan.  Each row's
 * cache range is read by its own items; the copies for the q_b rows of a
 * sequence are launched together so that they stream the same rows at the
 * same time.
 */
mla_status mla_decode_plan_multi(mla_decode_t h, int batch, const int32_t* qo_indptr_host,
                                 const int32_t* kv_indptr_host, const int32_t* kv_last_page_len_host,
                                 int split_override, size_t* workspace_bytes);

/* mla_decode_plan_preview for a multi-token plan (see mla_decode_plan_multi);
 * the first column of an item row is the query row. */
mla_status mla_decode_plan_preview_multi(int batch, const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                                         const int32_t* kv_last_page_len_host, int page_size,
                                         mla_kv_dtype kv_dtype, int split_override, int num_cus,
                                         int blocks_per_cu, int32_t* items_out, int max_items,
                                         int* num_items, int* num_slots, size_t* workspace_bytes);

/*
 * Describe the current plan: number of work items (workgroups launched,
 * unless the plan has bins: see mla_decode_plan_preview), the largest number
 * of items given to one sequence, and the number of partials written to the
 * workspace.  Any output pointer may be NULL.
 */
mla_status mla_decode_plan_info(mla_decode_t h, int* num_items, int* max_splits,
                                int* num_partials);

/*
 * Run the planned decode on `stream` (a hipStream_t; NULL = the default
 * stream).  Asynchronous: no allocation, no host synchronisation.  The split
 * kernel, then (when the plan needs one) the log-sum-exp merge, on that one
 * stream: the launchers `run_s1` / `run_rd` of 727205 ("v25: LEAN") and
 * `hip_mla_v71` of 700955 ("locked baseline dispatch"), with the work list of
 * the plan in place of their (batch x splits) grids.
 *   q                 bf16 [batch, 16, 576], row-major, 16-byte aligned.
 *   kv                cache rows (layout above), 16-byte aligned; may be NULL
 *                     only when every planned sequence is empty.
 *   kv_scales         FP8: float32[1] per-tensor scale.  MXFP4: uint8
 *                     [rows, kv_scale_stride] e8m0 scales.  BF16: ignored.
 *   kv_scale_stride   MXFP4 scale row stride in bytes (>= 18); else ignored.
 *   kv_indptr         int32 [batch+1] (as planned).
 *   kv_page_indices   int32 page ids (page_size > 1), else ignored.
 *   kv_last_page_len  int32 [batch] (page_size > 1), else ignored.
 *   out               bf16 [batch, 16, 512], row-major, 16-byte aligned; every
 *                     element written.
 *   workspace         device scratch of >= the planned size (16-byte aligned;
 *                     may be NULL when the planned size is 0).  Its contents
 *                     need no initialisation and are garbage afterwards.
 */
mla_status mla_decode_run(mla_decode_t h, const void* q, const void* kv, const void* kv_scales,
                          int64_t kv_scale_stride, const int32_t* kv_indptr,
                          const int32_t* kv_page_indices, const int32_t* kv_last_page_len,
                          void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_run without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the partials go to a device array of the library
 * (MLA_SCRATCH_BYTES, 16 MiB, room for 511 partials), which each GPU the
 * library runs on holds until the process ends.  No allocation, no host
 * synchronisation; the arguments are those of mla_decode_run less the
 * workspace.  Every call on one GPU shares that GPU's array: calls that
 * overlap on a GPU (from any handle, on any stream) race, and must be
 * ordered by the caller.  Nothing in the array needs clearing: a run writes
 * every partial it reads.  A plan whose workspace_bytes exceed
 * MLA_SCRATCH_BYTES is refused with MLA_ERR_UNSUPPORTED before any launch.
 */
#define MLA_SCRATCH_BYTES (16u << 20)
mla_status mla_decode_run_noalloc(mla_decode_t h, const void* q, const void* kv, const void* kv_scales,
                                  int64_t kv_scale_stride, const int32_t* kv_indptr,
                                  const int32_t* kv_page_indices, const int32_t* kv_last_page_len, void* out,
                                  void* stream);

/*
 * Precision of the query in the score contraction of the fp8 and MXFP4 split
 * kernels.  Default MLA_QUERY_EXACT: each query element enters as the sum of
 * two e4m3 codes (hi + lo) after a power-of-two scaling per (row, head), which
 * keeps every element exactly but those below 2^-10 of the head's largest.
 * MLA_QUERY_E4M3: each element enters as one e4m3 code -- the query row of
 * each head is scaled by the power of two 2^s that puts its largest |q| in
 * [128, 256), and q * 2^s is rounded to the nearest e4m3 value, ties to even
 * -- so the scores take one matrix product instead of two.  This is the
 * low-precision query of submission 599694 ("overhead elimination", the
 * static fp8 query scale of its fast path), with the scale found per row and
 * head instead of fixed in advance.  It rounds the query to 4 significant
 * bits: scores move by up to 2^-4 of |q|.|c_t| per element, which is harmless
 * on well-scaled caches but not on caches whose rows reach large magnitudes.
 * MLA_ERR_UNSUPPORTED for a bf16 cache; an MXFP4 run with an odd scale
 * stride or scale address (which uses the bf16-decoding kernel) is refused
 * with MLA_ERR_UNSUPPORTED while MLA_QUERY_E4M3 is set.  Takes effect from
 * the next run; MLA_ERR_INVALID_ARG for any other value.
 */
typedef enum {
  MLA_QUERY_EXACT = 0,
  MLA_QUERY_E4M3 = 1
} mla_query_format;

mla_status mla_decode_set_query_format(mla_decode_t h, int query_format);

/*
 * Kernel timing for measurement.  While enabled, mla_decode_run launches its
 * kernels with a pair of HIP events each, which the launch itself records
 * when the kernel starts and when it ends (hipExtLaunchKernel);
 * mla_decode_kernel_time_ms then waits for the last run's events and returns
 * the elapsed milliseconds of kernel `which` (0 = split stage, 1 = merge; a
 * merge that was not launched reports 0).  MLA_ERR_NOT_PLANNED if the last
 * run was not timed.
 */
mla_status mla_decode_set_profiling(mla_decode_t h, int enable);
mla_status mla_decode_kernel_time_ms(mla_decode_t h, int which, float* ms);

/*
 * Static resource usage of kernel `which` (0 = the split-stage kernel that
 * mla_decode_run launches for this handle's format, layout, query format and
 * current plan, for an MXFP4 scale array at even addresses; 1 = merge):
 * registers per lane, LDS bytes per workgroup, scratch (spill) bytes per
 * lane.  Any output pointer may be NULL.
 */
mla_status mla_decode_kernel_resources(mla_decode_t h, int which, int* vgprs, int* lds_bytes,
                                       int* scratch_bytes);

/*
 * Destroy a handle (NULL is accepted and ignored): frees its plan buffers,
 * upload stream and events.  No run of the handle may still be executing.
 * (The pages keep such per-shape state in module-level caches: 727205
 * `_cache`, 700955 `_cache` and `_custom_v71_scratch_cache`.)
 */
mla_status mla_decode_destroy(mla_decode_t h);

/* Detail of the last failure on this handle (empty string if none). */
const char* mla_decode_last_error(mla_decode_t h);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
