/*
 * splitkv.h -- C ABI of libsplitkv: exact split-KV attention on AMD MI355X (gfx950).
 *
 * The problem (Split-KV page, lede and "Timeline"): queries are a short block of
 * trailing tokens; keys/values are a long context kept where they are and cut into
 * context KV blocks; each block produces a result the size of the queries; the
 * results combine into exactly the unsharded attention; blocks are placed on
 * workers by a cost-aware longest-processing-time-first (LPT) plan whose load
 * imbalance the method reports. On one GPU the workers are workgroups, one per
 * compute unit.
 *
 * The pages print no formulas; this library uses the textbook ones:
 *   query row i of sequence s sits at position p_i = n_s - q_s + i and, with the
 *   causal mask, sees keys 0..p_i (bottom-right alignment); score = scale * <q, k>;
 *   query head h reads KV head h / (Hq / Hkv); a block's partial is
 *   O_b = sum_j e^{s_j} v_j / sum_j e^{s_j} and LSE_b = ln sum_j e^{s_j} over the
 *   block's visible keys (O_b = 0, LSE_b = -inf when none is visible); the merge is
 *   M = max_b LSE_b, w_b = e^{LSE_b - M}, O = sum_b w_b O_b / sum_b w_b,
 *   LSE = M + ln sum_b w_b (natural log), which equals unsharded softmax attention.
 *
 * Conventions
 *   - Every function returns an int status: SPLITKV_OK (0) or a negative error.
 *     Argument errors are reported before any HIP call is made.
 *   - Device memory (Q, K, V, plan buffer, workspace, outputs) is owned by the
 *     caller. The library never allocates or frees device memory and never
 *     synchronises a stream: kernels are enqueued on the caller's stream and
 *     execution errors surface at the caller's next synchronisation.
 *   - Plans are library-owned host objects (splitkv_plan_t, made by splitkv_plan, released by splitkv_plan_destroy).
 *   - Functions are thread-safe for distinct plans; splitkv_last_error() is per thread.
 *
 * Layouts (all packed by sequence, in batch order)
 *   Q   [sum_s q_s, Hq,  D]  element (t, h, d) at q + t*q_stride_tok + h*q_stride_head + d
 *   K,V [sum_s n_s, Hkv, D]  likewise with their own strides; d is contiguous
 *   out [sum_s q_s, Hq,  D]  fp32, contiguous
 *   lse [sum_s q_s, Hq]      fp32, natural log, contiguous
 *   Workspace: partial outputs first, then partial LSEs at byte offset
 *   info.ws_lse_offset. The partial of unit (s, b, kv head k) for query row
 *   r = i*g + (h - k*g) (query token i, query head h) is row
 *       R = seq_row_base[s] + (k * nb_s + b) * (q_s * g) + r
 *   with nb_s = ceil(n_s / B), g = Hq / Hkv and seq_row_base[s] the sum over earlier
 *   sequences of nb_t * Hkv * q_t * g. With SPLITKV_PARTIAL_F32 its output is the fp32
 *   ws[R*D .. R*D + D) and its LSE the fp32 ws_lse[R]. With SPLITKV_PARTIAL_F16_ROWSCALE
 *   its output is the fp16 elements ws_h[R*D .. R*D + D) (ws_h = the workspace base as
 *   fp16) times a row scale, and ws_lse holds the fp32 pair (LSE, scale) at [2R, 2R + 1];
 *   the scale is the row's largest |O| (0 for a row without a visible key), so every
 *   element is within scale * 2^-12 of the fp32 value.
 */
#ifndef SPLITKV_H
#define SPLITKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPLITKV_VERSION_MAJOR 0
#define SPLITKV_VERSION_MINOR 8

typedef enum {
  SPLITKV_OK = 0,
  SPLITKV_ERR_INVALID_ARG = -1, /* malformed problem, null pointer, bad stride or size   */
  SPLITKV_ERR_UNSUPPORTED = -2, /* valid but without a kernel (dtype/head_dim combination) */
  SPLITKV_ERR_WORKSPACE = -3,   /* workspace or plan buffer smaller than required         */
  SPLITKV_ERR_HIP = -4,         /* a HIP runtime call failed; text in splitkv_last_error  */
  SPLITKV_ERR_ALLOC = -5        /* host allocation failed                                 */
} splitkv_status;

typedef enum { SPLITKV_F32 = 0, SPLITKV_BF16 = 1 } splitkv_dtype;

/* What one LPT unit covers. The Split-KV page places "context KV blocks"; a block of
 * one KV head is the default unit (it serves g = Hq/Hkv query heads), a whole block
 * serving all Hq query heads is the coarser alternative. */
typedef enum { SPLITKV_UNIT_SEQ_BLOCK_KVHEAD = 0, SPLITKV_UNIT_SEQ_BLOCK = 1 } splitkv_granularity;

/* How the workgroups of a bf16 partial-attention launch take their jobs (a job is one
 * unit's KV head and up to 256 of its query rows; jobs are numbered in LPT order:
 * unit cost descending, ties in enumeration order).
 *   SPLITKV_SCHED_STATIC workgroup w runs the units the plan gave worker w, in order.
 *   SPLITKV_SCHED_QUEUE  workgroup w runs the plan's worker w units except the
 *                        cheapest ones at the end of the LPT order (about a fifth
 *                        of the estimated time, estimate = keys * max(rows, 128));
 *                        those form a shared tail, cut into chunks and dealt over 8
 *                        sub-queues, from which every workgroup draws (its own
 *                        sub-queue first) whenever it frees up: LPT's rule "next job
 *                        to the first free worker" applied at run time, so workgroups
 *                        that run faster (the CUs differ in memory bandwidth) take
 *                        more of the tail.
 *   SPLITKV_SCHED_AUTO   QUEUE when the plan has at least 16 jobs of fewer than 128
 *                        query rows per workgroup (otherwise one chunk is too large
 *                        a share to balance by), else STATIC.
 * Jobs of at least 128 query rows (8 row tiles) run in a launch of their own before
 * the others, statically: the jobs of each unit go to one XCD's workgroups (which
 * then share the block through L2) and, within it, each to the workgroup with the
 * least estimated time; the shared tail holds none of them.
 * All give bitwise identical results (a job's output does not depend on where it
 * runs). fp32 launches always use the static assignment. */
typedef enum { SPLITKV_SCHED_AUTO = 0, SPLITKV_SCHED_QUEUE = 1, SPLITKV_SCHED_STATIC = 2 } splitkv_schedule;

/* How the per-block partial outputs are stored in the workspace (layout above). The
 * row-scaled fp16 form halves the bytes the partials move (written by the partial
 * attention, read by the merge); bf16 inputs only. */
typedef enum { SPLITKV_PARTIAL_F32 = 0, SPLITKV_PARTIAL_F16_ROWSCALE = 1 } splitkv_partial_format;

/* Problem description. Host memory, caller-owned, read only during splitkv_plan. */
typedef struct {
  int32_t batch;            /* S >= 1 sequences                                      */
  const int64_t *kv_lens;   /* [S] context lengths n_s, n_s >= q_s                   */
  const int32_t *q_lens;    /* [S] trailing query counts q_s >= 1                    */
  int32_t num_q_heads;      /* Hq >= 1                                               */
  int32_t num_kv_heads;     /* Hkv >= 1, Hq % Hkv == 0                               */
  int32_t head_dim;         /* D; kernels exist for 64 and 128                      */
  int32_t block_len;        /* B >= 1 tokens per context KV block (last one ragged)  */
  int32_t num_workers;      /* m >= 1 LPT workers = workgroups of the attention launch */
  int32_t causal;           /* 1: bottom-right causal mask on the trailing queries   */
  int32_t granularity;      /* splitkv_granularity                                   */
  int32_t cost_ridge_rows;  /* R >= 0, the unit cost model (see splitkv_plan):          *
                             * 0 = the Split-KV page's q_s * len * heads;              *
                             * R > 0 = len * max(q_s * g, R) per KV head, i.e. a unit  *
                             * served by fewer than R query rows per KV head costs as  *
                             * streaming its block does (roofline-aware cost)          */
  const int32_t *xcd_speed; /* NULL, or [8] relative speeds (>= 1) of the GPU's 8 XCDs  *
                             * (workgroup w of a launch runs on XCD w % 8), e.g. from  *
                             * the worker_clock of a calibration launch: the plan's    *
                             * most loaded workers are then placed on workgroups of    *
                             * the fastest XCDs. The plan itself is unchanged.         */
  int32_t partial_format;   /* splitkv_partial_format; 0 (fp32 partials) is the only    *
                             * choice for fp32 inputs                                  */
} splitkv_problem;

typedef struct splitkv_plan_s splitkv_plan_t; /* opaque, library-owned host object */

typedef struct {
  int64_t num_units;      /* LPT units                                                 */
  int64_t total_cost;     /* sum of unit costs (the cost model of splitkv_problem)     */
  int64_t makespan;       /* largest worker load                                       */
  int64_t lower_bound;    /* max(ceil(total/m), largest unit cost)                     */
  double imbalance;       /* (m * makespan - total) / total, one float64 division      */
  int64_t total_q;        /* sum_s q_s                                                 */
  int64_t total_kv;       /* sum_s n_s                                                 */
  int64_t partial_rows;   /* workspace rows: sum_s nb_s * Hkv * q_s * g                */
  size_t plan_bytes;      /* device plan buffer size for splitkv_plan_upload           */
  size_t workspace_bytes; /* workspace size for partial_attn / merge / attn            */
  size_t ws_lse_offset;   /* byte offset of the partial LSEs inside the workspace      */
  /* How the bf16 partial-attention launch executes the plan. A job is one unit's KV
   * head and up to 256 of its query rows; the modelled imbalances below are
   * (m * max - total) / total over the launch's workgroups:                          */
  int64_t num_jobs;                 /* jobs of the bf16 kernel                          */
  double exec_imbalance_static;     /* SPLITKV_SCHED_STATIC lists as run (multi-job units *
                                     * dealt within XCD classes), under the page's cost   *
                                     * (a job's pass rows * block length)                 */
  double exec_imbalance_static_est; /* the same lists under the job-time estimate        *
                                     * len * max(rows, 128) (see splitkv_schedule)        */
  double exec_imbalance_queue_est;  /* SPLITKV_SCHED_QUEUE simulated with that estimate: *
                                     * each workgroup's list without the shared tail,     *
                                     * then the tail's chunks in order, each to the       *
                                     * workgroup with the least estimated time so far     */
  int32_t auto_schedule;            /* what SPLITKV_SCHED_AUTO runs: QUEUE or STATIC     */
  int64_t num_mma_jobs;             /* jobs of at least 128 query rows (8 row tiles),    *
                                     * run by a matrix-core kernel in a launch of their  *
                                     * own before the other jobs' launch                 */
  int32_t mma_partial_passes;       /* 1 when some such job covers fewer than 16 row    *
                                     * tiles: that launch then runs the kernel variant   *
                                     * whose waves may skip their second row tile; 0     *
                                     * when every such job covers 16 (or there is none)  */
  int32_t partial_format;           /* splitkv_partial_format of the plan               */
} splitkv_plan_info;

/* Device inputs. Pointers are device memory, caller-owned, read only. Strides are in
 * elements; the innermost (head_dim) stride is 1. Base pointers must be 16-byte
 * aligned and strides multiples of 16 bytes' worth of elements; with bf16 inputs
 * every stride must also be at most 2^24 elements (UNSUPPORTED otherwise). */
typedef struct {
  const void *q, *k, *v;
  int64_t q_stride_tok, q_stride_head;
  int64_t k_stride_tok, k_stride_head;
  int64_t v_stride_tok, v_stride_head;
  int32_t dtype;  /* splitkv_dtype, the same for q, k and v                          */
  float scale;    /* softmax scale; 0 selects 1/sqrt(head_dim)                       */
  int32_t schedule;           /* splitkv_schedule (bf16 launches)                    */
  uint64_t *worker_clock;     /* NULL, or device [2 * num_workers]: each workgroup of
                                 the partial-attention launch writes the GPU's
                                 constant 100 MHz clock when it starts and when it
                                 has finished its jobs (entries 2w and 2w + 1); the
                                 measured per-CU time imbalance comes from these.   */
} splitkv_inputs;

/* Version as (major << 16) | minor. */
int splitkv_version(void);

/* Build the LPT plan on the host (no HIP call). Split-KV page, "Timeline": context KV
 * blocks are allocated by a cost-aware LPT. Units are enumerated (seq, block, kv head)
 * lexicographically, stable sort by cost descending, each unit to the least-loaded
 * worker (ties to the lowest index). The cost of a unit serving heads query heads
 * (g per KV head, or Hq for a whole block) is, with R = cost_ridge_rows,
 *   R = 0:  q_s * len * heads                      (the page's cost: Lq x length x heads)
 *   R > 0:  len * max(q_s * g, R) * (heads / g)    (a block of one KV head is read in
 *           time ~ len and its q_s * g rows computed in time ~ len * rows / R, so R is
 *           the machine's ridge in query rows: its flop/byte ratio times the bytes per
 *           key over the flops per key and row; 312 for bf16 at MI355X's published
 *           peaks, about 128 for the attention kernels of this library as measured)
 * R = 0 and q_s * g >= R give the same cost. On success *out is a new plan the caller
 * releases with splitkv_plan_destroy.
 * Errors: INVALID_ARG (null pointers, S < 1, q_s < 1, n_s < q_s, Hq % Hkv != 0,
 * B < 1, m < 1, bad granularity, R < 0 or R > 2^30, total cost beyond 2^62), ALLOC. */
int splitkv_plan(const splitkv_problem *problem, splitkv_plan_t **out);

/* Plan statistics and buffer sizes. Errors: INVALID_ARG. */
int splitkv_plan_info_get(const splitkv_plan_t *plan, splitkv_plan_info *info);

/* Copy the plan out for inspection (host arrays, caller-owned; any may be NULL):
 * unit_seq/unit_block/unit_kv_head/unit_len/unit_cost [num_units] in enumeration
 * order (kv head -1 for whole-block units), worker_of [num_units],
 * worker_ptr [m + 1] and worker_units [num_units] (each worker's units in the order
 * it received them), load [m]. Errors: INVALID_ARG. */
int splitkv_plan_export(const splitkv_plan_t *plan, int32_t *unit_seq, int32_t *unit_block,
                        int32_t *unit_kv_head, int32_t *unit_len, int64_t *unit_cost,
                        int32_t *worker_of, int32_t *worker_ptr, int32_t *worker_units,
                        int64_t *load);

/* Copy the plan's device image (plan_bytes) to caller-owned device memory dev_plan
 * with an asynchronous host-to-device copy on hip_stream (NULL = default stream).
 * The plan must stay alive until that copy has completed. The image ends with a
 * 1024-byte scheduling area (the counters of the SPLITKV_SCHED_QUEUE tail): the
 * upload zeroes it, and every queue-scheduled launch updates it and leaves it zero
 * again, so launches that use one plan buffer must not overlap in time (use one
 * stream per plan buffer).
 * Errors: INVALID_ARG, WORKSPACE (bytes < plan_bytes), HIP. */
int splitkv_plan_upload(const splitkv_plan_t *plan, void *dev_plan, size_t bytes, void *hip_stream);

/* Release a plan (NULL is ignored). */
void splitkv_plan_destroy(splitkv_plan_t *plan);

/* Partial attention of every unit: for each context KV block and KV head, the output
 * and log-sum-exp of the queries against that block alone (the query-sized per-block
 * result of the Split-KV page's lede). One workgroup per LPT worker; in->schedule
 * says how the workgroups take the jobs. Writes the whole workspace (layout above);
 * every row is written, rows that see no key of a block get O = 0 and LSE = -inf.
 * dev_plan is the uploaded plan; the launch also uses its scheduling area.
 * Errors: INVALID_ARG (null/misaligned pointers, strides), UNSUPPORTED (no kernel for
 * dtype/head_dim, bf16 stride above 2^24, fp32 inputs on a plan with fp16 partials),
 * WORKSPACE (ws_bytes < workspace_bytes), HIP (launch failed). */
int splitkv_partial_attn(const splitkv_plan_t *plan, void *dev_plan, const splitkv_inputs *in,
                         float *ws, size_t ws_bytes, void *hip_stream);

/* Log-sum-exp merge of the partials in the workspace into out [sum q, Hq, D] and
 * lse [sum q, Hq] (fp32). Blocks are combined in block order, so the result does not
 * depend on the plan's worker count. The Split-KV page ("Timeline") states that the
 * method is exact: this merge reproduces unsharded attention up to rounding.
 * Errors: INVALID_ARG, WORKSPACE, HIP. */
int splitkv_merge(const splitkv_plan_t *plan, const void *dev_plan, const float *ws, size_t ws_bytes,
                  float *out, float *lse, void *hip_stream);

/* Fused call: partial attention and merge enqueued back to back on hip_stream, with
 * sequences of a single block written straight to out/lse. Same arguments and errors
 * as the two calls above. Its output is the bits of the two calls' output, except that
 * under SPLITKV_PARTIAL_F16_ROWSCALE the rows of single-block sequences skip the fp16
 * rounding of the stored partial (the two then differ by at most the bound above). */
int splitkv_attn(const splitkv_plan_t *plan, void *dev_plan, const splitkv_inputs *in,
                 float *ws, size_t ws_bytes, float *out, float *lse, void *hip_stream);

/* splitkv_attn without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The partials go to a workspace the library holds itself: one array of
 * SPLITKV_SCRATCH_BYTES (256 MiB) per GPU, in device memory from the library's load
 * until the process ends. This call allocates nothing (no hipMalloc, no hipFree, no
 * allocating library routine); the first call on a device looks up that device's
 * copy of the array. Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams, or different threads without
 * ordering) race and give wrong results; calls ordered on one stream are safe. Every
 * workspace row a call reads is written earlier in the same call, so nothing needs
 * clearing between calls. Same arguments and results as splitkv_attn otherwise.
 * Errors: as splitkv_attn; WORKSPACE when the plan's workspace_bytes exceeds
 * SPLITKV_SCRATCH_BYTES (use splitkv_attn with a caller workspace then), reported
 * before any HIP call; HIP when the array's address cannot be looked up. */
#define SPLITKV_SCRATCH_BYTES ((size_t)256 << 20)
int splitkv_attn_scratch(const splitkv_plan_t *plan, void *dev_plan, const splitkv_inputs *in,
                         float *out, float *lse, void *hip_stream);

/* Inputs of the backward pass besides Q, K and V (device memory, caller-owned). */
typedef struct {
  const void *d_out;                     /* upstream gradient dO [sum q, Hq, D], the dtype of q */
  int64_t do_stride_tok, do_stride_head; /* its strides in elements (multiples of 16 bytes)     */
  const float *out;                      /* the forward's O [sum q, Hq, D], contiguous          */
  const float *lse;                      /* the forward's LSE [sum q, Hq] (natural log)          */
  float *dq;                             /* written: dQ [sum q, Hq, D] fp32, contiguous          */
  void *dk;                              /* written: dK [sum n, Hkv, D], contiguous, dkv_dtype   */
  void *dv;                              /* written: dV [sum n, Hkv, D], contiguous, dkv_dtype   */
  int32_t dkv_dtype;                     /* splitkv_dtype of dK and dV: SPLITKV_F32 (0) or       *
                                          * SPLITKV_BF16 (1, each value rounded to nearest even  *
                                          * from the fp32 sum; half the bytes written)           */
} splitkv_grads;

/* Backward pass of split-KV attention: dQ, dK, dV of sum(dO * O) with respect to Q, K
 * and V, taken at the forward's O and LSE (from splitkv_attn on the same plan and
 * inputs). Split-KV page, "Timeline": the sharded computation is exact; with the
 * merged LSE every KV block's share of the gradients is exact on its own: a block's
 * keys get their dK and dV from that block alone, and each query row's dQ is the sum
 * of one query-sized part per block, summed here in block order (the same exchange
 * as the forward's merge, with a plain sum). Textbook gradients:
 *   D_i = <dO_i, O_i>, P = e^(scale q.k - LSE), dS = P (dO.v - D),
 *   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO,
 * with dK and dV summed over the query heads of each KV head. bf16 inputs only;
 * every sum is fp32; dQ is stored as fp32, dK and dV as grads->dkv_dtype. The workspace (splitkv_plan_info.workspace_bytes) holds the dQ parts,
 * D and the LSE in base 2. The fields schedule and worker_clock of in are not used.
 * Errors: INVALID_ARG (NULL or misaligned pointers, bad strides, dkv_dtype not a
 * splitkv_dtype), UNSUPPORTED (fp32 inputs, head_dim other than 64 or 128, bf16 strides
 * beyond 2^24), WORKSPACE, HIP. */
int splitkv_attn_backward(const splitkv_plan_t *plan, const void *dev_plan, const splitkv_inputs *in,
                          const splitkv_grads *grads, float *ws, size_t ws_bytes, void *hip_stream);

/* Static text for a status code. */
const char *splitkv_status_string(int status);

/* Detail text of the last error on the calling thread ("" if none). */
const char *splitkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPLITKV_H */
