/*
 * pg_attn.h -- C ABI of the grouped shared-prefix attention library (libpg_attn.so).
 *
 * The operation (web pages on "Prefix Grouper: Efficient GRPO Training through
 * Shared-Prefix Forward"; the Pith review on pith.science, sections "What
 * carries the argument" and "Core claim"; the skillsmp.com page
 * "prefix-grouper-grpo", sections "Core Concept" and "Step 3: Restructure
 * Input Format"):
 *
 *   A group is one shared prefix P followed by G responses, packed as the rows
 *   [P; R_1; ...; R_G]; a batch packs groups one after another, without padding.
 *   Attention is split in two: causal self-attention over the prefix rows,
 *   computed once per group, and a suffix pass in which the queries of
 *   response i attend to every prefix key and to the keys of response i up to
 *   themselves, never to another response.  Every row therefore sees exactly
 *   the causal context it has in the repeated-prefix baseline [P; R_i], and
 *   the outputs and gradients equal the baseline's; the gradient of a shared
 *   prefix row is the sum of the gradients of its G copies (Lemma 2.1).
 *
 *   Equivalently, with packed row indices, query row q of a group starting at
 *   row g0 with prefix end row pe sees key row k iff
 *       g0 <= k <= q  and  (k < pe  or  k >= start of q's response).
 *
 * Conventions
 *   - Rows: T packed rows.  Q, O, dQ, dO are [T, Hq, d]; K, V, dK, dV are
 *     [T, Hkv, d]; row-major, d contiguous, no padding between rows or heads.
 *   - LSE is float [Hq, T]: natural-log logsumexp of the scaled scores of
 *     each (head, row).
 *   - Grouped-query attention: query head h uses key/value head
 *     h / (Hq / Hkv).  Hq must be a multiple of Hkv.
 *   - Element type: PG_BF16 (bfloat16 storage, float32 accumulation) or
 *     PG_F32 (float32 throughout).  Outputs are in the input type, rounded to
 *     nearest even from float32.  head_dim 64 or 128.
 *   - Device pointers must be 16-byte aligned.  All tensors, descriptors and
 *     workspaces are allocated and owned by the caller.
 *   - State the library itself holds, per process, until it ends (nothing is
 *     freed): (1) pg_pack's pinned, device-mapped host staging buffers, at
 *     most 64, reused once the upload kernel that reads them has run; (2)
 *     pg_attn_bwd_noalloc's device scratch array, PG_NOALLOC_SCRATCH_BYTES per
 *     device, placed by the HIP runtime when the library's code objects are
 *     loaded on that device; (3) the kernel timing table and its event pool
 *     (pg_kernel_timing); (4) the thread-local message of pg_last_error.
 *     None of it carries results from one call to the next.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Kernels are
 *     enqueued on it; the call returns before they finish.
 *   - Results are bitwise reproducible for the same inputs, descriptor and
 *     device: no floating-point atomics, every reduction has a fixed order.
 *
 * Errors
 *   Every call validates its arguments on the host before enqueuing anything
 *   and returns a pg_status.  PG_ERR_INVALID_ARG: bad lengths, null or
 *   misaligned pointers, inconsistent descriptor.  PG_ERR_UNSUPPORTED: a
 *   head_dim or dtype the kernels do not implement.  PG_ERR_WORKSPACE: a
 *   buffer smaller than the size function reports.  PG_ERR_HIP: a HIP runtime
 *   call or a launch failed.  pg_last_error() returns a message for the last
 *   non-OK status of the calling thread.  Faults inside kernels surface at the
 *   caller's next synchronisation.  No call aborts the process and no C++
 *   exception crosses this interface.
 */
#ifndef PG_ATTN_H
#define PG_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PG_OK = 0,
  PG_ERR_INVALID_ARG = 1,
  PG_ERR_UNSUPPORTED = 2,
  PG_ERR_WORKSPACE = 3,
  PG_ERR_HIP = 4
} pg_status;

typedef enum { PG_F32 = 0, PG_BF16 = 1 } pg_dtype;

/* Row tiles of the work lists built by pg_pack (fixed by the library build). */
#define PG_TILE_Q 128  /* query rows per forward / dQ work item */
#define PG_TILE_KV 128 /* key rows per dK/dV work item */

/* Host description of a packed batch (input of pg_pack).  All arrays are
 * host memory, read during the call only.
 *   num_groups  >= 0
 *   prefix_len  [num_groups], each >= 0
 *   num_resp    [num_groups], each >= 1 (G of the group)
 *   resp_len    [sum(num_resp)], each >= 0, group-major (group 0's responses
 *               first, in packed order)
 * The total row count T = sum(prefix_len) + sum(resp_len) must fit int32. */
typedef struct {
  int32_t num_groups;
  const int32_t *prefix_len;
  const int32_t *num_resp;
  const int32_t *resp_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
} pg_groups;

/* Descriptor filled by pg_pack.  The pointer members address the caller's
 * buffer passed to pg_pack (device memory for pg_pack, host memory for
 * pg_pack_host) and stay valid as long as that buffer does.  Callers treat it
 * as read-only; it is reused unchanged by pg_attn_fwd, pg_attn_bwd and
 * pg_rope for every layer of the same batch.
 *   row_lo[T]    first key row of the row's own segment: the group's first
 *                row for a prefix row, the response's first row for a
 *                response row.  A query row q sees key rows
 *                [group start, min(prefix end, q + 1)) and [row_lo[q], q].
 *   row_hi[T]    one past the last query row that sees key row k: the group's
 *                end for a prefix row, the response's end for a response row.
 *                Key row k is seen by exactly the query rows [k, row_hi[k]).
 *   q_tiles      [num_q_tiles][4] = {q0, q1, group start, prefix end}: query
 *                rows [q0, q1) of one group, q1 - q0 <= PG_TILE_Q, ordered by
 *                decreasing run time: the key chunks a forward / dQ work item
 *                streams (64 rows each: the prefix keys up to q1, then the
 *                keys from the response start of row q0), then the visible
 *                (query, key) pairs.
 *   kv_tiles     [num_kv_tiles][4] = {k0, k1, q_end, prefix end}: key rows
 *                [k0, k1) of one group, k1 - k0 <= PG_TILE_KV, seen by query
 *                rows inside [k0, q_end), ordered by decreasing cost.
 *   kv_items     [num_kv_items][8] = {k0, k1, qa, qb, part, 0, 0, 0}: the bf16
 *                dK/dV work list, ordered by decreasing cost.  Key tile
 *                [k0, k1) against query rows [qa, qb).  part < 0: the whole
 *                tile (qa = k0, qb = q_end).  part >= 0: one piece of a tile
 *                whose walk was cut at 32-row query blocks (qa - k0 a multiple
 *                of 32), because it alone held more than the mean work per
 *                compute unit -- the prefix tiles of a group with a short
 *                prefix and many responses; its float partial dK/dV goes to
 *                workspace slot `part`.
 *   kv_sums      [num_kv_sums][4] = {k0, k1, first part, number of parts}:
 *                the cut tiles; their parts are consecutive and are added in
 *                part order, so the result does not depend on scheduling.
 *                num_kv_parts = total number of parts.
 *   group_start  [num_groups + 1], prefix_end [num_groups],
 *   resp_start   [num_resp], resp_len [num_resp], resp_group [num_resp]:
 *                the packed offsets, for callers.
 *   prefix_before [num_groups + 1]: prefix rows of the groups before g
 *                (prefix_before[num_groups] = total_prefix_rows), the
 *                offsets of pg_pack_rows' prefix buffer.
 *   scored_row, scored_pred, scored_resp [num_scored]: the response rows
 *                whose token the log-probability head scores, in packed
 *                order; the row whose logits score it (the previous position
 *                of its baseline sequence [P; R_i]: the previous response row,
 *                or for a response's first token the group's last prefix row,
 *                shared by all G responses); and its response index.  The
 *                first token of a response of an empty-prefix group has no
 *                predicting position and is not scored.
 *   pred_start [T + 1], pred_list [num_scored]: for packed row t, the
 *                scored entries it predicts are pred_list[pred_start[t] ..
 *                pred_start[t + 1]), in increasing order.
 *   max_walk_rows   the longest query-row range [qa, qb) of a kv_items
 *                   entry (bounded by the largest group);
 *   pairs           unmasked (query, key) pairs per query head;
 *   baseline_pairs  the same count for the repeated-prefix layout (each
 *                   [P; R_i] on its own). */
typedef struct {
  int32_t num_groups, num_resp, total_rows;
  int32_t num_q_heads, num_kv_heads, head_dim;
  int32_t num_q_tiles, num_kv_tiles;
  int32_t num_kv_items, num_kv_sums, num_kv_parts;
  int32_t total_prefix_rows;
  int32_t num_scored;
  int32_t max_walk_rows;
  int64_t pairs, baseline_pairs;
  const int32_t *row_lo;
  const int32_t *row_hi;
  const int32_t *q_tiles;
  const int32_t *kv_tiles;
  const int32_t *kv_items;
  const int32_t *kv_sums;
  const int32_t *group_start;
  const int32_t *prefix_end;
  const int32_t *prefix_before;
  const int32_t *resp_start;
  const int32_t *resp_len;
  const int32_t *resp_group;
  const int32_t *scored_row;
  const int32_t *scored_pred;
  const int32_t *scored_resp;
  const int32_t *pred_start;
  const int32_t *pred_list;
  size_t buf_bytes; /* bytes of the buffer actually used */
} pg_desc;

/* Bytes pg_pack needs in its device buffer for this batch; 0 if the
 * description is invalid (then pg_last_error() says why). */
size_t pg_pack_buffer_size(const pg_groups *g);

/* Plan a packed batch: validate the lengths, build row_lo/row_hi, the tile
 * work lists and the offsets, and copy them to the device buffer `d_buf`
 * (>= pg_pack_buffer_size bytes, 16-byte aligned).  If `d_pos_ids` is not
 * NULL it receives int32 [T] position ids as in the repeated-prefix baseline:
 * prefix row t of a group -> t, row j of a response -> P + j (Pith review,
 * "What carries the argument").  The plan is written into a pinned,
 * device-mapped host buffer that the library owns (reused once its copy has
 * run, kept until the process ends) and copied into d_buf by a kernel enqueued
 * on `stream`, so the call does not wait for the GPU; the caller's host arrays
 * may be freed when it returns.  d_buf and d_pos_ids
 * hold the plan for work ordered after the call on `stream` (other streams
 * must wait for it).  Fills *out. */
pg_status pg_pack(const pg_groups *g, void *d_buf, size_t buf_bytes, int32_t *d_pos_ids,
                  pg_desc *out, void *stream);

/* Same plan as pg_pack, written to host memory (no GPU involved); the
 * pointers in *out address `h_buf`.  For inspection and tests. */
pg_status pg_pack_host(const pg_groups *g, void *h_buf, size_t buf_bytes, int32_t *h_pos_ids,
                       pg_desc *out);

/* Gather per-row data into the packed layout: the shared prefix of each group
 * once, then its responses back to back (skillsmp.com "prefix-grouper-grpo",
 * "Step 3: Restructure Input Format", without the padding rows).  prefix_rows
 * holds the groups' prefix rows one group after another [total_prefix_rows],
 * resp_rows every response's rows in pg_groups order [T - total_prefix_rows],
 * packed_rows receives [T]; each row is row_bytes bytes (a positive multiple
 * of 4; 16-byte chunks and 16-byte aligned pointers when it is a multiple of
 * 16, else 4-byte).  Token ids, hidden states or any [T, ...] tensor of the
 * batch.  Device buffers, caller-owned, not overlapping; a buffer with no
 * rows may be NULL.  Enqueued on `stream`; one kernel reading and writing
 * each byte once. */
pg_status pg_pack_rows(const pg_desc *d, const void *prefix_rows, const void *resp_rows,
                       void *packed_rows, size_t row_bytes, void *stream);

/* The inverse scatter: packed rows back to the prefix and response buffers
 * (same layouts and rules as pg_pack_rows), e.g. to read the response rows of
 * an output or a gradient per response. */
pg_status pg_unpack_rows(const pg_desc *d, const void *packed_rows, void *prefix_rows,
                         void *resp_rows, size_t row_bytes, void *stream);

/* Forward: O = grouped attention(Q, K, V) and LSE, for every packed row and
 * query head.  softmax_scale <= 0 selects 1/sqrt(head_dim).  Prefix rows are
 * computed once per group (prefix-only causal attention); response rows
 * attend to the prefix and their own response (Pith review, "What carries the
 * argument").  q, k, v: input, o: output [T,Hq,d], lse: output float [Hq,T]
 * (natural log), or NULL when no backward follows -- forward-only scoring of
 * many short responses against one shared context, the other shared-prefix
 * use the pages name (Pith review, "Editorial extensions"); O is then
 * bitwise the same. */
pg_status pg_attn_fwd(const pg_desc *d, pg_dtype t, float softmax_scale, const void *q,
                      const void *k, const void *v, void *o, float *lse, void *stream);

/* Bytes of scratch pg_attn_bwd needs.  PG_BF16: two float [Hq, T] arrays,
 * rowsum(dO * O) and the logsumexp in base 2, each 16-byte aligned, and the
 * partial dK/dV sums of the cut key tiles, float
 * [num_kv_parts][num_kv_heads][2][PG_TILE_KV][head_dim].  PG_F32: 16 (its
 * one backward launch computes both row statistics where it uses them and
 * sums its partial results on chip). */
size_t pg_attn_bwd_workspace_size(const pg_desc *d, pg_dtype t);

/* Backward: gradients of sum(O * dO) with respect to Q, K, V, recomputing the
 * softmax from the saved LSE.  dK and dV of a prefix row are summed over the
 * query rows of the prefix and of all G responses of its group and over the
 * query heads sharing its key/value head, in a fixed order (Pith review,
 * "Core claim", Lemma 2.1).  Inputs q, k, v, o, lse, dout as produced by /
 * given to pg_attn_fwd; outputs dq [T,Hq,d], dk, dv [T,Hkv,d] are fully
 * overwritten.  `workspace` is device scratch of at least
 * pg_attn_bwd_workspace_size bytes (contents need not be initialised).
 * PG_BF16 needs (max_walk_rows + 32) * Hq * d * 2 < 2^32 (the query rows one
 * dK/dV work item walks, at most one group's, under 4 GiB of q: the kernel
 * bases its buffer descriptors at the item's first query row and addresses
 * the rest with 32-bit unsigned offsets) and Hq * T * 4 < 2^31 (the float
 * [Hq, T] arrays it reads), else PG_ERR_UNSUPPORTED.  q and dout themselves
 * may exceed 4 GiB. */
pg_status pg_attn_bwd(const pg_desc *d, pg_dtype t, float softmax_scale, const void *q,
                      const void *k, const void *v, const void *o, const float *lse,
                      const void *dout, void *dq, void *dk, void *dv, void *workspace,
                      size_t ws_bytes, void *stream);

/* Bytes of device scratch the library keeps per GPU for pg_attn_bwd_noalloc. */
#define PG_NOALLOC_SCRATCH_BYTES (64u << 20)

/* pg_attn_bwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight training or serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (minus the workspace), same kernels and bitwise the same results
 * as pg_attn_bwd.  The scratch pg_attn_bwd_workspace_size reports lives in a
 * device array of PG_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends (its address is looked up on the
 * first call on each device); a batch needing more returns PG_ERR_WORKSPACE
 * before anything is enqueued.  The call enqueues only kernel launches: no
 * hipMalloc, hipFree or allocating library routine, and no timing events
 * (pg_kernel_timing does not cover it).  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents; each call writes every
 * scratch value it reads first, so nothing needs clearing.  Calls that
 * overlap on one GPU (concurrent streams, or host threads without ordering)
 * race on the array: order them on one stream. */
pg_status pg_attn_bwd_noalloc(const pg_desc *d, pg_dtype t, float softmax_scale, const void *q,
                              const void *k, const void *v, const void *o, const float *lse,
                              const void *dout, void *dq, void *dk, void *dv, void *stream);

/* Rotary position embedding at the baseline position ids, in place on x
 * [T, num_heads, head_dim] (PG_BF16 or PG_F32, rotate-half pairing: element i
 * with element i + d/2, angle pos * theta^(-2i/d)), computed in float32.
 * pos_ids: int32 [T] from pg_pack.  inverse != 0 applies the transposed
 * rotation (the backward of the forward rotation).  Response row j of a group
 * is rotated as position P + j, so relative offsets match the baseline [P; R_i]
 * (Pith review, "What carries the argument" and "Load-bearing premise"). */
pg_status pg_rope(const pg_desc *d, pg_dtype t, void *x, int32_t num_heads, int32_t head_dim,
                  const int32_t *pos_ids, float theta, int32_t inverse, void *stream);

/* ---- Response log-probability head of the GRPO step (skillsmp.com
 * "prefix-grouper-grpo", "Step 4: Training Integration with GRPO"): the
 * log-softmax of the logits over the vocabulary, gathered at each response
 * token, summed per response, and the policy loss -mean_i(A_i * sum_i).
 * Only scored rows are computed (pg_desc's scored_row / scored_pred: the
 * logits of the row before each response token in its baseline sequence
 * [P; R_i]; a response's first token is scored by the group's last prefix
 * row).  Logits are hidden @ weight^T (LM head without bias), bf16 operands,
 * fp32 accumulation.  The logits are computed in this library's MFMA tile
 * kernels and reduced in place (forward: per-row max and sum of exponentials
 * per 256-entry vocab tile, and the target logit as one dot product;
 * backward: the gradient of the logits, stored as bf16), so they are never
 * written to memory; the backward's two products dH = G weight and dW = G^T H
 * run on the same tile kernel, from G and G^T and transposed copies of weight
 * and H.
 * hidden: bf16 [T, d_model] in packed order; weight: bf16 [vocab, d_model]
 * (under 4 GiB, as are the num_scored gathered hidden rows: larger heads
 * return PG_ERR_UNSUPPORTED); tokens: int32 [T] token id of every packed row
 * (read only at scored rows; an id outside [0, vocab) gives logp = NaN).
 * d_model a multiple of 8.  Device buffers, 16-byte aligned, caller-owned. */

/* Bytes of scratch pg_logprob_fwd / pg_logprob_bwd need: the gradient of the
 * logits as bf16 [num_scored, V64] and [vocab, n64] (V64, n64: vocab and
 * num_scored rounded up to multiples of 64), the gathered predicting rows
 * (bf16 [num_scored, d_model]) and their transpose (bf16 [d_model, n64]), the
 * transposed weight (bf16 [d_model, V64]), the predicting rows' gradient (fp32
 * [num_scored, d_model]), and the forward's per-tile row max and sum (fp32
 * [ceil(vocab / 256), num_scored] each), each 256-byte aligned.  0 if the
 * arguments are invalid. */
size_t pg_logprob_workspace_size(const pg_desc *d, int32_t vocab, int32_t d_model);

/* logp [num_scored]: log-probability of each scored token; lse
 * [num_scored]: logsumexp of its logits (kept for the backward). */
pg_status pg_logprob_fwd(const pg_desc *d, const void *hidden, const void *weight, int32_t vocab,
                         int32_t d_model, const int32_t *tokens, float *logp, float *lse,
                         void *workspace, size_t ws_bytes, void *stream);

/* Policy loss from the log-probabilities and one advantage per response
 * (float [num_resp], treated as a constant): loss[0] = -mean_i(A_i * S_i)
 * with S_i the sum of response i's logp, and dlogp [num_scored] =
 * d loss / d logp = -A_i / num_resp.  One workgroup, fixed order. */
pg_status pg_grpo_loss(const pg_desc *d, const float *logp, const float *advantages, float *loss,
                       float *dlogp, void *stream);

/* Backward of sum_k dlogp[k] * logp[k]: dhidden fp32 [T, d_model] (every row
 * written: zero for rows that score nothing; a group's last prefix row sums
 * the first tokens of its G responses, in response order) and dweight fp32
 * [vocab, d_model].  Recomputes the logits (same workspace size as the
 * forward; contents need not be kept between the calls). */
pg_status pg_logprob_bwd(const pg_desc *d, const void *hidden, const void *weight, int32_t vocab,
                         int32_t d_model, const int32_t *tokens, const float *lse,
                         const float *dlogp, float *dhidden, float *dweight, void *workspace,
                         size_t ws_bytes, void *stream);

/* Kernel timing for benchmarks.  While enabled, every kernel the library
 * launches is bracketed by two HIP events recorded on the stream it is
 * launched on.  pg_kernel_timing(1) clears the counters and enables,
 * pg_kernel_timing(0) disables.  pg_kernel_times waits for the recorded events
 * and returns the number of launches and their total duration in milliseconds
 * for one kernel id (PG_KERNEL_*); it fails with PG_ERR_INVALID_ARG for an
 * unknown id.  A HIP error met while folding the events of earlier launches
 * (an earlier kernel's fault, for instance) is returned as PG_ERR_HIP by the
 * next pg_kernel_timing or pg_kernel_times call, not by the launching call.
 * pg_kernel_name returns the kernel's name, or NULL.  Not
 * thread-safe with respect to concurrent enabling/reading.  The PG_F32
 * backward is one launch doing both the dK/dV and the dQ work, counted under
 * PG_KERNEL_BWD_DKDV; PG_KERNEL_BWD_PRE counts nothing (both backward paths
 * compute their row statistics inside their own kernels; the id keeps the
 * numbering). */
#define PG_KERNEL_FWD 0
#define PG_KERNEL_BWD_PRE 1
#define PG_KERNEL_BWD_DKDV 2
#define PG_KERNEL_BWD_DQ 3
#define PG_KERNEL_ROPE 4
#define PG_KERNEL_ROWS 5
#define PG_KERNEL_HEAD_FWD 6
#define PG_KERNEL_HEAD_BWD 7
#define PG_KERNEL_LOSS 8
#define PG_KERNEL_COUNT 9
pg_status pg_kernel_timing(int32_t enable);
pg_status pg_kernel_times(int32_t kernel_id, int64_t *launches, double *total_ms);
const char *pg_kernel_name(int32_t kernel_id);

/* Message for the last non-OK status returned on the calling thread. */
const char *pg_last_error(void);

/* Library version string. */
const char *pg_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PG_ATTN_H */
