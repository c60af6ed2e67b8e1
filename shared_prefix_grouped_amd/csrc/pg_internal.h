// Internal declarations shared by the host API and the HIP kernel files of
// libpg_attn.  Not part of the public C ABI (that is include/pg_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pg_attn.h"

namespace pg {

// Everything a kernel launch needs from the descriptor, by value.
struct Plan {
  int T, Hq, Hkv, D;
  int n_q_tiles, n_kv_tiles;
  int n_kv_items, n_kv_sums, n_kv_parts;
  const int32_t *row_lo, *row_hi;
  const int32_t *q_tiles, *kv_tiles;
  const int32_t *kv_items, *kv_sums;
  int n_groups;
  const int32_t *group_start, *prefix_end, *prefix_before;
};

// log2(e): scores are kept in the base-2 domain inside the kernels so that the
// exponential is a single v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Keys per K/V chunk of the bf16 forward and dQ kernels: a work item streams
// its key segments through LDS in chunks of this many rows, one barrier step
// each, so its run time follows its chunk count (the planner orders the query
// tiles by it).
constexpr int kKvChunk = 64;

// Forward (writes o and lse for every row and query head).
hipError_t launch_fwd_bf16(const Plan &p, float scale, const void *q, const void *k,
                           const void *v, void *o, float *lse, hipStream_t s);
hipError_t launch_fwd_f32(const Plan &p, float scale, const void *q, const void *k,
                          const void *v, void *o, float *lse, hipStream_t s);

// bf16 dK, dV (key-stationary) and dQ (query-stationary); no atomics.  `lse`
// passed to dK/dV is the base-2 logsumexp written, with delta, by the dQ
// kernel, which takes the forward's natural-log LSE.  The
// bf16 dK/dV launch walks the plan's kv_items; `partial` holds n_kv_parts
// float slots of [Hkv][2][PG_TILE_KV][D] for the pieces of split key tiles.
hipError_t launch_bwd_dkdv_bf16(const Plan &p, float scale, const void *q, const void *k,
                                const void *v, const float *lse, const float *delta,
                                const void *dout, void *dk, void *dv, float *partial,
                                hipStream_t s);
hipError_t launch_bwd_dq_bf16(const Plan &p, float scale, const void *q, const void *k,
                              const void *v, const void *o, const float *lse, float *lse2,
                              float *delta, const void *dout, void *dq, hipStream_t s);
// Float32 backward: one launch of dK/dV and dQ workgroups, which compute
// delta and the base-2 logsumexp themselves from O, dO and the forward's
// natural-log `lse`.
hipError_t launch_bwd_f32(const Plan &p, float scale, const void *q, const void *k,
                          const void *v, const void *o, const float *lse, const void *dout,
                          void *dq, void *dk, void *dv, hipStream_t s);

// Plan upload: `bytes` (a multiple of 16) from src_dev to dst and npos int32
// position ids from pos_src_dev to pos_dst, where the sources are device
// addresses of pinned host memory; a kernel on stream s.
hipError_t launch_upload(const void *src_dev, void *dst, size_t bytes, const void *pos_src_dev,
                         int32_t *pos_dst, size_t npos, hipStream_t s);

// Row gather (pack: the caller's prefix / response row buffers -> packed
// rows) or scatter (unpack), row_bytes a multiple of 4.
hipError_t launch_rows(const Plan &p, bool pack, void *packed, void *pre, void *resp,
                       size_t row_bytes, hipStream_t s);

// Log-probability head kernels: the logits products and the backward's two
// products run on this library's MFMA tile kernel (pg_head_mfma.hip).
inline int round8(int x) { return (x + 7) & ~7; }
// row stride of the head's transposed and gradient operands: whole 128-byte
// cache lines per row (a stride that is not a multiple of 128 bytes makes
// every 128-byte copy chunk straddle two lines)
inline int round64(int x) { return (x + 63) & ~63; }
hipError_t launch_gather_rows(const int32_t *pred, const void *hidden, void *out, int n,
                              int d_model, hipStream_t s);
// number of 256-entry vocab tiles (rows of the per-tile max / sum arrays)
int head_vocab_tiles(int V);
// logp and lse of the n scored rows; part_m / part_s: [head_vocab_tiles(V), n]
// floats of scratch
hipError_t launch_head_logprob(const void *hp, const void *w, const int32_t *scored_row,
                               const int32_t *tokens, float *part_m, float *part_s, float *logp,
                               float *lse, int n, int V, int dm, hipStream_t s);
// the gradient of the loss with respect to the logits, bf16, as G [n, round64(V)]
// and G^T [V, round64(n)] (pad entries zero)
hipError_t launch_head_grad(const void *hp, const void *w, const int32_t *scored_row,
                            const int32_t *tokens, const float *lse, const float *dlogp, void *g,
                            void *gt, int n, int V, int dm, hipStream_t s);
// c [M, ldc] fp32 = a [M, K] b [N, K]^T for bf16 a, b (row strides lda, ldb,
// multiples of 8; K a multiple of 8; M lda 2 and N ldb 2 under 2^32)
hipError_t launch_nt_f32(const void *a, const void *b, int M, int N, int K, int lda, int ldb,
                         float *c, int ldc, hipStream_t s);
// dst [C, ldd] bf16: dst[c][r] = src[rows ? rows[r] : r][c] for r < R, zero
// for R <= r < ldd (ldd even, C a multiple of 8)
hipError_t launch_transpose_pad(const void *src, const int32_t *rows, int R, int C, void *dst,
                                int ldd, hipStream_t s);
hipError_t launch_grpo_loss(const float *logp, const int32_t *scored_resp, const float *adv,
                            float *loss, float *dlogp, int n, int n_resp, hipStream_t s);
hipError_t launch_scatter_rows(const int32_t *pred_start, const int32_t *pred_list,
                               const float *dh_pred, float *dhidden, int T, int d_model,
                               hipStream_t s);

// Rotary embedding in place.
hipError_t launch_rope(int T, int H, int D, pg_dtype t, void *x, const int32_t *pos,
                       float theta, int inverse, hipStream_t s);

}  // namespace pg
