// Grouped shared-prefix attention, forward, bf16 storage / fp32 accumulation,
// for gfx950 (CDNA4, wave64, v_mfma_f32_32x32x16_bf16).
//
// One launch covers both parts of the method's attention (Pith review of
// Prefix Grouper, "What carries the argument"):
//   * prefix rows: causal self-attention over the prefix only, once per group;
//   * response rows: a two-segment pass over (A) every prefix key, with no
//     mask, then (B) the keys of the row's own response up to itself.
// A work item is up to 128 consecutive packed rows of one group and one query
// head.  Rows of several responses may share a work item: segment A is the
// same prefix K/V for all of them, so each prefix K/V chunk is staged through
// LDS once and consumed by every response row of the item; segment B is masked
// per row with the row's own response start (row_lo).  Both segments feed one
// online softmax per row.
//
// Wave layout: 4 waves x 32 query rows.  Each wave computes S^T = K Q^T for a
// 64-key chunk (A = K rows from LDS, B = the wave's Q rows held in registers),
// so lane l owns query row l % 32 and its softmax statistics are per-lane
// scalars; P^T then feeds O^T += V^T P^T directly from the accumulator
// registers, with V read transposed from row-major LDS (ds_read_b64_tr_b16).

#include "pg_device.h"
#include "pg_internal.h"

namespace pg {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int BM = PG_TILE_Q;  // query rows per workgroup
  static constexpr int NW = BM / 32;    // waves
  static constexpr int NT = NW * 64;    // threads
  static constexpr int BN = kKvChunk;   // keys per chunk
  static constexpr int NB = BN / 32;    // 32-key MFMA blocks per chunk
  static constexpr int OCC = 2;         // workgroups per CU (LDS: 4 * BN * D * 2 bytes each)
};

// A row keeps a stale running max until a chunk raises it by more than
// kRescale (base-2 units): probabilities then stay below 2^kRescale, and the
// O rescale runs only when some lane of the wave needs it, which after the
// first chunks is rare.
constexpr float kRescale = 8.0f;

template <int D>
__global__ __launch_bounds__(256, FwdCfg<D>::OCC) void fwd_bf16_kernel(
    const int32_t *__restrict__ q_tiles, const int32_t *__restrict__ row_lo,
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    bf16 *__restrict__ O, float *__restrict__ LSE, int T, int Hq, int Hkv, float scale_log2) {
  using C = FwdCfg<D>;
  // K and V chunks, double-buffered, row-major and swizzled (see swz): K is
  // read as MFMA rows, V transposed.
  __shared__ __attribute__((aligned(16))) bf16 sK[2 * C::BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV[2 * C::BN * D];

  int tile, h;
  xcd_qhead_work(blockIdx.x, Hq, Hkv, tile, h);
  const int hk = h / (Hq / Hkv);
  const int q0 = q_tiles[4 * tile + 0], q1 = q_tiles[4 * tile + 1];
  const int g0 = q_tiles[4 * tile + 2], pe = q_tiles[4 * tile + 3];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hi = lane >> 5;

  const int qw0 = q0 + wave * 32;         // first row of this wave
  const int qwl = min(q1, qw0 + 32) - 1;  // last valid row of this wave
  const bool wave_active = qw0 < q1;
  const int qrow = qw0 + l32;
  const bool row_ok = qrow < q1;
  const int lo = row_ok ? row_lo[qrow] : 0;
  const int lo_first = wave_active ? row_lo[qw0] : 0;
  const int lo_last = wave_active ? row_lo[qwl] : 0;

  // Q rows of this wave as MFMA B operands: column = query l32, k = 16 st + 8 hi + j.
  bf16x8 qf[D / 16];
  {
    const bf16 *qp = Q + ((size_t)qrow * Hq + h) * D + 8 * hi;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      if (row_ok) {
        qf[st] = *reinterpret_cast<const bf16x8 *>(qp + 16 * st);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) qf[st][j] = (__bf16)0.f;
      }
    }
  }

  // Segment A: prefix keys [g0, min(pe, q1)).  Segment B: own-response keys
  // [max(pe, row_lo[q0]), q1); row_lo is non-decreasing inside a group.
  const int a0 = g0, a1 = min(pe, q1);
  const int b0 = max(pe, row_lo[q0]), b1 = q1;
  const int nA = a1 > a0 ? (a1 - a0 + C::BN - 1) / C::BN : 0;
  const int nB = b1 > b0 ? (b1 - b0 + C::BN - 1) / C::BN : 0;
  const int nC = nA + nB;

  const size_t kv_row = (size_t)Hkv * D;
  const bf16 *Kh = K + (size_t)hk * D;
  const bf16 *Vh = V + (size_t)hk * D;
  auto chunk_range = [&](int ci, int &c0, int &cend) {
    if (ci < nA) {
      c0 = a0 + ci * C::BN;
      cend = a1;
    } else {
      c0 = b0 + (ci - nA) * C::BN;
      cend = b1;
    }
  };
  // chunk ci lives in LDS buffer ci % 2 and is copied one chunk ahead
  TileCopy<D, C::BN, C::NW> copy;
  copy.init(kv_row, wave, lane);
  const uint32_t sK_lds = lds_address(sK), sV_lds = lds_address(sV);
  SwzFrags<D> frag;
  frag.init(lane);
  auto issue = [&](int ci) {
    int c0, cend;
    chunk_range(ci, c0, cend);
    const int buf = (ci & 1) * C::BN * D;
    copy.issue(sK + buf, sK_lds + 2 * buf, Kh, kv_row, c0, T - 1, wave, lane);
    copy.issue(sV + buf, sV_lds + 2 * buf, Vh, kv_row, c0, T - 1, wave, lane);
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[nb][r] = 0.f;
  // Running max (base-2, scaled) and partial row sum.  m starts finite and
  // only grows, so a masked score (-inf) always gives exp2(-inf) = 0 exactly.
  float m = kMasked, l = 0.f;

  if (nC > 0) issue(0);
  // unrolled over the two buffers, so buffer addresses are immediates
  for (int ci0 = 0; ci0 < nC; ci0 += 2)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ci = ci0 + u;
    if (ci >= nC) break;
    int c0, cend;
    chunk_range(ci, c0, cend);
    // chunk ci has landed for every wave, and every wave is done reading the
    // other buffer, which the next copy overwrites
    wait_async_loads();
    __syncthreads();
    if (ci + 1 < nC) issue(ci + 1);
    lds_cchar *cK = lds_bytes(sK + u * C::BN * D);
    lds_cchar *cV = lds_bytes(sV + u * C::BN * D);
    if (!wave_active) continue;
    const int clast = min(c0 + C::BN, cend) - 1;
    if (c0 > qwl) continue;                       // every key follows every row
    if (c0 >= pe && clast < lo_first) continue;   // keys of earlier responses only
    const bool full = (c0 + C::BN <= cend) && (c0 + C::BN - 1 <= qw0) &&
                      (c0 + C::BN <= pe || c0 >= lo_last);

    // S^T = K Q^T for two 32-key blocks
    f32x16 s[C::NB];
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = 0.f;
    // both key blocks per k-step: consecutive MFMAs are independent
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
#pragma unroll
      for (int b = 0; b < C::NB; ++b) s[b] = mfma32(frag.row(cK, b * 32, st), qf[st], s[b]);
    if (!full) {
#pragma unroll
      for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = c0 + b * 32 + mfma_row(r, hi);
          const bool ok = key < cend && key <= qrow && (key < pe || key >= lo);
          s[b][r] = ok ? s[b][r] : -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
    {
      float lo, hi;
      wave_halves(mx, lo, hi);
      mx = fmaxf(lo, hi) * scale_log2;
    }
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescale)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nb][r] *= alpha;
    }
    const float neg_m = -m;
    float rs = 0.f;
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[b][r], scale_log2, neg_m));
        s[b][r] = p;
        rs += p;
      }
    l += rs;
    // O^T += V^T P^T: A = V^T read transposed from row-major LDS, B = P^T from registers
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const bf16x8 pf = pack8(s[b], sub * 8);
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const bf16x8 a = frag.tr(cV, b * 32 + sub * 16, nb);
          o[nb] = mfma32(a, pf, o[nb]);
        }
      }
  }
  if (!wave_active) return;
  float l_lo, l_hi;
  wave_halves(l, l_lo, l_hi);
  const float lt = l_lo + l_hi;
  if (!row_ok) return;
  const float inv = 1.f / lt;
  bf16 *op = O + ((size_t)qrow * Hq + h) * D;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = nb * 32 + rq * 8 + hi * 4;
      *reinterpret_cast<u32x2 *>(op + d0) =
          pack4_bf16(o[nb][rq * 4 + 0] * inv, o[nb][rq * 4 + 1] * inv, o[nb][rq * 4 + 2] * inv,
                     o[nb][rq * 4 + 3] * inv);
    }
  if (LSE != nullptr && hi == 0) LSE[(size_t)h * T + qrow] = (m + __log2f(lt)) * kLn2;
}

}  // namespace

hipError_t launch_fwd_bf16(const Plan &p, float scale, const void *q, const void *k,
                           const void *v, void *o, float *lse, hipStream_t s) {
  if (p.n_q_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_q_tiles * (unsigned)p.Hq), block(256);
  const float sl2 = scale * kLog2e;
  if (p.D == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, block, 0, s, p.q_tiles, p.row_lo,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (bf16 *)o, lse, p.T,
                       p.Hq, p.Hkv, sl2);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, block, 0, s, p.q_tiles, p.row_lo,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (bf16 *)o, lse, p.T,
                       p.Hq, p.Hkv, sl2);
  return hipGetLastError();
}

}  // namespace pg
