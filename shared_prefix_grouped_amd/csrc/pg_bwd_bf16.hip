// Grouped shared-prefix attention, backward, bf16 storage / fp32 accumulation,
// for gfx950 (CDNA4, wave64, v_mfma_f32_32x32x16_bf16).
//
// The softmax is recomputed from the logsumexp saved by the forward pass.
// Gradients equal those of the repeated-prefix baseline (Pith review of
// Prefix Grouper, "Core claim", Lemma 2.1): the dK/dV of a prefix key row is
// the sum over every query row that sees it -- the later prefix rows and every
// row of all G responses of the group -- which in the baseline is the sum over
// the G prefix copies.  No floating-point atomics are used:
//   * dkdv: key-stationary.  A workgroup owns 128 key rows of one key/value
//     head and walks, in a fixed order, every query head of that kv head and
//     every 32-row query block of its range, accumulating dK^T and dV^T in
//     registers (split over two waves per 32-key group, see below).  For a
//     prefix tile that walk covers the prefix rows and all responses of the
//     group, so the group reduction of Lemma 2.1 happens in registers, in a
//     fixed order.  When that walk alone outweighs the mean work per compute
//     unit (a short prefix shared by many responses), the planner cuts it
//     into pieces of whole query blocks: each piece writes float partial sums
//     and dkdv_sum_kernel adds them in piece order.
//   * dq: query-stationary, over the same two key segments as the forward.
// Both are deterministic: every output element is written by exactly one
// lane, after a reduction whose order does not depend on scheduling.

#include "pg_device.h"
#include "pg_internal.h"

namespace pg {
namespace {

// ---------------------------------------------------------------- dK, dV
// A workgroup owns 128 key rows of one kv head, as 4 groups of 32 keys, and
// runs 8 waves, two per key group.  Wave A holds the group's K and V rows and
// computes, per 32-row query block, S = Q K^T and dP = dO V^T, then
// P = exp(S - LSE) and dS = P * (dP - delta); it publishes P and dS, packed to
// bf16 in the MFMA operand layout, in LDS.  Wave B holds the dV^T and dK^T
// accumulators and adds dV^T += dO^T P and dK^T += Q^T dS.  Each role then
// issues 16 MFMAs per step, and B, free of operand registers, can keep its
// fragment reads in flight.
//
// The query rows are walked in steps of 32 (one MFMA block) with one barrier
// per step: in step n wave A forms P_n and dS_n; wave B consumes P_{n-1} and
// dS_{n-1} (published by the barrier that opened step n).  Q/dO rows (+ LSE,
// delta) live in a ring of NSLOT LDS slots, staged through registers of the
// A waves (see stage / commit below).
template <int D>
struct DkdvCfg {
  static constexpr int BN = PG_TILE_KV;  // key rows per workgroup
  static constexpr int NG = BN / 32;     // 32-key groups
  static constexpr int NW = 2 * NG;      // waves: role A and role B per key group
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32;          // query rows per step
  static constexpr int NSLOT = 4;        // ring slots: n-1, n read; n+1 landed; n+2 being written
};

template <int D>
__global__ __launch_bounds__(512) void dkdv_bf16_kernel(
    const int32_t *__restrict__ kv_items, const int32_t *__restrict__ row_hi,
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const float *__restrict__ LSE2, const float *__restrict__ Delta, const bf16 *__restrict__ dO,
    bf16 *__restrict__ dK, bf16 *__restrict__ dV, float *__restrict__ partial, int T, int Hq,
    int Hkv, float scale_log2, float scale) {
  using C = DkdvCfg<D>;
  // Q and dO rows of a step, row-major and swizzled: read as MFMA rows for
  // S = Q K^T and dP = dO V^T, and transposed for dV^T += dO^T P and
  // dK^T += Q^T dS.  LSE / delta slots hold 64 floats (32 used).
  __shared__ __attribute__((aligned(16))) bf16 sQ[C::NSLOT * C::BM * D];
  __shared__ __attribute__((aligned(16))) bf16 sdO[C::NSLOT * C::BM * D];
  __shared__ __attribute__((aligned(16))) float sL[C::NSLOT * 64];
  __shared__ __attribute__((aligned(16))) float sDl[C::NSLOT * 64];
  // P and dS of one 32x32 block per key group, by step parity, as bf16 MFMA
  // B operands: [group][parity][P0, P1, dS0, dS1][lane].
  __shared__ __attribute__((aligned(16))) bf16x8 sX[C::NG][2][4][64];

  int item, hk;
  xcd_kvhead_work(blockIdx.x, Hkv, item, hk);
  const int rep = Hq / Hkv;
  // key rows [k0, k1), query rows [qa, qb); part >= 0: one piece of a cut tile
  const int k0 = kv_items[8 * item + 0], k1 = kv_items[8 * item + 1];
  const int qa = kv_items[8 * item + 2], qb = kv_items[8 * item + 3];
  const int part = kv_items[8 * item + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hi = lane >> 5;
  const bool roleA = wave < C::NG;        // S, P, dV   (else dP, dS, dK)
  const int kg = roleA ? wave : wave - C::NG;

  const int kw0 = k0 + kg * 32;
  const int kwl = min(k1, kw0 + 32) - 1;
  const bool group_active = kw0 < k1;
  const int key = kw0 + l32;
  const bool key_ok = key < k1;
  const int hik = key_ok ? row_hi[key] : 0;  // queries [key, hik) see this key
  // smallest / largest visibility end over the group's keys
  int min_hi = key_ok ? hik : 0x7fffffff, max_hi = hik;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    min_hi = min(min_hi, __shfl_xor(min_hi, w));
    max_hi = max(max_hi, __shfl_xor(max_hi, w));
  }
  min_hi = __builtin_amdgcn_readfirstlane(min_hi);  // equal in every lane now
  max_hi = __builtin_amdgcn_readfirstlane(max_hi);
  SwzFrags<D> frag;
  frag.init(lane);

  // K and V rows of the group (role A) as MFMA B operands: column = key
  // l32, k = d.  The resources span rows [kw0, k1), so keys past the tile
  // read as zero; the head offset rides in the scalar offset.
  bf16x8 kf[D / 16], vf[D / 16];
  if (roleA) {
    const size_t kv_row = (size_t)Hkv * D * sizeof(bf16);
    const size_t span = group_active ? (size_t)(k1 - kw0) * kv_row : 0;
    const __amdgpu_buffer_rsrc_t rK = buffer_resource(K + (size_t)kw0 * Hkv * D, span);
    const __amdgpu_buffer_rsrc_t rV = buffer_resource(V + (size_t)kw0 * Hkv * D, span);
    const int voff = l32 * (int)kv_row + 16 * hi;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      kf[st] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rK, voff + 32 * st, hk * D * 2, 0));
      vf[st] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rV, voff + 32 * st, hk * D * 2, 0));
    }
  }
  // Let these loads complete here: left to the compiler, the wait for them
  // lands at their first use inside the step loop, where it would also wait
  // for the prefetch copies issued in the same step.
  wait_async_loads();
  pin(kf);
  pin(vf);

  // dK^T and dV^T (role B): register r of lane l holds d = 32 nb +
  // mfma_row(r, hi), key = l32.
  f32x16 acck[D / 32], accv[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acck[nb][r] = 0.f;
      accv[nb][r] = 0.f;
    }

  // Steps: 32-row query blocks [qa + 32 b, ...) for b = nB-1 down to 0, the
  // query heads of the kv head interleaved per block.  Walking down from
  // the end of the group, which every prefix tile of the group shares, keeps
  // the workgroups that run side by side on one XCD on the same Q/dO rows,
  // so those rows are fetched into that XCD's L2 once.
  const int nB = (qb - qa + C::BM - 1) / C::BM;  // blocks per query head
  const int nS = nB * rep;
  const size_t q_row = (size_t)Hq * D;
  // Step n = bi * rep + j covers query head hk * rep + j and the rows
  // [c0, c0 + 32), c0 = qa + (nB - 1 - bi) * 32; walking the steps in order
  // is a counter and a row pointer, with no division.
  struct Step {
    int j, c0;
  };
  const Step first{0, qa + (nB - 1) * C::BM};
  auto advance = [&](Step &st) {
    if (++st.j == rep) {
      st.j = 0;
      st.c0 -= C::BM;
    }
  };

  // Copies of step n into slot n % NSLOT go through registers of the role-A
  // waves (role B carries both accumulators and has no registers to spare;
  // it only meets the barrier): each A thread loads CPT 16-byte chunks of Q
  // and of dO (and waves 0 / 1 one LSE / delta value per row) at step n-3
  // and stores them into LDS with ordinary LDS writes at step n-2, after the
  // barrier that retired the slot's previous rows.  (Direct global->LDS
  // copies would compete with the fragment reads of both roles for the LDS,
  // and lose: the step would wait for them.)
  static_assert((C::NSLOT & (C::NSLOT - 1)) == 0, "slot index by mask");
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int NA = C::NG * 64;            // role-A threads
  constexpr int CPT = C::BM * CPR / NA;     // chunks per A thread and tensor
  static_assert(CPT >= 1 && CPT * NA == C::BM * CPR, "chunks split evenly over role A");
  // Buffer loads with one scalar descriptor per tensor, based at the work
  // item's first query row qa (the 64-bit base sits in the descriptor, so
  // only the walk's own span, not the tensor, has to fit the 32-bit
  // offsets): the row offset of the step from qa is part of the vector
  // offset, which the range check covers, so rows past the end of the batch
  // read as zero (the visibility mask covers them); the head offset rides in
  // the unchecked scalar offset and stays inside the row.
  const size_t q_avail = (size_t)(T - qa) * q_row * sizeof(bf16);
  const uint32_t q_span = (uint32_t)min(q_avail, (size_t)0xFFFFFFFFu);
  const __amdgpu_buffer_rsrc_t rQ = buffer_resource(Q + (size_t)qa * q_row, q_span);
  const __amdgpu_buffer_rsrc_t rdO = buffer_resource(dO + (size_t)qa * q_row, q_span);
  const __amdgpu_buffer_rsrc_t rL = buffer_resource(wave == 0 ? LSE2 : Delta, (size_t)Hq * T * 4);
  int coff[CPT], cdst[CPT];  // chunk c of this thread: source byte offset, swizzled LDS element
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int i = tid + c * NA, crow = i / CPR, cch = i % CPR;
    coff[c] = crow * (int)(q_row * sizeof(bf16)) + cch * 16;
    cdst[c] = crow * D + ((cch ^ swz_chunk<D>(crow)) << 3);
  }
  bf16x8 stq[CPT], sto[CPT];
  float stl = 0.f;
  // The rows of the steps are staged in step order; `stg` is the next one.
  Step stg = first;
  auto stage = [&]() {
    const int h = hk * rep + stg.j, c0 = stg.c0;
    advance(stg);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      // unsigned 32-bit byte offset from row qa (walks up to 4 GiB of Q rows)
      const int off = (int)((uint32_t)coff[c] +
                            (uint32_t)(c0 - qa) * (uint32_t)(q_row * sizeof(bf16)));
      stq[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rQ, off, h * D * 2, 0));
      sto[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rdO, off, h * D * 2, 0));
    }
    if (wave < 2) {
      // every lane loads, so no lane mask is needed: lanes past the 32 rows,
      // and rows past the batch, use an offset past the resource (read as 0)
      // (h T + row) * 4 < 2^31: the host checks Hq * T * 4 < 2^31
      const int off = (lane < C::BM && c0 + lane < T) ? (h * T + c0 + lane) * 4 : 0x7fffffff;
      stl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rL, off, 0, 0));
    }
  };
  auto commit = [&](int slot) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      *reinterpret_cast<bf16x8 *>(sQ + slot * C::BM * D + cdst[c]) = stq[c];
      *reinterpret_cast<bf16x8 *>(sdO + slot * C::BM * D + cdst[c]) = sto[c];
    }
    // lanes 32..63 land in the unused half of the 64-float slot; the delta
    // slot holds -delta, the start value of the dP accumulators
    if (wave < 2) (wave == 0 ? sL : sDl)[slot * 64 + lane] = wave == 0 ? stl : -stl;
  };
  // Start of step n (slot k = n mod NSLOT): every wave has finished step
  // n-1 and slot k (written in step n-2) is visible.  Then (role A) slot k+2,
  // last read in step n-1, receives the rows staged in step n-1, and the
  // rows of step n+3 are loaded.  The step loops below are unrolled NSLOT
  // times, so k, and with it every slot address, is a compile-time constant.
  auto open_step = [&](int n, int k) {
    __syncthreads();
    if (n + 2 < nS) commit((k + 2) & (C::NSLOT - 1));
    if (n + 3 < nS) stage();
  };
  auto slot_q = [&](int k) { return lds_bytes(sQ + (k & (C::NSLOT - 1)) * C::BM * D); };
  auto slot_do = [&](int k) { return lds_bytes(sdO + (k & (C::NSLOT - 1)) * C::BM * D); };

  // Whether query block [c0, c0 + 32) meets the group's keys at all, and
  // whether every (query, key) pair of it is visible.
  auto block_live = [&](int c0) { return group_active && !(c0 + 31 < kw0 || c0 >= max_hi); };
  auto block_full = [&](int c0) { return (c0 >= kwl) && (c0 + 32 <= min_hi); };

  if (roleA) {
    for (int j = 0; j < 3 && j < nS; ++j) {
      stage();
      if (j < 2) commit(j);
    }
  }
  // Drain the prologue's loads here: otherwise the compiler's wait analysis
  // carries them into the loop and waits for every step's own loads mid-step.
  // (pin keeps the loads above the wait: the wait itself orders no memory.)
  wait_async_loads();
  pin(stq);
  pin(sto);
  pin(stl);
  if (roleA) {
    // S, dP -> P, dS for step n, published for wave B, which uses them in
    // step n+1.  The loop runs to n = nS so that every wave meets the same
    // barriers.
    Step cur = first;
    for (int n0 = 0; n0 <= nS; n0 += C::NSLOT)
#pragma unroll
    for (int k = 0; k < C::NSLOT; ++k) {
      const int n = n0 + k;
      if (n > nS) break;
      open_step(n, k);
      const int c0 = cur.c0;
      advance(cur);
      if (n < nS && block_live(c0)) {
        lds_cchar *cQ = slot_q(k);
        lds_cchar *cdO = slot_do(k);
        const float *cL = sL + k * 64;
        const float *cDl = sDl + k * 64;
        // dp starts at -delta of its query row, so it ends as dP - delta
        f32x16 sc, dp;
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x4 nD = *reinterpret_cast<const f32x4 *>(&cDl[rq * 8 + hi * 4]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            sc[rq * 4 + j] = 0.f;
            dp[rq * 4 + j] = nD[j];
          }
        }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          sc = mfma32(frag.row(cQ, 0, st), kf[st], sc);
          dp = mfma32(frag.row(cdO, 0, st), vf[st], dp);
        }
        f32x16 p;
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const f32x4 Lq = *reinterpret_cast<const f32x4 *>(&cL[rq * 8 + hi * 4]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            p[rq * 4 + j] = fast_exp2(fmaf(sc[rq * 4 + j], scale_log2, -Lq[j]));
        }
        if (!block_full(c0)) {
          // query row c0 + 8 rq + 4 hi + j sees this key iff its distance
          // from the key is in [0, hik - key): one unsigned compare each.
          // (The empty asm keeps this a branch: if-converted, every block
          // would pay for the compares.)
          asm volatile("");
          const int dq0 = c0 + hi * 4 - key;
          const unsigned span = (unsigned)(hik - key);
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              p[rq * 4 + j] = (unsigned)(dq0 + rq * 8 + j) < span ? p[rq * 4 + j] : 0.f;
        }
        // dS = P * (dP - delta)
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = p[r] * dp[r];
        sX[kg][k & 1][0][lane] = pack8(p, 0);
        sX[kg][k & 1][1][lane] = pack8(p, 8);
        sX[kg][k & 1][2][lane] = pack8(dp, 0);
        sX[kg][k & 1][3][lane] = pack8(dp, 8);
      }
    }
  } else {
    // Nothing is in flight here, but the compiler lays the role-A loop out
    // with a path into this one, and its wait analysis would otherwise carry
    // that loop's copies in and wait for them (and so for this step's own
    // copies) in the middle of every step.
    wait_async_loads();
    bool live_prev = false;
    Step cur = first;
    for (int n0 = 0; n0 <= nS; n0 += C::NSLOT)
#pragma unroll
    for (int k = 0; k < C::NSLOT; ++k) {
      const int n = n0 + k;
      if (n > nS) break;
      __syncthreads();
      const int c0 = cur.c0;
      advance(cur);
      const bool live = n < nS && block_live(c0);
      const int kp = (k + C::NSLOT - 1) & (C::NSLOT - 1);  // slot of step n-1
      if (live_prev) {
        // dV^T += dO_{n-1}^T P_{n-1}, dK^T += Q_{n-1}^T dS_{n-1}
        lds_cchar *cQ = slot_q(kp);
        lds_cchar *cdO = slot_do(kp);
        const bf16x8 p0 = sX[kg][kp & 1][0][lane], p1 = sX[kg][kp & 1][1][lane];
        const bf16x8 d0 = sX[kg][kp & 1][2][lane], d1 = sX[kg][kp & 1][3][lane];
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          accv[nb] = mfma32(frag.tr(cdO, 0, nb), p0, accv[nb]);
          acck[nb] = mfma32(frag.tr(cQ, 0, nb), d0, acck[nb]);
        }
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          accv[nb] = mfma32(frag.tr(cdO, 16, nb), p1, accv[nb]);
          acck[nb] = mfma32(frag.tr(cQ, 16, nb), d1, acck[nb]);
        }
      }
      live_prev = live;
    }
  }

  if (roleA || !group_active || !key_ok) return;
  // kind 0: dV, kind 1: dK (scaled)
#pragma unroll
  for (int kind = 0; kind < 2; ++kind) {
    const f32x16 *acc = kind == 0 ? accv : acck;
    const float f = kind == 0 ? 1.f : scale;
    if (part < 0) {
      bf16 *dst = (kind == 0 ? dV : dK) + ((size_t)key * Hkv + hk) * D;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d0 = nb * 32 + rq * 8 + hi * 4;
          *reinterpret_cast<u32x2 *>(dst + d0) =
              pack4_bf16(acc[nb][rq * 4 + 0] * f, acc[nb][rq * 4 + 1] * f,
                         acc[nb][rq * 4 + 2] * f, acc[nb][rq * 4 + 3] * f);
        }
    } else {
      // partial slot [part][hk][dV, dK][key - k0][d], float
      float *dst = partial + (((size_t)part * Hkv + hk) * 2 + kind) * (C::BN * D) +
                   (size_t)(key - k0) * D;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d0 = nb * 32 + rq * 8 + hi * 4;
          f32x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = acc[nb][rq * 4 + j] * f;
          *reinterpret_cast<f32x4 *>(dst + d0) = v;
        }
    }
  }
}

// Sum of the pieces of each cut key tile, in piece order, to bf16 dK / dV.
// kv_sums[s] = {k0, k1, first part, parts}.  A block adds SUM_ROWS key rows
// (1024 floats) of one (cut tile, kv head, dV / dK): each thread one 4-float
// chunk, over the parts in order.  The partials were just written by the
// dK/dV kernel and are mostly L2-resident; with a block per 1024 floats the
// sum spreads over the whole GPU even when a single tile was cut.
template <int D>
__global__ __launch_bounds__(256) void dkdv_sum_kernel(const int32_t *__restrict__ kv_sums,
                                                       const float *__restrict__ partial,
                                                       bf16 *__restrict__ dK,
                                                       bf16 *__restrict__ dV, int Hkv) {
  constexpr int BN = PG_TILE_KV, CH = D / 4;
  constexpr int SUM_ROWS = 1024 / D;            // key rows per block
  constexpr int NRB = BN / SUM_ROWS;            // row blocks per tile
  static_assert(SUM_ROWS * CH == 256, "one 4-float chunk per thread");
  const int rb = blockIdx.x % NRB;
  const int rest = blockIdx.x / NRB;
  const int kind = rest & 1;
  const int sh = rest >> 1;
  const int si = sh / Hkv, hk = sh - si * Hkv;
  const int k0 = kv_sums[4 * si + 0], k1 = kv_sums[4 * si + 1];
  const int first = kv_sums[4 * si + 2], np = kv_sums[4 * si + 3];
  const int kl = rb * SUM_ROWS + (int)threadIdx.x / CH;  // key row within the tile
  const int c = (int)threadIdx.x % CH;
  if (k0 + kl >= k1) return;
  const size_t pstride = (size_t)Hkv * 2 * BN * D;
  const float *src = partial + (((size_t)first * Hkv + hk) * 2 + kind) * (BN * D) +
                     (size_t)kl * D + 4 * c;
  // the parts' loads are issued eight at a time (the partials come from
  // other XCDs' writes, a long round trip each), then added in part order
  f32x4 a = *reinterpret_cast<const f32x4 *>(src);
  int j = 1;
  for (; j + 8 <= np; j += 8) {
    f32x4 b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) b[u] = *reinterpret_cast<const f32x4 *>(src + (size_t)(j + u) * pstride);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += b[u][e];
  }
  for (; j < np; ++j) {
    const f32x4 b = *reinterpret_cast<const f32x4 *>(src + (size_t)j * pstride);
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += b[e];
  }
  bf16 *out = kind == 0 ? dV : dK;
  *reinterpret_cast<u32x2 *>(out + ((size_t)(k0 + kl) * Hkv + hk) * D + 4 * c) =
      pack4_bf16(a[0], a[1], a[2], a[3]);
}

// ---------------------------------------------------------------- dQ
template <int D>
struct DqCfg {
  static constexpr int BM = PG_TILE_Q;  // query rows per workgroup
  static constexpr int NW = BM / 32;
  static constexpr int NT = NW * 64;
  static constexpr int BN = kKvChunk;   // keys per chunk
};

// It also does the backward's preprocessing for the rows it owns (each row
// and query head belongs to exactly one dq work item): delta = rowsum(dO * O)
// and the base-2 logsumexp, used here and stored for the dK/dV kernel, which
// runs after it.
template <int D>
__global__ __launch_bounds__(256, 2) void dq_bf16_kernel(
    const int32_t *__restrict__ q_tiles, const int32_t *__restrict__ row_lo,
    const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ V,
    const bf16 *__restrict__ O, const float *__restrict__ LSE, float *__restrict__ LSE2,
    float *__restrict__ Delta, const bf16 *__restrict__ dO, bf16 *__restrict__ dQ, int T, int Hq,
    int Hkv, float scale_log2, float scale) {
  using C = DqCfg<D>;
  // K and V chunks, double-buffered, row-major and swizzled: K is read as MFMA
  // rows for S^T = K Q^T and transposed for dQ^T += K^T dS^T; V as rows for
  // dP^T = V dO^T.
  __shared__ __attribute__((aligned(16))) bf16 sK[2 * C::BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV[2 * C::BN * D];

  int tile, h;
  xcd_qhead_work(blockIdx.x, Hq, Hkv, tile, h);
  const int hk = h / (Hq / Hkv);
  const int q0 = q_tiles[4 * tile + 0], q1 = q_tiles[4 * tile + 1];
  const int g0 = q_tiles[4 * tile + 2], pe = q_tiles[4 * tile + 3];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hi = lane >> 5;

  const int qw0 = q0 + wave * 32;
  const int qwl = min(q1, qw0 + 32) - 1;
  const bool wave_active = qw0 < q1;
  const int qrow = qw0 + l32;
  const bool row_ok = qrow < q1;
  const int lo = row_ok ? row_lo[qrow] : 0;
  const int lo_first = wave_active ? row_lo[qw0] : 0;
  const int lo_last = wave_active ? row_lo[qwl] : 0;
  bf16x8 qf[D / 16], of[D / 16];
  // delta of the lane's row: this lane's half of the columns (16 st + 8 hi
  // + j), then the other half from lane l ^ 32, added in that order in both
  float dpart = 0.f;
  {
    const size_t base = ((size_t)qrow * Hq + h) * D + 8 * hi;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      if (row_ok) {
        qf[st] = *reinterpret_cast<const bf16x8 *>(Q + base + 16 * st);
        of[st] = *reinterpret_cast<const bf16x8 *>(dO + base + 16 * st);
      }
    }
    // The O rows are loaded once the Q and dO rows have arrived: with the
    // strided rows of all three tensors in flight at once, a small launch ran
    // 1.4-1.8x slower (most when the three tensors sit at conflicting
    // addresses); at large sizes the order makes no difference.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      if (row_ok) {
        const bf16x8 ov = *reinterpret_cast<const bf16x8 *>(O + base + 16 * st);
#pragma unroll
        for (int j = 0; j < 8; ++j) dpart = fmaf((float)of[st][j], (float)ov[j], dpart);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          qf[st][j] = (__bf16)0.f;
          of[st][j] = (__bf16)0.f;
        }
      }
    }
  }
  float Dq, negL;
  {
    float d_lo, d_hi;
    wave_halves(dpart, d_lo, d_hi);
    Dq = d_lo + d_hi;
    const float l2 = row_ok ? LSE[(size_t)h * T + qrow] * kLog2e : 0.f;
    negL = -l2;
    if (row_ok && hi == 0) {
      Delta[(size_t)h * T + qrow] = Dq;
      LSE2[(size_t)h * T + qrow] = l2;
    }
  }

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

  f32x16 dq[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[nb][r] = 0.f;

  if (nC > 0) issue(0);
  // the fragment offsets carry the buffer of chunk ci (flipped every chunk),
  // so the tile bases are constants and the reads take immediate offsets
  static_assert(((C::BN * D * 2) & (C::BN * D * 2 - 1)) == 0, "buffer size a power of two");
  lds_cchar *const cK = lds_bytes(sK);
  lds_cchar *const cV = lds_bytes(sV);
  for (int ci = 0; ci < nC; ++ci) {
    if (ci > 0) frag.flip(C::BN * D * 2);
    int c0, cend;
    chunk_range(ci, c0, cend);
    wait_async_loads();
    __syncthreads();
    if (ci + 1 < nC) issue(ci + 1);
    if (!wave_active) continue;
    const int clast = min(c0 + C::BN, cend) - 1;
    if (c0 > qwl) continue;
    if (c0 >= pe && clast < lo_first) continue;
    const bool full = (c0 + C::BN <= cend) && (c0 + C::BN - 1 <= qw0) &&
                      (c0 + C::BN <= pe || c0 >= lo_last);

#pragma unroll
    for (int b = 0; b < 2; ++b) {
      // dp starts at -delta of the lane's query, so it ends as dP - delta
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = -Dq;
      }
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        s = mfma32(frag.row(cK, b * 32, st), qf[st], s);
        dp = mfma32(frag.row(cV, b * 32, st), of[st], dp);
      }
      // register r holds key c0 + b*32 + mfma_row(r, hi); the lane's column is its query
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], scale_log2, negL));
      if (!full) {
        // key kr is visible iff kr <= kmax (its chunk end and the query) and
        // it is not in [pe, lo), the responses before the query's own.  (The
        // empty asm keeps this a branch, taken by partial chunks only.)
        asm volatile("");
        const int kb = c0 + b * 32 + 4 * hi;
        const int kmax = min(cend - 1, qrow) - kb;
        const unsigned gap = (unsigned)max(lo - pe, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = mfma_row(r, 0);  // key - kb
          const bool ok = kr <= kmax && (unsigned)(kr + kb - pe) >= gap;
          s[r] = ok ? s[r] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = s[r] * dp[r];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const bf16x8 db = pack8(s, sub * 8);
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb)
          dq[nb] = mfma32(frag.tr(cK, b * 32 + sub * 16, nb), db, dq[nb]);
      }
    }
  }

  if (!wave_active || !row_ok) return;
  bf16 *qp = dQ + ((size_t)qrow * Hq + h) * D;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = nb * 32 + rq * 8 + hi * 4;
      *reinterpret_cast<u32x2 *>(qp + d0) =
          pack4_bf16(dq[nb][rq * 4 + 0] * scale, dq[nb][rq * 4 + 1] * scale,
                     dq[nb][rq * 4 + 2] * scale, dq[nb][rq * 4 + 3] * scale);
    }
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16(const Plan &p, float scale, const void *q, const void *k,
                                const void *v, const float *lse, const float *delta,
                                const void *dout, void *dk, void *dv, float *partial,
                                hipStream_t s) {
  if (p.n_kv_items == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_kv_items * (unsigned)p.Hkv), block(DkdvCfg<128>::NT);
  const float sl2 = scale * kLog2e;
  if (p.D == 128)
    hipLaunchKernelGGL(dkdv_bf16_kernel<128>, grid, block, 0, s, p.kv_items, p.row_hi,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, lse, delta,
                       (const bf16 *)dout, (bf16 *)dk, (bf16 *)dv, partial, p.T, p.Hq, p.Hkv,
                       sl2, scale);
  else
    hipLaunchKernelGGL(dkdv_bf16_kernel<64>, grid, block, 0, s, p.kv_items, p.row_hi,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, lse, delta,
                       (const bf16 *)dout, (bf16 *)dk, (bf16 *)dv, partial, p.T, p.Hq, p.Hkv,
                       sl2, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_kv_sums == 0) return e;
  const unsigned nrb = PG_TILE_KV / (1024u / (unsigned)p.D);  // row blocks per cut tile
  const dim3 sgrid((unsigned)p.n_kv_sums * (unsigned)p.Hkv * 2u * nrb), sblock(256);
  if (p.D == 128)
    hipLaunchKernelGGL(dkdv_sum_kernel<128>, sgrid, sblock, 0, s, p.kv_sums,
                       (const float *)partial, (bf16 *)dk, (bf16 *)dv, p.Hkv);
  else
    hipLaunchKernelGGL(dkdv_sum_kernel<64>, sgrid, sblock, 0, s, p.kv_sums,
                       (const float *)partial, (bf16 *)dk, (bf16 *)dv, p.Hkv);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const Plan &p, float scale, const void *q, const void *k,
                              const void *v, const void *o, const float *lse, float *lse2,
                              float *delta, const void *dout, void *dq, hipStream_t s) {
  if (p.n_q_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_q_tiles * (unsigned)p.Hq), block(256);
  const float sl2 = scale * kLog2e;
  if (p.D == 128)
    hipLaunchKernelGGL(dq_bf16_kernel<128>, grid, block, 0, s, p.q_tiles, p.row_lo,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (const bf16 *)o, lse,
                       lse2, delta, (const bf16 *)dout, (bf16 *)dq, p.T, p.Hq, p.Hkv, sl2, scale);
  else
    hipLaunchKernelGGL(dq_bf16_kernel<64>, grid, block, 0, s, p.q_tiles, p.row_lo,
                       (const bf16 *)q, (const bf16 *)k, (const bf16 *)v, (const bf16 *)o, lse,
                       lse2, delta, (const bf16 *)dout, (bf16 *)dq, p.T, p.Hq, p.Hkv, sl2, scale);
  return hipGetLastError();
}

}  // namespace pg
