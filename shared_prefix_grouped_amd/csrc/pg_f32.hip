// Grouped shared-prefix attention in float32 throughout, and the rotary
// embedding at baseline position ids.
//
// The float32 path keeps full single precision (no bf16 rounding of any
// operand) and the visibility rule of the bf16 MFMA kernels: query row q sees
// prefix keys [group start, min(prefix end, q + 1)) and own-response keys
// [max(prefix end, row_lo[q]), q + 1); key row k is seen by query rows
// [k, row_hi[k]) (Pith review of Prefix Grouper, "What carries the argument").
//
// It targets small problems, where the time is set by the longest serial walk
// (keys for a query row, query rows for a key row), not by arithmetic.  So a
// workgroup owns a sub-tile of 8 rows of one plan tile and one head, each row's
// head dimension is spread over 8 adjacent lanes (d / 8 columns each, so one
// wave holds the sub-tile's rows), and the workgroup's eight
// waves split the walk eight ways, interleaved; their partial results are
// combined in a fixed order at the end (online-softmax merge for the forward,
// plain sums for the gradients), so results are bitwise repeatable.  The walk
// is staged through the LDS in chunks of 32 rows, double buffered: the next
// chunk's global loads are in flight while the current chunk is used.
//
// The backward is one launch: dK/dV workgroups first, then dQ workgroups.
// Both compute delta = rowsum(dO * O) and the base-2 logsumexp of the query
// rows they use themselves (dK/dV for each staged chunk, dQ for its own rows),
// so no preprocessing pass runs before it.

#include "pg_device.h"
#include "pg_internal.h"

namespace pg {
namespace {

constexpr int kRowLanes = 8;   // lanes sharing one row's head dimension
constexpr int kWalkWaves = 8;  // waves splitting one sub-tile's walk
constexpr int kF32Threads = 64 * kWalkWaves;
constexpr int kChunk = 32;     // walk rows per LDS chunk
static_assert(PG_TILE_Q == PG_TILE_KV, "one sub-tile split for query and key tiles");

template <int D>
struct F32Split {
  static constexpr int L = kRowLanes;       // lanes per row
  static constexpr int SL = D / L;           // columns per lane
  static constexpr int R = 64 / L;           // rows per sub-tile
  static constexpr int SUB = PG_TILE_Q / R;  // sub-tiles per plan tile
  // A staged chunk of one tensor keeps each SL-column part of its rows
  // together ([part][row][SL]); the parts are 4 floats apart beyond whole
  // rows, so the L lanes of a row, which read the same row in different
  // parts, hit different LDS banks.
  static constexpr int PART = kChunk * SL + 4;
  static constexpr int TENSOR = L * PART;
  static constexpr int NL = kChunk * D / 4 / kF32Threads;  // 16-byte loads per thread and tensor
  static_assert(NL * 4 * kF32Threads == kChunk * D, "chunk is a whole number of loads");
};

// Swap partners within a row's lane group: DPP quad permutations for lane
// distances 1 and 2, a ds_swizzle (xor mode within 32 lanes) beyond.
__device__ __forceinline__ float lane_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  static_assert(M >= 4 && M <= 16, "ds_swizzle xor mode covers lanes within 32");
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (M << 10)));
}

// Sum over the N consecutive lanes of an aligned group (N a power of two,
// N <= 32).  Each step adds a lane's value to its partner's; IEEE addition is
// commutative, so every lane of the group ends with the same bits.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += lane_xor1(x);
  if constexpr (N >= 4) x += lane_xor2(x);
  if constexpr (N >= 8) x += lane_xor<4>(x);
  if constexpr (N >= 16) x += lane_xor<8>(x);
  if constexpr (N >= 32) x += lane_xor<16>(x);
  return x;
}

// Partial dot product of a lane's N columns with N staged floats.
template <int N>
__device__ __forceinline__ float dotn(const float (&a)[N], const float *__restrict__ b) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < N; c += 4) {
    const f32x4 y = *reinterpret_cast<const f32x4 *>(b + c);
    s += a[c] * y[0];
    s += a[c + 1] * y[1];
    s += a[c + 2] * y[2];
    s += a[c + 3] * y[3];
  }
  return s;
}

template <int N>
__device__ __forceinline__ void loadn(float (&a)[N], const float *__restrict__ p) {
#pragma unroll
  for (int c = 0; c < N; c += 4) {
    const f32x4 y = *reinterpret_cast<const f32x4 *>(p + c);
    a[c] = y[0];
    a[c + 1] = y[1];
    a[c + 2] = y[2];
    a[c + 3] = y[3];
  }
}

// Staging of one chunk: 16-byte piece n of thread t is float4
// i = t + kF32Threads * n of the chunk's [kChunk][D] rows.
template <int D>
struct ChunkPiece {
  int row, col;  // row within the chunk, first column
  __device__ __forceinline__ ChunkPiece(int n) {
    const int i = (int)threadIdx.x + n * kF32Threads;
    row = i / (D / 4);
    col = (i % (D / 4)) * 4;
  }
  // offset of the piece in a staged tensor ([part][row][SL] layout)
  __device__ __forceinline__ int lds() const {
    constexpr int SL = F32Split<D>::SL;
    return (col / SL) * F32Split<D>::PART + row * SL + col % SL;
  }
};

// Rows [s, s + n) of a [T][H][D] tensor at head hh: 16-byte pieces into
// registers, zero past row s + n.
template <int D>
__device__ __forceinline__ void load_chunk(f32x4 (&r)[F32Split<D>::NL], const float *__restrict__ X,
                                           int s, int n, int H, int hh) {
#pragma unroll
  for (int j = 0; j < F32Split<D>::NL; ++j) {
    const ChunkPiece<D> pc(j);
    r[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (pc.row < n)
      r[j] = *reinterpret_cast<const f32x4 *>(X + ((size_t)(s + pc.row) * H + hh) * D + pc.col);
  }
}

template <int D>
__device__ __forceinline__ void store_chunk(float *__restrict__ dst, const f32x4 (&r)[F32Split<D>::NL]) {
#pragma unroll
  for (int j = 0; j < F32Split<D>::NL; ++j) {
    const ChunkPiece<D> pc(j);
    *reinterpret_cast<f32x4 *>(dst + pc.lds()) = r[j];
  }
}

// The key segments a query sub-tile [qa, qb) walks: prefix keys
// [g0, min(pe, qb)) in nA chunks, then own-response keys from the first row's
// response start, [max(pe, row_lo[qa]), qb), in the remaining chunks.
struct KeyWalk {
  int g0, a_end, b0, qb, nA, n;
  __device__ __forceinline__ KeyWalk(int g0_, int pe, int qa_lo, int qb_) {
    g0 = g0_;
    qb = qb_;
    a_end = min(pe, qb);
    b0 = max(pe, qa_lo);
    nA = a_end > g0 ? (a_end - g0 + kChunk - 1) / kChunk : 0;
    n = nA + (qb > b0 ? (qb - b0 + kChunk - 1) / kChunk : 0);
  }
  __device__ __forceinline__ int start(int c) const {
    return c < nA ? g0 + c * kChunk : b0 + (c - nA) * kChunk;
  }
  __device__ __forceinline__ int count(int c) const {
    return min(kChunk, (c < nA ? a_end : qb) - start(c));
  }
};

template <int D>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(
    const int32_t *__restrict__ q_tiles, const int32_t *__restrict__ row_lo,
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int T, int Hq, int Hkv, float scale_log2) {
  using S = F32Split<D>;
  constexpr int SL = S::SL;
  __shared__ __align__(16) float sm[2 * 2 * S::TENSOR];  // [buffer][K, V]
  static_assert(2 * 2 * S::TENSOR >= kWalkWaves * 64 * (SL + 4), "combine fits the buffers");
  const int h = (int)blockIdx.x % Hq;
  const int rest = (int)blockIdx.x / Hq;
  const int sub = rest % S::SUB, tile = rest / S::SUB;
  const int t0 = q_tiles[4 * tile + 0], q1 = q_tiles[4 * tile + 1];
  const int qa = t0 + sub * S::R;
  if (qa >= q1) return;  // whole workgroup
  const int qb = min(q1, qa + S::R);
  const int hk = h / (Hq / Hkv);
  const int w = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int part = lane % S::L;
  const bool own = qa + lane / S::L < qb;
  const int qrow = min(qa + lane / S::L, qb - 1);  // lanes past the end mirror the last row
  const int pe = q_tiles[4 * tile + 3];
  const int lo = max(pe, row_lo[qrow]);
  const KeyWalk kw(q_tiles[4 * tile + 2], pe, row_lo[qa], qb);

  float qv[SL], acc[SL];
  loadn(qv, Q + ((size_t)qrow * Hq + h) * D + part * SL);
#pragma unroll
  for (int c = 0; c < SL; ++c) acc[c] = 0.f;
  float m = kMasked, l = 0.f;

  f32x4 rk[S::NL], rv[S::NL];
  load_chunk<D>(rk, K, kw.start(0), kw.count(0), Hkv, hk);
  load_chunk<D>(rv, V, kw.start(0), kw.count(0), Hkv, hk);
  store_chunk<D>(sm, rk);
  store_chunk<D>(sm + S::TENSOR, rv);
  __syncthreads();
  for (int c = 0; c < kw.n; ++c) {
    if (c + 1 < kw.n) {
      load_chunk<D>(rk, K, kw.start(c + 1), kw.count(c + 1), Hkv, hk);
      load_chunk<D>(rv, V, kw.start(c + 1), kw.count(c + 1), Hkv, hk);
    }
    const float *sk = sm + (c & 1) * 2 * S::TENSOR + part * S::PART;
    const float *sv = sk + S::TENSOR;
    const int s0 = kw.start(c), cnt = kw.count(c);
    const bool segA = c < kw.nA;
    for (int j = w; j < cnt; j += kWalkWaves) {
      const int key = s0 + j;
      const bool vis = key <= qrow && (segA || key >= lo);
      const float s = group_sum<S::L>(dotn(qv, sk + j * SL)) * scale_log2;
      const float mn = vis ? fmaxf(m, s) : m;
      const float alpha = fast_exp2(m - mn);
      const float p = vis ? fast_exp2(s - mn) : 0.f;
      l = l * alpha + p;
      const float *vr = sv + j * SL;
#pragma unroll
      for (int cc = 0; cc < SL; ++cc) acc[cc] = acc[cc] * alpha + p * vr[cc];
      m = mn;
    }
    if (c + 1 < kw.n) {
      float *nb = sm + ((c + 1) & 1) * 2 * S::TENSOR;
      store_chunk<D>(nb, rk);
      store_chunk<D>(nb + S::TENSOR, rv);
    }
    __syncthreads();
  }

  // merge the waves' (max, sum, accumulator) in wave order; thread
  // (w, lane) with 4w < SL finishes columns [4w, 4w + 4) of its lane's SL
  constexpr int CS = SL + 4;
  float *mine = sm + (w * 64 + lane) * CS;
#pragma unroll
  for (int c = 0; c < SL; c += 4)
    *reinterpret_cast<f32x4 *>(mine + c) = f32x4{acc[c], acc[c + 1], acc[c + 2], acc[c + 3]};
  mine[SL] = m;
  mine[SL + 1] = l;
  __syncthreads();
  if (4 * w >= SL || !own) return;
  float M = kMasked;
#pragma unroll
  for (int x = 0; x < kWalkWaves; ++x) M = fmaxf(M, sm[(x * 64 + lane) * CS + SL]);
  float lsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < kWalkWaves; ++x) {
    const float *px = sm + (x * 64 + lane) * CS;
    const float f = fast_exp2(px[SL] - M);
    lsum += px[SL + 1] * f;
    o += *reinterpret_cast<const f32x4 *>(px + 4 * w) * f;
  }
  const float inv = 1.f / lsum;
  *reinterpret_cast<f32x4 *>(O + ((size_t)qrow * Hq + h) * D + part * SL + 4 * w) = o * inv;
  if (LSE != nullptr && w == 0 && part == 0) LSE[(size_t)h * T + qrow] = (M + __log2f(lsum)) * kLn2;
}

// dK/dV of one key sub-tile and kv head: the walk is query rows [ka, qend)
// for each query head of the kv head, chunks of kChunk rows staged with the
// rows' delta and base-2 logsumexp.
template <int D>
__device__ __forceinline__ void dkdv_f32_body(
    int bid, float *__restrict__ sm, const int32_t *__restrict__ kv_tiles,
    const int32_t *__restrict__ row_hi, const float *__restrict__ Q, const float *__restrict__ K,
    const float *__restrict__ V, const float *__restrict__ O, const float *__restrict__ LSE,
    const float *__restrict__ dO, float *__restrict__ dK, float *__restrict__ dV, int T, int Hq,
    int Hkv, float scale_log2, float scale) {
  using S = F32Split<D>;
  constexpr int SL = S::SL;
  constexpr int BUF = 2 * S::TENSOR + 2 * kChunk;  // Q, dO, lse2, delta
  const int hk = bid % Hkv;
  const int rest = bid / Hkv;
  const int sub = rest % S::SUB, tile = rest / S::SUB;
  const int k0 = kv_tiles[4 * tile + 0], k1 = kv_tiles[4 * tile + 1];
  const int ka = k0 + sub * S::R;
  if (ka >= k1) return;  // whole workgroup
  const int kb = min(k1, ka + S::R);
  const int rep = Hq / Hkv;
  const int w = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int part = lane % S::L;
  const bool own = ka + lane / S::L < kb;
  const int key = min(ka + lane / S::L, kb - 1);
  const int hi = row_hi[key];
  // within a group the prefix keys come first and are seen to the group's
  // end; response keys are seen to their response's end, increasing
  const int qend = max(row_hi[ka], row_hi[kb - 1]);
  const int nch = (qend - ka + kChunk - 1) / kChunk;
  const int steps = rep * nch;

  float kv[SL], vv[SL], gk[SL], gv[SL];
  loadn(kv, K + ((size_t)key * Hkv + hk) * D + part * SL);
  loadn(vv, V + ((size_t)key * Hkv + hk) * D + part * SL);
#pragma unroll
  for (int c = 0; c < SL; ++c) {
    gk[c] = 0.f;
    gv[c] = 0.f;
  }

  // staging: Q and dO pieces, O pieces for delta, and the chunk rows' lse;
  // the loads are issued a chunk ahead, delta is formed when they are stored
  f32x4 rq[S::NL], rg[S::NL], ro[S::NL];
  float rl = 0.f;
  auto load = [&](int st) {
    const int h = hk * rep + st / nch;
    const int s = ka + (st % nch) * kChunk;
    const int n = min(kChunk, qend - s);
    load_chunk<D>(rq, Q, s, n, Hq, h);
    load_chunk<D>(rg, dO, s, n, Hq, h);
    load_chunk<D>(ro, O, s, n, Hq, h);
    rl = 0.f;
    if ((int)threadIdx.x < n) rl = LSE[(size_t)h * T + s + (int)threadIdx.x] * kLog2e;
  };
  auto store = [&](float *b) {
    store_chunk<D>(b, rq);
    store_chunk<D>(b + S::TENSOR, rg);
#pragma unroll
    for (int j = 0; j < S::NL; ++j) {
      const f32x4 pr = rg[j] * ro[j];
      // a row's D / 4 pieces sit in consecutive lanes
      const float del = group_sum<D / 4>(pr[0] + pr[1] + pr[2] + pr[3]);
      const ChunkPiece<D> pc(j);
      if (pc.col == 0) b[2 * S::TENSOR + kChunk + pc.row] = del;
    }
    if ((int)threadIdx.x < kChunk) b[2 * S::TENSOR + threadIdx.x] = rl;
  };

  load(0);
  store(sm);
  __syncthreads();
  for (int st = 0; st < steps; ++st) {
    if (st + 1 < steps) load(st + 1);
    const float *b = sm + (st & 1) * BUF;
    const float *sq = b + part * S::PART;
    const float *sg = sq + S::TENSOR;
    const float *sl = b + 2 * S::TENSOR, *sd = sl + kChunk;
    const int s0 = ka + (st % nch) * kChunk;
    const int cnt = min(kChunk, qend - s0);
    for (int j = w; j < cnt; j += kWalkWaves) {
      const int row = s0 + j;
      const bool vis = row >= key && row < hi;
      const float *qr = sq + j * SL, *gr = sg + j * SL;
      const float s = group_sum<S::L>(dotn(kv, qr));
      const float dp = group_sum<S::L>(dotn(vv, gr));
      const float p = vis ? fast_exp2(s * scale_log2 - sl[j]) : 0.f;
      const float ds = p * (dp - sd[j]);
#pragma unroll
      for (int cc = 0; cc < SL; ++cc) {
        gv[cc] += p * gr[cc];
        gk[cc] += ds * qr[cc];
      }
    }
    if (st + 1 < steps) store(sm + ((st + 1) & 1) * BUF);
    __syncthreads();
  }

  // sum the waves' partials in wave order; thread (w, lane) with
  // 4w < SL finishes columns [4w, 4w + 4) of its lane's SL for dK and dV
  constexpr int CS = 2 * SL + 4;
  float *mine = sm + (w * 64 + lane) * CS;
#pragma unroll
  for (int c = 0; c < SL; c += 4) {
    *reinterpret_cast<f32x4 *>(mine + c) = f32x4{gk[c], gk[c + 1], gk[c + 2], gk[c + 3]};
    *reinterpret_cast<f32x4 *>(mine + SL + c) = f32x4{gv[c], gv[c + 1], gv[c + 2], gv[c + 3]};
  }
  __syncthreads();
  if (4 * w >= SL || !own) return;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < kWalkWaves; ++x) {
    const float *px = sm + (x * 64 + lane) * CS;
    sk += *reinterpret_cast<const f32x4 *>(px + 4 * w);
    sv += *reinterpret_cast<const f32x4 *>(px + SL + 4 * w);
  }
  const size_t off = ((size_t)key * Hkv + hk) * D + part * SL + 4 * w;
  *reinterpret_cast<f32x4 *>(dK + off) = sk * scale;
  *reinterpret_cast<f32x4 *>(dV + off) = sv;
}

// dQ of one query sub-tile and query head: the forward's key walk, with the
// row's delta and base-2 logsumexp computed in the prologue.
template <int D>
__device__ __forceinline__ void dq_f32_body(
    int bid, float *__restrict__ sm, const int32_t *__restrict__ q_tiles,
    const int32_t *__restrict__ row_lo, const float *__restrict__ Q, const float *__restrict__ K,
    const float *__restrict__ V, const float *__restrict__ O, const float *__restrict__ LSE,
    const float *__restrict__ dO, float *__restrict__ dQ, int T, int Hq, int Hkv, float scale_log2,
    float scale) {
  using S = F32Split<D>;
  constexpr int SL = S::SL;
  const int h = bid % Hq;
  const int rest = bid / Hq;
  const int sub = rest % S::SUB, tile = rest / S::SUB;
  const int t0 = q_tiles[4 * tile + 0], q1 = q_tiles[4 * tile + 1];
  const int qa = t0 + sub * S::R;
  if (qa >= q1) return;  // whole workgroup
  const int qb = min(q1, qa + S::R);
  const int hk = h / (Hq / Hkv);
  const int w = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int part = lane % S::L;
  const bool own = qa + lane / S::L < qb;
  const int qrow = min(qa + lane / S::L, qb - 1);
  const int pe = q_tiles[4 * tile + 3];
  const int lo = max(pe, row_lo[qrow]);
  const KeyWalk kw(q_tiles[4 * tile + 2], pe, row_lo[qa], qb);

  const size_t roff = ((size_t)qrow * Hq + h) * D + part * SL;
  float qv[SL], gv[SL], acc[SL];
  loadn(qv, Q + roff);
  loadn(gv, dO + roff);
  float dpart = 0.f;
  {
    float ov[SL];
    loadn(ov, O + roff);
#pragma unroll
    for (int c = 0; c < SL; ++c) dpart += gv[c] * ov[c];
  }
  const float Dq = group_sum<S::L>(dpart);
  const float Lq = LSE[(size_t)h * T + qrow] * kLog2e;
#pragma unroll
  for (int c = 0; c < SL; ++c) acc[c] = 0.f;

  f32x4 rk[S::NL], rv[S::NL];
  load_chunk<D>(rk, K, kw.start(0), kw.count(0), Hkv, hk);
  load_chunk<D>(rv, V, kw.start(0), kw.count(0), Hkv, hk);
  store_chunk<D>(sm, rk);
  store_chunk<D>(sm + S::TENSOR, rv);
  __syncthreads();
  for (int c = 0; c < kw.n; ++c) {
    if (c + 1 < kw.n) {
      load_chunk<D>(rk, K, kw.start(c + 1), kw.count(c + 1), Hkv, hk);
      load_chunk<D>(rv, V, kw.start(c + 1), kw.count(c + 1), Hkv, hk);
    }
    const float *sk = sm + (c & 1) * 2 * S::TENSOR + part * S::PART;
    const float *sv = sk + S::TENSOR;
    const int s0 = kw.start(c), cnt = kw.count(c);
    const bool segA = c < kw.nA;
    for (int j = w; j < cnt; j += kWalkWaves) {
      const int key = s0 + j;
      const bool vis = key <= qrow && (segA || key >= lo);
      const float *kr = sk + j * SL;
      const float s = group_sum<S::L>(dotn(qv, kr));
      const float dp = group_sum<S::L>(dotn(gv, sv + j * SL));
      const float p = vis ? fast_exp2(s * scale_log2 - Lq) : 0.f;
      const float ds = p * (dp - Dq);
#pragma unroll
      for (int cc = 0; cc < SL; ++cc) acc[cc] += ds * kr[cc];
    }
    if (c + 1 < kw.n) {
      float *nb = sm + ((c + 1) & 1) * 2 * S::TENSOR;
      store_chunk<D>(nb, rk);
      store_chunk<D>(nb + S::TENSOR, rv);
    }
    __syncthreads();
  }

  constexpr int CS = SL + 4;
  float *mine = sm + (w * 64 + lane) * CS;
#pragma unroll
  for (int c = 0; c < SL; c += 4)
    *reinterpret_cast<f32x4 *>(mine + c) = f32x4{acc[c], acc[c + 1], acc[c + 2], acc[c + 3]};
  __syncthreads();
  if (4 * w >= SL || !own) return;
  f32x4 sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < kWalkWaves; ++x)
    sq += *reinterpret_cast<const f32x4 *>(sm + (x * 64 + lane) * CS + 4 * w);
  *reinterpret_cast<f32x4 *>(dQ + roff + 4 * w) = sq * scale;
}

template <int D>
struct BwdLds {
  // dK/dV: two buffers of (Q, dO, lse2, delta); dQ: two buffers of (K, V);
  // both reuse them for the final combine
  static constexpr int STAGE = 2 * (2 * F32Split<D>::TENSOR + 2 * kChunk);
  static constexpr int COMBINE = kWalkWaves * 64 * (2 * F32Split<D>::SL + 4);
  static constexpr int FLOATS = STAGE > COMBINE ? STAGE : COMBINE;
};

template <int D>
__global__ __launch_bounds__(kF32Threads) void bwd_f32_kernel(
    const int32_t *__restrict__ q_tiles, const int32_t *__restrict__ kv_tiles,
    const int32_t *__restrict__ row_lo, const int32_t *__restrict__ row_hi,
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ O, const float *__restrict__ LSE, const float *__restrict__ dO,
    float *__restrict__ dQ, float *__restrict__ dK, float *__restrict__ dV, int T, int Hq,
    int Hkv, int n_dkdv_blocks, float scale_log2, float scale) {
  __shared__ __align__(16) float sm[BwdLds<D>::FLOATS];
  const int bid = (int)blockIdx.x;
  if (bid < n_dkdv_blocks)
    dkdv_f32_body<D>(bid, sm, kv_tiles, row_hi, Q, K, V, O, LSE, dO, dK, dV, T, Hq, Hkv,
                     scale_log2, scale);
  else
    dq_f32_body<D>(bid - n_dkdv_blocks, sm, q_tiles, row_lo, Q, K, V, O, LSE, dO, dQ, T, Hq, Hkv,
                   scale_log2, scale);
}

// Rotary embedding, rotate-half pairing; angle computed in double so that
// large positions keep full precision.  One thread per (row, pair index):
// the angle depends on those two only, so its cosine and sine are computed
// once and applied to that pair of every head of the row.
template <typename Tx>
__global__ __launch_bounds__(256) void rope_kernel(Tx *__restrict__ x, const int32_t *__restrict__ pos,
                                                   int T, int H, int D, double log_theta,
                                                   int inverse) {
  const int half = D / 2;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)T * half) return;
  const int i = (int)(idx % half);
  const int t = (int)(idx / half);
  const double inv_freq = exp(-log_theta * (2.0 * i) / D);
  const double ang = (double)pos[t] * inv_freq;
  const float c = (float)cos(ang);
  float s = (float)sin(ang);
  if (inverse) s = -s;
  Tx *row = x + (size_t)t * H * D;
  for (int h = 0; h < H; ++h) {
    Tx *r = row + (size_t)h * D;
    const float a = (float)r[i], b = (float)r[i + half];
    r[i] = (Tx)(a * c - b * s);
    r[i + half] = (Tx)(b * c + a * s);
  }
}

// Workgroups of a float32 launch over `tiles` plan tiles and `heads` heads,
// or -1 when the count does not fit the kernels' int workgroup index.
long long f32_blocks(int tiles, int D, int heads) {
  const long long sub = D == 128 ? F32Split<128>::SUB : F32Split<64>::SUB;
  const long long n = (long long)tiles * sub * heads;
  return n > 0x7FFFFFFFLL ? -1 : n;
}

}  // namespace

hipError_t launch_fwd_f32(const Plan &p, float scale, const void *q, const void *k,
                          const void *v, void *o, float *lse, hipStream_t s) {
  const long long nb = f32_blocks(p.n_q_tiles, p.D, p.Hq);
  if (nb == 0) return hipSuccess;
  if (nb < 0) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nb), block(kF32Threads);
  const float sl2 = scale * kLog2e;
  if (p.D == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, s, p.q_tiles, p.row_lo,
                       (const float *)q, (const float *)k, (const float *)v, (float *)o, lse, p.T,
                       p.Hq, p.Hkv, sl2);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, s, p.q_tiles, p.row_lo,
                       (const float *)q, (const float *)k, (const float *)v, (float *)o, lse, p.T,
                       p.Hq, p.Hkv, sl2);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const Plan &p, float scale, const void *q, const void *k,
                          const void *v, const void *o, const float *lse, const void *dout,
                          void *dq, void *dk, void *dv, hipStream_t s) {
  const long long nkv = f32_blocks(p.n_kv_tiles, p.D, p.Hkv);
  const long long nq = f32_blocks(p.n_q_tiles, p.D, p.Hq);
  if (nkv < 0 || nq < 0 || nkv + nq > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  if (nkv + nq == 0) return hipSuccess;
  const dim3 grid((unsigned)(nkv + nq)), block(kF32Threads);
  const float sl2 = scale * kLog2e;
  if (p.D == 128)
    hipLaunchKernelGGL(bwd_f32_kernel<128>, grid, block, 0, s, p.q_tiles, p.kv_tiles, p.row_lo,
                       p.row_hi, (const float *)q, (const float *)k, (const float *)v,
                       (const float *)o, lse, (const float *)dout, (float *)dq, (float *)dk,
                       (float *)dv, p.T, p.Hq, p.Hkv, (int)nkv, sl2, scale);
  else
    hipLaunchKernelGGL(bwd_f32_kernel<64>, grid, block, 0, s, p.q_tiles, p.kv_tiles, p.row_lo,
                       p.row_hi, (const float *)q, (const float *)k, (const float *)v,
                       (const float *)o, lse, (const float *)dout, (float *)dq, (float *)dk,
                       (float *)dv, p.T, p.Hq, p.Hkv, (int)nkv, sl2, scale);
  return hipGetLastError();
}

hipError_t launch_rope(int T, int H, int D, pg_dtype t, void *x, const int32_t *pos, float theta,
                       int inverse, hipStream_t s) {
  const long long n = (long long)T * (D / 2);  // one thread per (row, pair index)
  if (n == 0 || H == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  const double lt = log((double)theta);
  if (t == PG_BF16)
    hipLaunchKernelGGL(rope_kernel<__bf16>, grid, block, 0, s, (__bf16 *)x, pos, T, H, D, lt,
                       inverse);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, block, 0, s, (float *)x, pos, T, H, D, lt,
                       inverse);
  return hipGetLastError();
}

}  // namespace pg
