// Grouped shared-prefix attention in float32 throughout, and the rotary
// embedding at baseline position ids.
//
// The float32 path keeps full single precision (no bf16 rounding of any
// operand), one lane pair per query row (forward, dQ) or key row (dK/dV), with
// the same work lists and visibility rule as the bf16 MFMA kernels:
// query row q sees prefix keys [group start, min(prefix end, q + 1)) and
// own-response keys [max(prefix end, row_lo[q]), q + 1); key row k is seen by
// query rows [k, row_hi[k]) (Pith review of Prefix Grouper, "What carries the
// argument").  It targets small problems where launch latency, not
// arithmetic, dominates.

#include "pg_device.h"
#include "pg_internal.h"

namespace pg {
namespace {

// Each row's head dimension is split over a pair of adjacent lanes (DH = D / 2
// columns each), so that per-thread state stays in registers at d = 128; the
// two partial dot products are combined with one lane swap.
constexpr int kF32Threads = 2 * PG_TILE_Q;  // 2 lanes per row, PG_TILE_Q == PG_TILE_KV rows
static_assert(PG_TILE_Q == PG_TILE_KV, "one block size for all float32 kernels");

template <int N>
__device__ __forceinline__ float dot_part(const float *__restrict__ a, const float *__restrict__ b) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < N; c += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4 *>(a + c);
    const f32x4 y = *reinterpret_cast<const f32x4 *>(b + c);
    s += x[0] * y[0];
    s += x[1] * y[1];
    s += x[2] * y[2];
    s += x[3] * y[3];
  }
  return s;
}

// Full dot product of a row split over a lane pair.
__device__ __forceinline__ float pair_sum(float part) { return part + __shfl_xor(part, 1); }

template <int D>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(
    const int32_t *__restrict__ q_tiles, const int32_t *__restrict__ row_lo,
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    float *__restrict__ O, float *__restrict__ LSE, int T, int Hq, int Hkv, float scale_log2) {
  constexpr int DH = D / 2;
  const int tile = blockIdx.x / Hq;
  const int h = blockIdx.x - tile * Hq;
  const int hk = h / (Hq / Hkv);
  const int q0 = q_tiles[4 * tile + 0], q1 = q_tiles[4 * tile + 1];
  const int g0 = q_tiles[4 * tile + 2], pe = q_tiles[4 * tile + 3];
  const int qrow = q0 + (int)(threadIdx.x >> 1);
  const int c0 = (threadIdx.x & 1) * DH;  // this lane's columns [c0, c0 + DH)
  if (qrow >= q1) return;                 // both lanes of the pair leave together
  const int lo = row_lo[qrow];
  const float *qp = Q + ((size_t)qrow * Hq + h) * D + c0;
  float qv[DH], acc[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    qv[c] = qp[c];
    acc[c] = 0.f;
  }
  float m = kMasked, l = 0.f;
  auto visit = [&](int key) {
    const float *kp = K + ((size_t)key * Hkv + hk) * D + c0;
    const float *vp = V + ((size_t)key * Hkv + hk) * D + c0;
    const float s = pair_sum(dot_part<DH>(qv, kp)) * scale_log2;
    const float m_new = fmaxf(m, s);
    const float alpha = fast_exp2(m - m_new);
    const float p = fast_exp2(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int c = 0; c < DH; ++c) acc[c] = acc[c] * alpha + p * vp[c];
    m = m_new;
  };
  const int a1 = min(pe, qrow + 1);
  for (int key = g0; key < a1; ++key) visit(key);
  for (int key = max(pe, lo); key <= qrow; ++key) visit(key);
  const float inv = 1.f / l;
  float *op = O + ((size_t)qrow * Hq + h) * D + c0;
#pragma unroll
  for (int c = 0; c < DH; ++c) op[c] = acc[c] * inv;
  if (LSE != nullptr && c0 == 0) LSE[(size_t)h * T + qrow] = (m + __log2f(l)) * kLn2;
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void dq_f32_kernel(
    const int32_t *__restrict__ q_tiles, const int32_t *__restrict__ row_lo,
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ LSE2, const float *__restrict__ Delta, const float *__restrict__ dO,
    float *__restrict__ dQ, int T, int Hq, int Hkv, float scale_log2, float scale) {
  constexpr int DH = D / 2;
  const int tile = blockIdx.x / Hq;
  const int h = blockIdx.x - tile * Hq;
  const int hk = h / (Hq / Hkv);
  const int q0 = q_tiles[4 * tile + 0], q1 = q_tiles[4 * tile + 1];
  const int g0 = q_tiles[4 * tile + 2], pe = q_tiles[4 * tile + 3];
  const int qrow = q0 + (int)(threadIdx.x >> 1);
  const int c0 = (threadIdx.x & 1) * DH;
  if (qrow >= q1) return;
  const int lo = row_lo[qrow];
  const float Lq = LSE2[(size_t)h * T + qrow];
  const float Dq = Delta[(size_t)h * T + qrow];
  const float *qp = Q + ((size_t)qrow * Hq + h) * D + c0;
  const float *gp = dO + ((size_t)qrow * Hq + h) * D + c0;
  float qv[DH], gv[DH], acc[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    qv[c] = qp[c];
    gv[c] = gp[c];
    acc[c] = 0.f;
  }
  auto visit = [&](int key) {
    const float *kp = K + ((size_t)key * Hkv + hk) * D + c0;
    const float *vp = V + ((size_t)key * Hkv + hk) * D + c0;
    const float p = fast_exp2(pair_sum(dot_part<DH>(qv, kp)) * scale_log2 - Lq);
    const float ds = p * (pair_sum(dot_part<DH>(gv, vp)) - Dq);
#pragma unroll
    for (int c = 0; c < DH; ++c) acc[c] += ds * kp[c];
  };
  const int a1 = min(pe, qrow + 1);
  for (int key = g0; key < a1; ++key) visit(key);
  for (int key = max(pe, lo); key <= qrow; ++key) visit(key);
  float *dp = dQ + ((size_t)qrow * Hq + h) * D + c0;
#pragma unroll
  for (int c = 0; c < DH; ++c) dp[c] = acc[c] * scale;
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void dkdv_f32_kernel(
    const int32_t *__restrict__ kv_tiles, const int32_t *__restrict__ row_hi,
    const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ V,
    const float *__restrict__ LSE2, const float *__restrict__ Delta, const float *__restrict__ dO,
    float *__restrict__ dK, float *__restrict__ dV, int T, int Hq, int Hkv, float scale_log2,
    float scale) {
  constexpr int DH = D / 2;
  const int tile = blockIdx.x / Hkv;
  const int hk = blockIdx.x - tile * Hkv;
  const int rep = Hq / Hkv;
  const int k0 = kv_tiles[4 * tile + 0], k1 = kv_tiles[4 * tile + 1];
  const int key = k0 + (int)(threadIdx.x >> 1);
  const int c0 = (threadIdx.x & 1) * DH;
  if (key >= k1) return;
  const int hik = row_hi[key];
  const float *kp = K + ((size_t)key * Hkv + hk) * D + c0;
  const float *vp = V + ((size_t)key * Hkv + hk) * D + c0;
  float gk[DH], gv[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    gk[c] = 0.f;
    gv[c] = 0.f;
  }
  // fixed order: query heads of this kv head, then query rows ascending
  for (int j = 0; j < rep; ++j) {
    const int h = hk * rep + j;
    for (int qr = key; qr < hik; ++qr) {
      const float *qp = Q + ((size_t)qr * Hq + h) * D + c0;
      const float *gp = dO + ((size_t)qr * Hq + h) * D + c0;
      const float p =
          fast_exp2(pair_sum(dot_part<DH>(qp, kp)) * scale_log2 - LSE2[(size_t)h * T + qr]);
      const float ds = p * (pair_sum(dot_part<DH>(gp, vp)) - Delta[(size_t)h * T + qr]);
#pragma unroll
      for (int c = 0; c < DH; ++c) {
        gv[c] += p * gp[c];
        gk[c] += ds * qp[c];
      }
    }
  }
  float *dkp = dK + ((size_t)key * Hkv + hk) * D + c0;
  float *dvp = dV + ((size_t)key * Hkv + hk) * D + c0;
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    dkp[c] = gk[c] * scale;
    dvp[c] = gv[c];
  }
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

}  // namespace

hipError_t launch_fwd_f32(const Plan &p, float scale, const void *q, const void *k,
                          const void *v, void *o, float *lse, hipStream_t s) {
  if (p.n_q_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_q_tiles * (unsigned)p.Hq), block(kF32Threads);
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

hipError_t launch_bwd_dq_f32(const Plan &p, float scale, const void *q, const void *k,
                             const void *v, const float *lse, const float *delta,
                             const void *dout, void *dq, hipStream_t s) {
  if (p.n_q_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_q_tiles * (unsigned)p.Hq), block(kF32Threads);
  const float sl2 = scale * kLog2e;
  if (p.D == 128)
    hipLaunchKernelGGL(dq_f32_kernel<128>, grid, block, 0, s, p.q_tiles, p.row_lo,
                       (const float *)q, (const float *)k, (const float *)v, lse, delta,
                       (const float *)dout, (float *)dq, p.T, p.Hq, p.Hkv, sl2, scale);
  else
    hipLaunchKernelGGL(dq_f32_kernel<64>, grid, block, 0, s, p.q_tiles, p.row_lo,
                       (const float *)q, (const float *)k, (const float *)v, lse, delta,
                       (const float *)dout, (float *)dq, p.T, p.Hq, p.Hkv, sl2, scale);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const Plan &p, float scale, const void *q, const void *k,
                               const void *v, const float *lse, const float *delta,
                               const void *dout, void *dk, void *dv, hipStream_t s) {
  if (p.n_kv_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_kv_tiles * (unsigned)p.Hkv), block(kF32Threads);
  const float sl2 = scale * kLog2e;
  if (p.D == 128)
    hipLaunchKernelGGL(dkdv_f32_kernel<128>, grid, block, 0, s, p.kv_tiles, p.row_hi,
                       (const float *)q, (const float *)k, (const float *)v, lse, delta,
                       (const float *)dout, (float *)dk, (float *)dv, p.T, p.Hq, p.Hkv, sl2,
                       scale);
  else
    hipLaunchKernelGGL(dkdv_f32_kernel<64>, grid, block, 0, s, p.kv_tiles, p.row_hi,
                       (const float *)q, (const float *)k, (const float *)v, lse, delta,
                       (const float *)dout, (float *)dk, (float *)dv, p.T, p.Hq, p.Hkv, sl2,
                       scale);
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
