// Response log-probability head of the GRPO step on the packed layout
// (skillsmp.com "prefix-grouper-grpo", "Step 4: Training Integration with
// GRPO": log-softmax of the logits over the vocabulary, gathered at each
// response token, summed per response; loss -mean(A_i * sum_i)).
//
// Only the scored rows are computed: the predicting row of every response
// token (the previous position of its baseline sequence; a response's first
// token is scored by the group's last prefix row, shared by the G responses).
// The logits Z = H_pred W^T and the two backward products are plain GEMMs
// (rocBLAS, bf16 operands, fp32 accumulation); the kernels here are the
// memory-bound steps around them:
//   gather_rows   H_pred[k] = hidden[pred[k]]
//   lsm_fwd       per scored row: logsumexp over the vocabulary (one pass,
//                 running max) and logp = z[token] - lse
//   grpo_loss     loss = -mean_i(A_i * S_i), S_i = sum of response i's logp,
//                 summed entry by entry; dlogp[k] = -A_{resp(k)} / n_resp
//   lsm_bwd       G[k, v] = dlogp[k] * ([v == token] - exp(z[k, v] - lse[k]))
//   scatter_rows  dhidden[t] = sum of dH_pred[k] over the entries t predicts,
//                 in entry order (the last prefix row of a group sums its G
//                 responses' first tokens: the prefix gradient is the sum of
//                 its copies', Pith review, "Core claim", Lemma 2.1)
// Every reduction has a fixed order: results are bitwise repeatable.

#include "pg_device.h"
#include "pg_internal.h"

namespace pg {
namespace {

constexpr int kHeadThreads = 256;

__global__ __launch_bounds__(kHeadThreads) void gather_rows_kernel(
    const int32_t *__restrict__ pred, const uint4 *__restrict__ hidden, uint4 *__restrict__ out,
    int n, int cpr) {
  const long long i = (long long)blockIdx.x * kHeadThreads + threadIdx.x;
  if (i >= (long long)n * cpr) return;
  const int k = (int)(i / cpr), c = (int)(i - (long long)k * cpr);
  out[i] = hidden[(size_t)pred[k] * cpr + c];
}

// Block reduction of (max, sum of exp(x - max)) pairs, fixed tree order.
__device__ __forceinline__ void combine(float &m, float &s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  s = (m == -INFINITY ? 0.f : s * __expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - mn));
  m = mn;
}

template <bool kVec4>
__global__ __launch_bounds__(kHeadThreads) void lsm_fwd_kernel(
    const float *__restrict__ z, const int32_t *__restrict__ scored_row,
    const int32_t *__restrict__ tokens, float *__restrict__ logp, float *__restrict__ lse, int V) {
  const int k = blockIdx.x, tid = threadIdx.x;
  const float *row = z + (size_t)k * V;
  float m = -INFINITY, s = 0.f;
  if (kVec4) {
    const float4 *r4 = reinterpret_cast<const float4 *>(row);
    for (int i = tid; i < V / 4; i += kHeadThreads) {
      const float4 x = r4[i];
      const float xm = fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w));
      const float mn = fmaxf(m, xm);
      s = (m == -INFINITY ? 0.f : s * __expf(m - mn)) + __expf(x.x - mn) + __expf(x.y - mn) +
          __expf(x.z - mn) + __expf(x.w - mn);
      m = mn;
    }
  } else {
    for (int i = tid; i < V; i += kHeadThreads) {
      const float x = row[i];
      const float mn = fmaxf(m, x);
      s = (m == -INFINITY ? 0.f : s * __expf(m - mn)) + __expf(x - mn);
      m = mn;
    }
  }
  __shared__ float sm[kHeadThreads], ss[kHeadThreads];
  sm[tid] = m;
  ss[tid] = s;
  __syncthreads();
  for (int w = kHeadThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      float a = sm[tid], b = ss[tid];
      combine(a, b, sm[tid + w], ss[tid + w]);
      sm[tid] = a;
      ss[tid] = b;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const float l = sm[0] + __logf(ss[0]);
    lse[k] = l;
    const int tok = tokens[scored_row[k]];
    logp[k] = (unsigned)tok < (unsigned)V ? row[tok] - l : __int_as_float(0x7fc00000);  // NaN: bad id
  }
}

// One block: loss = -(1/n_resp) sum_r A_r S_r = -(1/n_resp) sum_k A_{resp(k)} logp_k,
// each thread taking entries k = tid, tid + 256, ... and a fixed tree after.
__global__ __launch_bounds__(kHeadThreads) void grpo_loss_kernel(
    const float *__restrict__ logp, const int32_t *__restrict__ scored_resp,
    const float *__restrict__ adv, float *__restrict__ loss, int n, int n_resp) {
  __shared__ float part[kHeadThreads];
  float acc = 0.f;
  for (int k = threadIdx.x; k < n; k += kHeadThreads) acc += adv[scored_resp[k]] * logp[k];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kHeadThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = -part[0] / (float)n_resp;
}

__global__ __launch_bounds__(kHeadThreads) void grpo_dlogp_kernel(
    const int32_t *__restrict__ scored_resp, const float *__restrict__ adv,
    float *__restrict__ dlogp, int n, int n_resp) {
  const int k = blockIdx.x * kHeadThreads + threadIdx.x;
  if (k < n) dlogp[k] = -adv[scored_resp[k]] / (float)n_resp;
}

template <bool kVec4>
__global__ __launch_bounds__(kHeadThreads) void lsm_bwd_kernel(
    const float *__restrict__ z, const int32_t *__restrict__ scored_row,
    const int32_t *__restrict__ tokens, const float *__restrict__ lse,
    const float *__restrict__ dlogp, bf16 *__restrict__ g, int V) {
  const int k = blockIdx.x, tid = threadIdx.x;
  const float *row = z + (size_t)k * V;
  bf16 *grow = g + (size_t)k * V;
  const float l = lse[k], d = dlogp[k];
  const int tok = tokens[scored_row[k]];
  if (kVec4) {
    const float4 *r4 = reinterpret_cast<const float4 *>(row);
    for (int i = tid; i < V / 4; i += kHeadThreads) {
      const float4 x = r4[i];
      const int v = 4 * i;
      const float g0 = d * ((v + 0 == tok ? 1.f : 0.f) - __expf(x.x - l));
      const float g1 = d * ((v + 1 == tok ? 1.f : 0.f) - __expf(x.y - l));
      const float g2 = d * ((v + 2 == tok ? 1.f : 0.f) - __expf(x.z - l));
      const float g3 = d * ((v + 3 == tok ? 1.f : 0.f) - __expf(x.w - l));
      *reinterpret_cast<u32x2 *>(grow + v) = pack4_bf16(g0, g1, g2, g3);
    }
  } else {
    for (int v = tid; v < V; v += kHeadThreads)
      grow[v] = (bf16)(d * ((v == tok ? 1.f : 0.f) - __expf(row[v] - l)));
  }
}

__global__ __launch_bounds__(kHeadThreads) void scatter_rows_kernel(
    const int32_t *__restrict__ pred_start, const int32_t *__restrict__ pred_list,
    const float4 *__restrict__ dh_pred, float4 *__restrict__ dhidden, int T, int cpr) {
  const long long i = (long long)blockIdx.x * kHeadThreads + threadIdx.x;
  if (i >= (long long)T * cpr) return;
  const int t = (int)(i / cpr), c = (int)(i - (long long)t * cpr);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int e = pred_start[t]; e < pred_start[t + 1]; ++e) {
    const float4 x = dh_pred[(size_t)pred_list[e] * cpr + c];
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  dhidden[i] = acc;
}

unsigned blocks_for(long long work) { return (unsigned)((work + kHeadThreads - 1) / kHeadThreads); }

}  // namespace

hipError_t launch_gather_rows(const int32_t *pred, const void *hidden, void *out, int n,
                              int d_model, hipStream_t s) {
  const int cpr = d_model / 8;  // 16-byte chunks of bf16
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks_for((long long)n * cpr)), dim3(kHeadThreads),
                     0, s, pred, (const uint4 *)hidden, (uint4 *)out, n, cpr);
  return hipGetLastError();
}

hipError_t launch_lsm_fwd(const float *z, const int32_t *scored_row, const int32_t *tokens,
                          float *logp, float *lse, int n, int V, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (V % 4 == 0)
    hipLaunchKernelGGL(lsm_fwd_kernel<true>, dim3(n), dim3(kHeadThreads), 0, s, z, scored_row,
                       tokens, logp, lse, V);
  else
    hipLaunchKernelGGL(lsm_fwd_kernel<false>, dim3(n), dim3(kHeadThreads), 0, s, z, scored_row,
                       tokens, logp, lse, V);
  return hipGetLastError();
}

hipError_t launch_grpo_loss(const float *logp, const int32_t *scored_resp, const float *adv,
                            float *loss, float *dlogp, int n, int n_resp, hipStream_t s) {
  hipLaunchKernelGGL(grpo_loss_kernel, dim3(1), dim3(kHeadThreads), 0, s, logp, scored_resp, adv,
                     loss, n, n_resp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n == 0) return e;
  hipLaunchKernelGGL(grpo_dlogp_kernel, dim3(blocks_for(n)), dim3(kHeadThreads), 0, s,
                     scored_resp, adv, dlogp, n, n_resp);
  return hipGetLastError();
}

hipError_t launch_lsm_bwd(const float *z, const int32_t *scored_row, const int32_t *tokens,
                          const float *lse, const float *dlogp, void *g, int n, int V,
                          hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (V % 4 == 0)
    hipLaunchKernelGGL(lsm_bwd_kernel<true>, dim3(n), dim3(kHeadThreads), 0, s, z, scored_row,
                       tokens, lse, dlogp, (bf16 *)g, V);
  else
    hipLaunchKernelGGL(lsm_bwd_kernel<false>, dim3(n), dim3(kHeadThreads), 0, s, z, scored_row,
                       tokens, lse, dlogp, (bf16 *)g, V);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const int32_t *pred_start, const int32_t *pred_list,
                               const float *dh_pred, float *dhidden, int T, int d_model,
                               hipStream_t s) {
  const int cpr = d_model / 4;  // float4 chunks
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3(blocks_for((long long)T * cpr)), dim3(kHeadThreads),
                     0, s, pred_start, pred_list, (const float4 *)dh_pred, (float4 *)dhidden, T,
                     cpr);
  return hipGetLastError();
}

}  // namespace pg
