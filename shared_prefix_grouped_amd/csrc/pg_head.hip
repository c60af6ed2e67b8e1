// Response log-probability head of the GRPO step on the packed layout
// (skillsmp.com "prefix-grouper-grpo", "Step 4: Training Integration with
// GRPO": log-softmax of the logits over the vocabulary, gathered at each
// response token, summed per response; loss -mean(A_i * sum_i)).
//
// Only the scored rows are computed: the predicting row of every response
// token (the previous position of its baseline sequence; a response's first
// token is scored by the group's last prefix row, shared by the G responses).
// The logits products and the log-softmax around them are the tile kernels of
// pg_head_mfma.hip; the kernels here are the row moves and the loss:
//   gather_rows   H_pred[k] = hidden[pred[k]]
//   grpo_loss     loss = -mean_i(A_i * S_i), S_i = sum of response i's logp,
//                 summed entry by entry; dlogp[k] = -A_{resp(k)} / n_resp
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
