/* Plain-C client of libpg_attn on the GPU: plans a packed batch with pg_pack,
 * runs pg_attn_fwd and pg_attn_bwd on device buffers it allocates with the HIP
 * runtime, and writes the outputs to a file.  Inputs and outputs are raw
 * little-endian files (bf16 bit patterns for Q, K, V, dO, O, dQ, dK, dV; float
 * for LSE).  The test compares the outputs with the Python binding's on the
 * same inputs.  Only C99, the library header and the HIP runtime API.
 *
 * usage: attn_device_run in.bin out.bin hq hkv d P R_1 ... R_G  (one group) */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "pg_attn.h"

#define CHECK_HIP(x)                                                      \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));             \
      return 1;                                                           \
    }                                                                     \
  } while (0)
#define CHECK_PG(x)                                                       \
  do {                                                                    \
    pg_status s_ = (x);                                                   \
    if (s_ != PG_OK) {                                                    \
      fprintf(stderr, "%s: %d %s\n", #x, (int)s_, pg_last_error());       \
      return 1;                                                           \
    }                                                                     \
  } while (0)

int main(int argc, char **argv) {
  if (argc < 8) return 2;
  const int hq = atoi(argv[3]), hkv = atoi(argv[4]), d = atoi(argv[5]);
  const int32_t prefix = atoi(argv[6]);
  const int32_t G = argc - 7;
  int32_t *resp = (int32_t *)malloc(sizeof(int32_t) * (size_t)G);
  int64_t T = prefix;
  for (int i = 0; i < G; ++i) {
    resp[i] = atoi(argv[7 + i]);
    T += resp[i];
  }
  const pg_groups g = {1, &prefix, &G, resp, hq, hkv, d};
  const size_t nq = (size_t)T * hq * d, nk = (size_t)T * hkv * d;

  /* inputs: Q [T, hq, d], K, V [T, hkv, d], dO [T, hq, d] as bf16 bits */
  uint16_t *h_in = (uint16_t *)malloc(2 * (2 * nq + 2 * nk));
  FILE *f = fopen(argv[1], "rb");
  if (!f || fread(h_in, 2, 2 * nq + 2 * nk, f) != 2 * nq + 2 * nk) return 3;
  fclose(f);

  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  void *q, *k, *v, *dout, *o, *dq, *dk, *dv, *lse, *buf, *ws;
  CHECK_HIP(hipMalloc(&q, 2 * nq));
  CHECK_HIP(hipMalloc(&k, 2 * nk));
  CHECK_HIP(hipMalloc(&v, 2 * nk));
  CHECK_HIP(hipMalloc(&dout, 2 * nq));
  CHECK_HIP(hipMalloc(&o, 2 * nq));
  CHECK_HIP(hipMalloc(&dq, 2 * nq));
  CHECK_HIP(hipMalloc(&dk, 2 * nk));
  CHECK_HIP(hipMalloc(&dv, 2 * nk));
  CHECK_HIP(hipMalloc(&lse, sizeof(float) * (size_t)hq * T));
  CHECK_HIP(hipMemcpy(q, h_in, 2 * nq, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(k, h_in + nq, 2 * nk, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v, h_in + nq + nk, 2 * nk, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dout, h_in + nq + 2 * nk, 2 * nq, hipMemcpyHostToDevice));

  const size_t bytes = pg_pack_buffer_size(&g);
  if (bytes == 0) {
    fprintf(stderr, "pg_pack_buffer_size: %s\n", pg_last_error());
    return 1;
  }
  CHECK_HIP(hipMalloc(&buf, bytes));
  pg_desc desc;
  CHECK_PG(pg_pack(&g, buf, bytes, NULL, &desc, s));
  CHECK_PG(pg_attn_fwd(&desc, PG_BF16, 0.f, q, k, v, o, (float *)lse, s));
  const size_t wsb = pg_attn_bwd_workspace_size(&desc, PG_BF16);
  CHECK_HIP(hipMalloc(&ws, wsb));
  CHECK_PG(pg_attn_bwd(&desc, PG_BF16, 0.f, q, k, v, o, (const float *)lse, dout, dq, dk, dv, ws,
                       wsb, s));
  CHECK_HIP(hipStreamSynchronize(s));

  /* outputs: O, dQ, dK, dV (bf16 bits) then LSE (float) */
  uint16_t *h_out = (uint16_t *)malloc(2 * (2 * nq + 2 * nk));
  float *h_lse = (float *)malloc(sizeof(float) * (size_t)hq * T);
  CHECK_HIP(hipMemcpy(h_out, o, 2 * nq, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_out + nq, dq, 2 * nq, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_out + 2 * nq, dk, 2 * nk, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_out + 2 * nq + nk, dv, 2 * nk, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_lse, lse, sizeof(float) * (size_t)hq * T, hipMemcpyDeviceToHost));
  f = fopen(argv[2], "wb");
  if (!f) return 3;
  fwrite(h_out, 2, 2 * nq + 2 * nk, f);
  fwrite(h_lse, sizeof(float), (size_t)hq * T, f);
  fclose(f);
  printf("rows %lld pairs %lld\n", (long long)T, (long long)desc.pairs);
  return 0;
}
