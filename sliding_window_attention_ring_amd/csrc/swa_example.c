/*
 * swa_example.c -- drives libswa.so through include/swa.h alone (no Python):
 * allocates a bf16 ring cache with hipMalloc, appends tokens, decodes, and
 * checks two closed forms of single-query attention on the host:
 *   1. with one visible token the output is that token's value row exactly;
 *   2. with every visible key identical the weights are uniform, so the
 *      output is the mean of the visible value rows.
 * It also checks the position invariant with swa_validate and an error path.
 * Prints "swa_example ok" and returns 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "swa.h"

#define CHECK_HIP(x)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      fprintf(stderr, "%s:%d HIP error %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 2;                                                                        \
    }                                                                                  \
  } while (0)
#define CHECK_SWA(x)                                                                   \
  do {                                                                                 \
    int s_ = (x);                                                                      \
    if (s_ != SWA_OK) {                                                                \
      fprintf(stderr, "%s:%d swa error %d: %s\n", __FILE__, __LINE__, s_, swa_status_string(s_)); \
      return 3;                                                                        \
    }                                                                                  \
  } while (0)

/* float -> bf16 bits, round to nearest even (inputs here are finite) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(void) {
  const int B = 2, H = 3, D = 128, W = 64, T = 40;
  const size_t rows = (size_t)B * H * W * D, nnew = (size_t)B * H * T * D;
  swa_cache c;
  memset(&c, 0, sizeof c);
  c.kind = SWA_KV_BF16;
  c.B = B; c.H = H; c.D = D; c.W = W;
  c.layout = SWA_LAYOUT_RING;
  CHECK_HIP(hipMalloc(&c.k, rows * 2));
  CHECK_HIP(hipMalloc(&c.v, rows * 2));
  CHECK_HIP(hipMalloc((void **)&c.pos, (size_t)B * W * 4));
  CHECK_HIP(hipMalloc((void **)&c.next_position, (size_t)B * 4));
  CHECK_SWA(swa_cache_reset(&c, NULL));

  /* Token j of every (b, h): key = all ones (identical keys), value = row
   * of small integers depending on (b, h, j, d), exact in bf16. */
  uint16_t *hk = malloc(nnew * 2), *hv = malloc(nnew * 2), *hq = malloc((size_t)B * H * D * 2);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int j = 0; j < T; ++j)
        for (int d = 0; d < D; ++d) {
          size_t i = (((size_t)b * H + h) * T + j) * D + d;
          hk[i] = to_bf16(1.0f);
          hv[i] = to_bf16((float)((b * 7 + h * 5 + j * 3 + d) % 17 - 8));
        }
  for (size_t i = 0; i < (size_t)B * H * D; ++i) hq[i] = to_bf16(0.5f * (float)(i % 5) - 1.0f);
  void *dk, *dv, *dq, *ws;
  float *dout;
  int32_t *dviol;
  CHECK_HIP(hipMalloc(&dk, nnew * 2));
  CHECK_HIP(hipMalloc(&dv, nnew * 2));
  CHECK_HIP(hipMalloc(&dq, (size_t)B * H * D * 2));
  CHECK_HIP(hipMalloc((void **)&dout, (size_t)B * H * D * 4));
  CHECK_HIP(hipMalloc((void **)&dviol, 4));
  CHECK_HIP(hipMemcpy(dk, hk, nnew * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, hv, nnew * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dq, hq, (size_t)B * H * D * 2, hipMemcpyHostToDevice));
  const size_t ws_bytes = swa_workspace_bytes(&c);
  CHECK_HIP(hipMalloc(&ws, ws_bytes > 16 ? ws_bytes : 16));
  CHECK_SWA(swa_workspace_init(ws, ws_bytes, NULL));

  float *out = malloc((size_t)B * H * D * 4);
  int failures = 0;

  /* 1. one token: output = its value row, exactly.  The first token of each
   *    sequence is row j = 0 of the chunk, so append it as a T=1 chunk. */
  uint16_t *k1 = malloc((size_t)B * H * D * 2), *v1 = malloc((size_t)B * H * D * 2);
  for (int bh = 0; bh < B * H; ++bh) {
    memcpy(k1 + (size_t)bh * D, hk + (size_t)bh * T * D, D * 2);
    memcpy(v1 + (size_t)bh * D, hv + (size_t)bh * T * D, D * 2);
  }
  void *dk1, *dv1;
  CHECK_HIP(hipMalloc(&dk1, (size_t)B * H * D * 2));
  CHECK_HIP(hipMalloc(&dv1, (size_t)B * H * D * 2));
  CHECK_HIP(hipMemcpy(dk1, k1, (size_t)B * H * D * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv1, v1, (size_t)B * H * D * 2, hipMemcpyHostToDevice));
  CHECK_SWA(kv_append(&c, dk1, dv1, 1, NULL));
  CHECK_SWA(decode_attn(&c, dq, dout, ws, ws_bytes, NULL));
  CHECK_HIP(hipMemcpy(out, dout, (size_t)B * H * D * 4, hipMemcpyDeviceToHost));
  for (int bh = 0; bh < B * H; ++bh)
    for (int d = 0; d < D; ++d)
      if (out[(size_t)bh * D + d] != from_bf16(v1[(size_t)bh * D + d])) ++failures;

  /* 2. reset, append all T tokens (identical keys): output = mean of values. */
  CHECK_SWA(swa_cache_reset(&c, NULL));
  CHECK_SWA(kv_append(&c, dk, dv, T, NULL));
  CHECK_SWA(decode_attn(&c, dq, dout, ws, ws_bytes, NULL));
  CHECK_HIP(hipMemcpy(out, dout, (size_t)B * H * D * 4, hipMemcpyDeviceToHost));
  double worst = 0.0;
  for (int bh = 0; bh < B * H; ++bh)
    for (int d = 0; d < D; ++d) {
      double mean = 0.0;
      for (int j = 0; j < T; ++j) mean += from_bf16(hv[((size_t)bh * T + j) * D + d]);
      mean /= T;
      double err = fabs(out[(size_t)bh * D + d] - mean);
      if (err > worst) worst = err;
    }
  if (worst > 2e-3) ++failures;

  /* position invariant and one host-checked error path */
  CHECK_HIP(hipMemset(dviol, 0, 4));
  CHECK_SWA(swa_validate(&c, dviol, NULL));
  int32_t viol = -1;
  CHECK_HIP(hipMemcpy(&viol, dviol, 4, hipMemcpyDeviceToHost));
  if (viol != 0) ++failures;
  if (decode_attn(&c, dq, dout, ws, ws_bytes > 0 ? ws_bytes - 1 : 0, NULL) != SWA_EWORKSPACE && ws_bytes > 0)
    ++failures;

  printf("swa_example %s: one-token rows exact, identical-key mean max err %.3g, violations %d\n",
         failures ? "FAILED" : "ok", worst, viol);
  hipFree(c.k); hipFree(c.v); hipFree(c.pos); hipFree(c.next_position);
  hipFree(dk); hipFree(dv); hipFree(dq); hipFree(dout); hipFree(dviol); hipFree(ws); hipFree(dk1); hipFree(dv1);
  free(hk); free(hv); free(hq); free(out); free(k1); free(v1);
  return failures ? 1 : 0;
}
