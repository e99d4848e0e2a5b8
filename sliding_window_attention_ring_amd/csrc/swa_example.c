/*
 * swa_example.c -- drives libswa.so through include/swa.h alone (no Python):
 * allocates a bf16 ring cache with hipMalloc, appends tokens, decodes, and
 * checks two closed forms of single-query attention on the host:
 *   1. with one visible token the output is that token's value row exactly;
 *   2. with every visible key identical the weights are uniform, so the
 *      output is the mean of the visible value rows.
 * It also checks the position invariant with swa_validate and an error path.
 * A second part uses an INT8 cache with the witness bound, then one with
 * subtractive dither, stepping each with decode_step_int8 (append + decode
 * in one call) on one cache and with kv_append + the separate decode on a
 * twin, and with decode_step_int8_static (no workspace) on a third: the
 * three must agree bit for bit, and with identical keys and values that are
 * exact multiples of their block scale the output is the mean of the value
 * rows (within the dither's half step for the dithered kind).
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

  /* ---- INT8 (witness; then dithered): fused step vs append + decode ---- */
  const int T8 = 37, D8 = 128, W8 = 64;
  const size_t n8 = (size_t)B * H * T8 * D8;
  uint16_t *k8 = malloc(n8 * 2), *v8 = malloc(n8 * 2);
  for (int bh = 0; bh < B * H; ++bh)
    for (int j = 0; j < T8; ++j)
      for (int d = 0; d < D8; ++d) {
        const size_t i = ((size_t)bh * T8 + j) * D8 + d;
        k8[i] = to_bf16(1.0f);
        /* value = m/16 with |m| <= 127 and m = 127 at d = 0: every block's scale is exactly 1/16 */
        const int m = d == 0 ? 127 : (bh * 13 + j * 7 + d * 3) % 255 - 127;
        v8[i] = to_bf16((float)m / 16.0f);
      }
  void *dq8, *dkt, *dvt;
  CHECK_HIP(hipMalloc(&dq8, (size_t)B * H * D8 * 2));
  CHECK_HIP(hipMemcpy(dq8, hq, (size_t)B * H * D8 * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMalloc(&dkt, (size_t)B * H * D8 * 2));
  CHECK_HIP(hipMalloc(&dvt, (size_t)B * H * D8 * 2));
  uint16_t *kt = malloc((size_t)B * H * D8 * 2), *vt = malloc((size_t)B * H * D8 * 2);
  float *o0 = malloc((size_t)B * H * D8 * 4), *o1 = malloc((size_t)B * H * D8 * 4);
  float *o2 = malloc((size_t)B * H * D8 * 4);
  float cm0[64], cm1[64], cm2[64];
  uint64_t rid[2] = {0x0123456789abcdefull, 42u};  /* the dithered kind's request ids */
  uint64_t *drid;
  CHECK_HIP(hipMalloc((void **)&drid, sizeof rid));
  CHECK_HIP(hipMemcpy(drid, rid, sizeof rid, hipMemcpyHostToDevice));
  int mism[2] = {0, 0}, mism_static[2] = {0, 0};
  double worst8[2] = {0.0, 0.0};
  for (int pass = 0; pass < 2; ++pass) {
    const int kind = pass == 0 ? SWA_KV_INT8 : SWA_KV_INT8_DITHER;
    /* c8[0]: decode_step_int8; c8[1]: kv_append + the decode; c8[2]: decode_step_int8_static (no workspace) */
    swa_cache c8[3];
    void *ws8[3];
    float *dout8[3], *dcm8[3];
    for (int t = 0; t < 3; ++t) {
      swa_cache *x = &c8[t];
      memset(x, 0, sizeof *x);
      x->kind = kind; x->B = B; x->H = H; x->D = D8; x->W = W8; x->layout = SWA_LAYOUT_RING;
      CHECK_HIP(hipMalloc(&x->k, (size_t)B * H * W8 * D8));
      CHECK_HIP(hipMalloc(&x->v, (size_t)B * H * W8 * D8));
      CHECK_HIP(hipMalloc((void **)&x->k_scale, (size_t)B * H * (W8 / 16) * 4));
      CHECK_HIP(hipMalloc((void **)&x->v_scale, (size_t)B * H * (W8 / 16) * 4));
      if (kind == SWA_KV_INT8) {
        CHECK_HIP(hipMalloc((void **)&x->witness, (size_t)B * H * W8 * (D8 / 8) * 2));
      } else {
        x->request_id = drid;
        x->layer = 3;
      }
      CHECK_HIP(hipMalloc(&x->k_stage, (size_t)B * H * 16 * D8 * 2));
      CHECK_HIP(hipMalloc(&x->v_stage, (size_t)B * H * 16 * D8 * 2));
      CHECK_HIP(hipMalloc((void **)&x->pos, (size_t)B * W8 * 4));
      CHECK_HIP(hipMalloc((void **)&x->next_position, (size_t)B * 4));
      CHECK_HIP(hipMalloc((void **)&x->step_sync, (size_t)B * 64 * 4)); /* fused-step counters */
      CHECK_SWA(swa_cache_reset(x, NULL));                                /* zeroes them too */
      const size_t wsb = swa_workspace_bytes(x);
      CHECK_HIP(hipMalloc(&ws8[t], wsb > 16 ? wsb : 16));
      CHECK_HIP(hipMalloc((void **)&dout8[t], (size_t)B * H * D8 * 4));
      CHECK_HIP(hipMalloc((void **)&dcm8[t], (size_t)B * H * 4));
    }
    /* token j of every sequence, one step at a time; the rows are [B][H][1][D] */
    for (int j = 0; j < T8; ++j) {
      for (int bh = 0; bh < B * H; ++bh) {
        memcpy(kt + (size_t)bh * D8, k8 + ((size_t)bh * T8 + j) * D8, D8 * 2);
        memcpy(vt + (size_t)bh * D8, v8 + ((size_t)bh * T8 + j) * D8, D8 * 2);
      }
      CHECK_HIP(hipMemcpy(dkt, kt, (size_t)B * H * D8 * 2, hipMemcpyHostToDevice));
      CHECK_HIP(hipMemcpy(dvt, vt, (size_t)B * H * D8 * 2, hipMemcpyHostToDevice));
      const float delta = kind == SWA_KV_INT8 ? 1.0f : 1e-3f;
      CHECK_SWA(decode_step_int8(&c8[0], dkt, dvt, dq8, dout8[0], dcm8[0], NULL, NULL, 0.2f, delta, ws8[0],
                                 swa_workspace_bytes(&c8[0]), NULL));
      CHECK_SWA(decode_step_int8_static(&c8[2], dkt, dvt, dq8, dout8[2], dcm8[2], NULL, NULL, 0.2f, delta, NULL));
      CHECK_SWA(kv_append(&c8[1], dkt, dvt, 1, NULL));
      if (kind == SWA_KV_INT8)
        CHECK_SWA(decode_attn_int8_witness(&c8[1], dq8, dout8[1], dcm8[1], NULL, ws8[1],
                                           swa_workspace_bytes(&c8[1]), NULL));
      else
        CHECK_SWA(decode_attn_int8_dither(&c8[1], dq8, dout8[1], dcm8[1], NULL, NULL, 0.2f, delta, ws8[1],
                                          swa_workspace_bytes(&c8[1]), NULL));
      CHECK_HIP(hipMemcpy(o0, dout8[0], (size_t)B * H * D8 * 4, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(o1, dout8[1], (size_t)B * H * D8 * 4, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(cm0, dcm8[0], (size_t)B * H * 4, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(cm1, dcm8[1], (size_t)B * H * 4, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(o2, dout8[2], (size_t)B * H * D8 * 4, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(cm2, dcm8[2], (size_t)B * H * 4, hipMemcpyDeviceToHost));
      if (memcmp(o0, o1, (size_t)B * H * D8 * 4) != 0 || memcmp(cm0, cm1, (size_t)B * H * 4) != 0) ++mism[pass];
      if (memcmp(o0, o2, (size_t)B * H * D8 * 4) != 0 || memcmp(cm0, cm2, (size_t)B * H * 4) != 0)
        ++mism_static[pass];
    }
    for (int bh = 0; bh < B * H; ++bh)
      for (int d = 0; d < D8; ++d) {
        double mean = 0.0;
        for (int j = 0; j < T8; ++j) mean += from_bf16(v8[((size_t)bh * T8 + j) * D8 + d]);
        mean /= T8;
        const double err = fabs(o0[(size_t)bh * D8 + d] - mean);
        if (err > worst8[pass]) worst8[pass] = err;
      }
    /* Witness kind: the values are exact multiples of their scale, so the output is the exact mean.  Dithered
     * kind: each value reads back s*(code - u), within s/2 = 1/32 of the input, and the keys read back within
     * 1/254 of 1, so the weights stay uniform to within a fraction of a percent. */
    if (mism[pass] || mism_static[pass] || worst8[pass] > (kind == SWA_KV_INT8 ? 2e-3 : 0.05)) ++failures;
    int32_t np8[2];
    CHECK_HIP(hipMemcpy(np8, c8[0].next_position, (size_t)B * 4, hipMemcpyDeviceToHost));
    if (np8[0] != T8 || np8[1] != T8) ++failures;
    for (int t = 0; t < 3; ++t) {
      hipFree(c8[t].k); hipFree(c8[t].v); hipFree(c8[t].k_scale); hipFree(c8[t].v_scale);
      if (c8[t].witness) hipFree(c8[t].witness);
      hipFree(c8[t].k_stage); hipFree(c8[t].v_stage); hipFree(c8[t].pos); hipFree(c8[t].next_position);
      hipFree(c8[t].step_sync); hipFree(ws8[t]); hipFree(dout8[t]); hipFree(dcm8[t]);
    }
  }

  printf("swa_example %s: one-token rows exact, identical-key mean max err %.3g, violations %d; "
         "int8 fused step == append+decode on %d steps (%d mismatches; static-scratch step %d), exact-value mean "
         "max err %.3g; dithered int8 fused step == append+decode (%d mismatches; static-scratch step %d), mean max "
         "err %.3g\n",
         failures ? "FAILED" : "ok", worst, viol, T8, mism[0], mism_static[0], worst8[0], mism[1], mism_static[1],
         worst8[1]);
  hipFree(dq8); hipFree(dkt); hipFree(dvt); hipFree(drid);
  free(k8); free(v8); free(kt); free(vt); free(o0); free(o1); free(o2);
  hipFree(c.k); hipFree(c.v); hipFree(c.pos); hipFree(c.next_position);
  hipFree(dk); hipFree(dv); hipFree(dq); hipFree(dout); hipFree(dviol); hipFree(ws); hipFree(dk1); hipFree(dv1);
  free(hk); free(hv); free(hq); free(out); free(k1); free(v1);
  return failures ? 1 : 0;
}
