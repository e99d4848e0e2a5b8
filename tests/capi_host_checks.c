/*
 * Host-side checks of the C ABI under AddressSanitizer and UBSan (built by
 * tests/test_capi_sanitizers.py, host code only).  Every call below is
 * rejected by the library's own argument checks before any launch, so the
 * program needs no GPU: it exercises the descriptor checks, the split
 * plan and the workspace arithmetic at their limits, and the status
 * strings.  Prints "host checks ok" and returns 0.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "swa.h"

static int failures = 0;
#define EXPECT(call, want)                                                                         \
  do {                                                                                             \
    int got_ = (call);                                                                             \
    if (got_ != (want)) {                                                                          \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (want)); \
      ++failures;                                                                                  \
    }                                                                                              \
  } while (0)

static swa_cache desc(int kind, int B, int H, int D, int W, int layout) {
  swa_cache c;
  memset(&c, 0, sizeof c);
  c.kind = kind; c.B = B; c.H = H; c.D = D; c.W = W; c.layout = layout;
  c.k = (void *)0x10000; c.v = (void *)0x20000;
  c.pos = (int32_t *)0x30000; c.next_position = (int32_t *)0x40000;
  c.k_scale = (float *)0x50000; c.v_scale = (float *)0x60000;
  c.witness = (uint16_t *)0x70000; c.k_stage = (void *)0x80000; c.v_stage = (void *)0x90000;
  c.block_table = (int32_t *)0xC0000; c.num_pages = 8;
  c.request_id = (uint64_t *)0xD0000; c.layer = 3;
  c.step_sync = (int32_t *)0xE0000;
  return c;
}

int main(void) {
  void *A = (void *)0xA0000, *ODD = (void *)0xA0004, *ws = (void *)0xB0000;
  float *F = (float *)0xA0000;
  int32_t *I = (int32_t *)0xA0000;
  const int kinds[4] = {SWA_KV_BF16, SWA_KV_FP32, SWA_KV_INT8, SWA_KV_INT8_DITHER};
  const int dims[4] = {128, 16, 128, 128};
  const int all_dims[5] = {16, 32, 64, 128, 256};

  for (int s = -8; s <= 1; ++s) {
    const char *t = swa_status_string(s);
    if (t == NULL || t[0] == 0) ++failures;
  }
  EXPECT(kv_append(NULL, A, A, 1, NULL), SWA_ENULL);

  for (int i = 0; i < 4; ++i) {
    for (int layout = 0; layout < 2; ++layout) {
      swa_cache c = desc(kinds[i], 2, 4, dims[i], 64, layout);
      const size_t need = swa_workspace_bytes(&c);
      if (need == 0 || need % 256 != 0) {
        fprintf(stderr, "kind %d layout %d: workspace %zu\n", kinds[i], layout, need);
        ++failures;
      }
      /* rejected before launching anything */
      EXPECT(kv_append(&c, ODD, A, 1, NULL), SWA_EALIGN);
      EXPECT(kv_append(&c, NULL, A, 1, NULL), SWA_ENULL);
      EXPECT(kv_append(&c, A, A, -3, NULL), SWA_EINVAL);
      EXPECT(kv_append(&c, A, A, 0, NULL), SWA_EINVAL);
      EXPECT(decode_attn(&c, A, F, ws, need - 1, NULL), i < 2 ? SWA_EWORKSPACE : SWA_EUNSUPPORTED);
      EXPECT(decode_attn_int8_witness(&c, A, F, NULL, NULL, ws, need, NULL),
             kinds[i] == SWA_KV_INT8 ? SWA_ENULL : SWA_EUNSUPPORTED);
      EXPECT(decode_attn_int8_witness_tv(&c, A, F, F, NULL, I, 0.2f, NULL, ws, need, NULL),
             kinds[i] == SWA_KV_INT8 ? SWA_ENULL : SWA_EUNSUPPORTED);
      EXPECT(decode_attn_int8_dither(&c, A, F, F, F, I, 0.2f, 0.0f, ws, need, NULL),
             kinds[i] == SWA_KV_INT8_DITHER ? SWA_EINVAL : SWA_EUNSUPPORTED);
      EXPECT(decode_step_int8(&c, A, A, A, F, F, NULL, NULL, 0.2f, 0.1f, ws, need - 1, NULL),
             i >= 2 ? SWA_EWORKSPACE : SWA_EUNSUPPORTED);
      EXPECT(decode_step(&c, A, A, A, F, ws, need - 1, NULL), i < 2 ? SWA_EWORKSPACE : SWA_EUNSUPPORTED);
      EXPECT(decode_step_int8_static(&c, NULL, A, A, F, F, NULL, NULL, 0.2f, 0.1f, NULL),
             i >= 2 ? SWA_ENULL : SWA_EUNSUPPORTED); /* rejected before any HIP call */
      swa_cache ns = c;
      ns.step_sync = NULL; /* the fused steps need the completion counters */
      EXPECT(decode_step(&ns, A, A, A, F, ws, need, NULL), i < 2 ? SWA_ENULL : SWA_EUNSUPPORTED);
      EXPECT(decode_step_int8(&ns, A, A, A, F, F, NULL, NULL, 0.2f, 0.1f, ws, need, NULL),
             i >= 2 ? SWA_ENULL : SWA_EUNSUPPORTED);
      EXPECT(kv_append(&ns, NULL, A, 1, NULL), SWA_ENULL); /* the other calls do not */
      ns.step_sync = (int32_t *)0xE0002;
      EXPECT(kv_append(&ns, NULL, A, 1, NULL), SWA_EALIGN);
      EXPECT(kv_truncate(&c, NULL, NULL, NULL), SWA_ENULL);
      EXPECT(kv_truncate(&c, (const int32_t *)0xA0002, NULL, NULL), SWA_EALIGN);
      EXPECT(swa_validate(&c, NULL, NULL), SWA_ENULL);
    }
  }

  /* head dims: every kind takes {16, 32, 64, 128, 256}, except that the
     INT8 kinds take 128 only; anything else is invalid.  A valid
     descriptor reaches the argument checks (k_new NULL). */
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j) {
      swa_cache d = desc(kinds[i], 2, 4, all_dims[j], 64, 0);
      EXPECT(kv_append(&d, NULL, A, 1, NULL), i < 2 || all_dims[j] == 128 ? SWA_ENULL : SWA_EUNSUPPORTED);
    }
    swa_cache d = desc(kinds[i], 2, 4, 48, 64, 0);
    EXPECT(kv_append(&d, NULL, A, 1, NULL), SWA_EINVAL);
    d = desc(kinds[i], 2, 4, 512, 64, 0);
    EXPECT(kv_append(&d, NULL, A, 1, NULL), SWA_EINVAL);
  }

  /* descriptor limits */
  swa_cache c = desc(SWA_KV_BF16, 65536, 1, 128, 64, 0);
  EXPECT(kv_append(&c, A, A, 1, NULL), SWA_EINVAL);            /* B above the grid limit */
  c = desc(SWA_KV_BF16, 1, 65536, 128, 64, 0);
  EXPECT(kv_append(&c, A, A, 1, NULL), SWA_EINVAL);            /* H above the grid limit */
  c = desc(SWA_KV_BF16, 1, 1, 256, 8388608, 0);
  EXPECT(kv_append(&c, NULL, A, 1, NULL), SWA_EINVAL);         /* one (b, h) region reaches 4 GiB */
  c = desc(SWA_KV_FP32, 1, 1, 256, 4194303, 0);
  EXPECT(kv_append(&c, NULL, A, 1, NULL), SWA_ENULL);          /* largest fp32 D=256 window below 4 GiB */
  c.W = 4194304;
  EXPECT(kv_append(&c, NULL, A, 1, NULL), SWA_EINVAL);
  c = desc(SWA_KV_INT8, 1, 1, 128, 33554416, 0);
  EXPECT(kv_append(&c, NULL, A, 1, NULL), SWA_ENULL);          /* largest INT8 window below 4 GiB */
  if (swa_workspace_bytes(&c) == 0) ++failures;
  c = desc(SWA_KV_BF16, 65535, 65535, 128, 16, 0);
  if (swa_workspace_bytes(&c) < (size_t)65535 * 65535 * (128 + 4) * 4) ++failures;  /* no 32-bit overflow */
  c = desc(SWA_KV_INT8, 65535, 65535, 128, 2048, 1);
  c.num_pages = (int64_t)1 << 40;
  EXPECT(kv_append(&c, NULL, A, 1, NULL), SWA_ENULL);
  if (swa_workspace_bytes(&c) == 0) ++failures;
  c = desc(7, 1, 1, 128, 64, 0);
  EXPECT(kv_append(&c, A, A, 1, NULL), SWA_EUNSUPPORTED);
  c = desc(SWA_KV_INT8_DITHER, 1, 1, 128, 64, 0);
  c.request_id = NULL;
  EXPECT(kv_append(&c, A, A, 1, NULL), SWA_ENULL);
  c = desc(SWA_KV_BF16, 2, 2, 128, 64, 1);
  c.num_pages = 0;
  EXPECT(kv_append(&c, A, A, 1, NULL), SWA_EINVAL);
  EXPECT(swa_workspace_init(NULL, 16, NULL), SWA_ENULL);
  EXPECT(swa_workspace_init(ODD, 16, NULL), SWA_EALIGN);
  EXPECT(swa_workspace_init(A, 0, NULL), SWA_OK);

  if (failures) {
    printf("host checks FAILED (%d)\n", failures);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
