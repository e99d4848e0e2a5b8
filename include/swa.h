/*
 * swa.h -- C ABI of the sliding-window ring-buffer KV cache and its decode
 * step, built as hand-written HIP for AMD gfx950 (MI355X).
 *
 * Pages cited, by title (sections as named on each page):
 *  [Lean-SWA]     "用Lean4形式化验证滑动窗口KV Cache的正确性"
 *  [Prefix-Reuse] "LLM 機制實驗（五）：改了歷史，能否只重算變化的後綴？"
 *  [KV-Loop]      "【AI 工业核题 D4】KV Cache 自回归生成推理（增量更新与状态拼接）"
 *  [WitCert]      "WitCert：运行时误差仪表盘，把崩溃的KV量化从22.8拉回79.7"
 *
 * The cache follows the record of [Prefix-Reuse] (section 哪些東西必須一起裁剪):
 * keys, values, the absolute position of every stored row, and
 * next_position, the position the next token receives.  Its physical form is
 * the fixed array of W slots of [Lean-SWA] §3.4: the token at absolute
 * position p lives in slot p mod W and overwrites the oldest.  The decode
 * query of step t attends to exactly the positions [t-len+1, t],
 * len = min(W, t+1) ([Lean-SWA] §2.1 window and causal masks; §2.4 goal 3).
 *
 * Conventions shared by every entry point
 * - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *   never allocates, frees or synchronizes; every call only enqueues kernels
 *   on `stream` (a hipStream_t; NULL = the default stream) and returns.
 * - Layouts are dense row-major, innermost dimension last, as written next
 *   to each field.  K/V, q, out, staging and workspace pointers must be
 *   16-byte aligned.
 * - Return value: SWA_OK (0) or a negative SWA_E* code for a condition the
 *   host can check (bad sizes, NULL, misalignment, unsupported shape, small
 *   workspace, launch failure).  On error nothing has been enqueued.
 *   Device-side preconditions (next_position >= 0, next_position + T <
 *   2^31) are not checked on the hot path; swa_validate checks the cache.
 * - Positions are 0-based int32.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SWA_OK = 0,
  SWA_EINVAL = -1,       /* B, H, W < 1, T < 1, D not in {16, 32, 64, 128, 256},
                            W*D*elem >= 2^32, unknown layout, or W not a multiple of 16
                            for INT8 kinds or PAGED */
  SWA_ENULL = -2,        /* a required pointer is NULL */
  SWA_EALIGN = -3,       /* a K/V/q/out/staging/workspace pointer is not 16-byte aligned */
  SWA_EUNSUPPORTED = -4, /* unknown kind, a kind this entry point does not take, or an
                            INT8 kind with D != 128 */
  SWA_EWORKSPACE = -5,   /* ws_bytes < swa_workspace_bytes(cache) */
  SWA_EHIP = -6          /* a kernel launch failed */
};

enum {
  SWA_KV_BF16 = 0, /* K/V rows bf16; q and new rows bf16 */
  SWA_KV_FP32 = 1, /* K/V rows fp32; q and new rows fp32 */
  SWA_KV_INT8 = 2, /* K/V INT8 codes per 16-token block + fp16 band witness; q, new rows bf16 */
  SWA_KV_INT8_DITHER = 3 /* K/V INT8 codes with subtractive dither, no witness; q, new rows bf16 */
};

/* Physical layout of the rows (the logical cache is the same either way:
 * the window lastWindow(W, history), [Lean-SWA] §3.4 and §6.1).
 * RING:  one contiguous ring of W slots per (b, h).
 * PAGED: pools of 16-token pages shared by all sequences (the paging of
 *        [KV-Loop] §八, pages of 16 tokens); block_table[b][j] names the
 *        page holding ring slots 16j..16j+15 of sequence b.  Needs W % 16 == 0. */
enum { SWA_LAYOUT_RING = 0, SWA_LAYOUT_PAGED = 1 };

/* Cache descriptor.  head_dim D is one of {16, 32, 64, 128, 256} for the
 * BF16 and FP32 kinds ([KV-Loop] §三 takes head_dim as a free parameter).
 * The INT8 kinds take D = 128 only: [WitCert] (section 频带酉性与双层证书)
 * fixes 16 bands of 8 dims and 32 witness bytes per token and head at its
 * head_dim of 128; another D is SWA_EUNSUPPORTED.
 *
 *  RING layout                   PAGED layout (P = num_pages)
 *  k, v       [B][H][W][D]       [P][H][16][D]    bf16 | fp32 | int8 codes
 *  INT8 and INT8_DITHER:
 *  k_scale,   [B][H][W/16] fp32  [P][H] fp32      absmax/127 of the block
 *  v_scale
 *  INT8 only (ignored by INT8_DITHER, may be NULL there):
 *  witness    [B][H][W][D/8]     [P][H][16][D/8]  fp16 bits: band norms of the
 *                                                 key residual, rounded up
 *  INT8_DITHER only (ignored otherwise):
 *  request_id [B] uint64 (device) request id of each sequence, the first
 *                                member of the dither's five-tuple key
 *  layer      uint32             layer id of this cache, another member
 *  Both layouts:
 *  pos            [B][W]  int32  absolute position held by each slot, -1 if
 *                                none (INT8 kinds: position of the committed
 *                                code row)
 *  next_position  [B]     int32  position the next appended token receives
 *  k_stage,v_stage [B][H][16][D] bf16 (INT8 kinds) rows of the incomplete newest
 *                                block, row index = position mod 16
 *  block_table    [B][W/16] int32 (PAGED) page of each 16-slot ring block;
 *                                entries for blocks the sequence uses must be
 *                                in [0, P), and no two sequences may share a
 *                                page; unused entries are ignored
 *  step_sync      [B][64] int32  completion counters of the fused decode step
 *                                (decode_step, decode_step_int8): element
 *                                [b][0] counts the work-groups of sequence b
 *                                that finished the current step; when
 *                                decode_step merges several splits in its
 *                                launch (H <= 63), element [b][1 + h] counts
 *                                the splits of head h that published their
 *                                partials.  The rest of the 256-byte line is
 *                                padding, so sequences never queue on one
 *                                line.  Zero after swa_cache_reset, and every
 *                                fused step leaves it zero.  May be NULL if
 *                                the fused steps are not used (they return
 *                                SWA_ENULL then).
 */
typedef struct swa_cache {
  int32_t kind, B, H, D, W;
  int32_t layout; /* SWA_LAYOUT_RING or SWA_LAYOUT_PAGED */
  void *k, *v;
  int32_t *pos;
  int32_t *next_position;
  float *k_scale, *v_scale;
  uint16_t *witness;
  void *k_stage, *v_stage;
  int32_t *block_table; /* PAGED only */
  int64_t num_pages;    /* PAGED only */
  uint64_t *request_id; /* INT8_DITHER only */
  uint32_t layer;       /* INT8_DITHER only */
  int32_t *step_sync;   /* fused decode steps only */
} swa_cache;

/* Empty the cache: next_position[b] = 0, pos[b][*] = -1 and step_sync[b][*]
 * = 0 (when set) for every b (a RING cache of an INT8 kind also clears its
 * block scales; PAGED pools, which other caches may share, are not touched).  Row contents are left as they are; no
 * slot is visible until written.  Errors: SWA_EINVAL, SWA_ENULL, SWA_EHIP. */
int swa_cache_reset(const swa_cache *c, void *stream);

/* Append T >= 1 tokens per sequence (prefill chunk or one decode token).
 * [Lean-SWA] §2.2 and §3.3-§3.4: write, evict the oldest when over W;
 * [KV-Loop] §三 step 1 (write at the current position); [Prefix-Reuse]
 * (section 哪些東西必須一起裁剪: next_position advances with the rows).
 *  k_new, v_new  [B][H][T][D] in the cache's input dtype (INT8 kinds: bf16).
 * Token j of sequence b gets position p = next_position[b] + j and slot
 * p mod W; pos[b][slot] = p; afterwards next_position[b] += T.  Only the last
 * min(T, W) tokens are stored (the others would be overwritten).
 * INT8 kind ([WitCert], section 频带酉性与双层证书: the
 * write path quantizes and records band norms of the residual): a token first
 * goes to the staging rows; when the block of positions [16m, 16m+16) is
 * complete it is quantized into slots (16m mod W).. with one fp32 absmax/127
 * scale per block and tensor, codes rint(x/s) clamped to +-127, and the key
 * residual's 16 band norms written rounded up to fp16.
 * INT8_DITHER kind ([WitCert], section 频带酉性与双层证书, Tier B: a uniform
 * pseudo-random dither is added before rounding at write time and subtracted
 * at read time; section SGLang 生产级落地: Philox keyed by request, layer,
 * KV head, token and channel): the same blocks and scales, and
 * code = rint(f32(x/s) + u) with u = 1/2 - (m + 1/2)/256, where m is byte
 * c mod 16 of Philox-4x32-10 (Salmon et al., SC 2011) with key
 * (request_id mod 2^32, request_id div 2^32) and counter (position, c / 16,
 * head, layer); the words are taken in order, each little-endian.  Keys and
 * values of one token share u.  request_id must be set.  No witness is
 * written.  T < 1 is SWA_EINVAL. */
int kv_append(const swa_cache *c, const void *k_new, const void *v_new, int32_t T, void *stream);

/* Decode attention for one query per sequence over the last min(W, n) tokens,
 * n = next_position[b] (append first, then attend: [KV-Loop] §三 steps 2-4;
 * scores q.k/sqrt(D), max-subtracted softmax, weighted V).  BF16 and FP32
 * kinds.  Split over the context with an online softmax; a second kernel
 * merges the splits of each (b, h).
 *  q    [B][H][D]  cache input dtype
 *  out  [B][H][D]  fp32; a sequence with n = 0 gets zeros
 *  ws   device workspace of ws_bytes >= swa_workspace_bytes(c) holding the
 *       split partials; its contents need no initialization, and no call
 *       leaves state in it that a later call reads.  One workspace may serve
 *       any caches (of any shape) as long as it is large enough for each and
 *       the calls that use it are ordered on one stream. */
int decode_attn(const swa_cache *c, const void *q, float *out, void *ws, size_t ws_bytes,
                void *stream);

/* INT8 decode attention with the fused witness bound ([WitCert], section
 * 频带酉性与双层证书: |q.r_t|/sqrt(d) <= c_t = (1/sqrt(d)) sum_b ||q_b|| w_{t,b};
 * section SGLang 生产级落地: per-block scales fold into per-token scalars).
 * Visible tokens in committed blocks are read as scale*code, the newest
 * n mod 16 tokens exactly from the staging rows (their c_t is 0).
 *  q      [B][H][D] bf16
 *  out    [B][H][D] fp32
 *  cmax   [B][H]    fp32: max of c_t over the visible tokens (0 if none are
 *                   quantized), times (1 + 2^-12) to cover float32 rounding
 *  c_all  NULL, or [B][H][W] fp32: c_t of the visible token in each slot,
 *         0 for slots with no visible quantized token (verification only)
 *  ws, ws_bytes: as for decode_attn. */
int decode_attn_int8_witness(const swa_cache *c, const void *q, float *out, float *cmax,
                             float *c_all, void *ws, size_t ws_bytes, void *stream);

/* decode_attn_int8_witness plus a total-variation bound and a gate flag
 * ([WitCert], section 为什么在线监控 KV 误差如此困难: prior work bounds the TV of
 * the attention weights by tanh of the largest logit error; section SGLang
 * 生产级落地: the decode pass emits a per-step TV bound for the gate).
 * Every visible logit moved by at most cmax, so
 *  tv    [B][H] fp32: tanh(cmax/2), an upper bound on the total variation
 *        between the attention weights over the exact keys and over the
 *        quantized keys (tight in the worst case over logit perturbations
 *        of that size; tanh(cmax) would also be sound, and looser)
 *  gate  NULL, or [B][H] int32: 1 where tv > tau, else 0 (tau = 0.2 marks the
 *        pages' danger threshold); gate needs tv.
 * tv = NULL makes this identical to decode_attn_int8_witness.  Errors as
 * there, plus SWA_ENULL for gate without tv and SWA_EINVAL for a NaN tau. */
int decode_attn_int8_witness_tv(const swa_cache *c, const void *q, float *out, float *cmax, float *tv,
                                int32_t *gate, float tau, float *c_all, void *ws, size_t ws_bytes,
                                void *stream);

/* Tier B decode ([WitCert], section 频带酉性与双层证书: with dithered INT8 the
 * residual is uniform and independent of the data, so a sub-Gaussian
 * concentration bound with a failure budget replaces the stored witness).
 * INT8_DITHER kind.  Committed tokens are read as s * (code - u), with u
 * regenerated from the same Philox stream; the newest n mod 16 tokens are
 * exact.  For every visible quantized token j the logit error e_j =
 * q.(k^_j - k_j)/sqrt(D) is, over the dither, a sum of independent terms: per
 * channel the residual is uniform on a 256-point grid (variance proxy 1/12,
 * mean within beta = 2^-9 + 2^-16 of zero in code units).  A union bound over
 * the n_q visible quantized tokens gives, with probability >= 1 - delta,
 *   max_j |e_j| <= cert = (S/sqrt(D)) (||q||_2 sqrt(ln(2 n_q/delta)/6)
 *                                      + ||q||_1 beta),
 * S the largest key scale among those tokens (cert = 0 when n_q = 0).
 *  q      [B][H][D] bf16
 *  out    [B][H][D] fp32
 *  cert   [B][H]    fp32: the bound above, times (1 + 2^-12) for float32
 *                   rounding
 *  tv     NULL, or [B][H] fp32: tanh(cert/2), the TV bound on the attention
 *         weights that holds together with cert
 *  gate   NULL, or [B][H] int32: 1 where tv > tau (needs tv)
 *  delta  failure budget of one (sequence, head) query, in (0, 1]; a
 *         request's budget is split over its steps, layers and heads by the
 *         caller (union bound)
 *  ws, ws_bytes: as for decode_attn.
 * Errors: descriptor errors, SWA_EUNSUPPORTED for another kind, SWA_ENULL,
 * SWA_EALIGN, SWA_EINVAL for delta outside (0, 1] or a NaN tau,
 * SWA_EWORKSPACE, SWA_EHIP. */
int decode_attn_int8_dither(const swa_cache *c, const void *q, float *out, float *cert, float *tv,
                            int32_t *gate, float tau, float delta, void *ws, size_t ws_bytes, void *stream);

/* One decode step in one call for the BF16 and FP32 kinds: kv_append of
 * one token per sequence, then decode_attn ([KV-Loop] §三: write at the
 * current position, then attend).  The result is bit for bit that of
 * kv_append(c, k_new, v_new, 1) followed by decode_attn.  The append and
 * the decode are one kernel launch: the work-group whose split holds slot
 * next_position mod W of a (b, h) writes the token's rows there, then every
 * work-group decodes its split; the last work-group of a sequence to finish,
 * counted in the cache's step_sync, advances next_position.  With several
 * splits per (b, h) and H <= 63, the last split of each (b, h) to finish,
 * counted in step_sync[b][1 + h], merges the splits in the same launch;
 * with more heads a merge launch follows, as in decode_attn.
 *  k_new, v_new  [B][H][1][D] in the cache's input dtype
 *  q, out, ws    as for decode_attn
 * Errors: descriptor errors, SWA_EUNSUPPORTED for an INT8 kind, SWA_ENULL
 * (also for a NULL step_sync), SWA_EALIGN, SWA_EWORKSPACE, SWA_EHIP. */
int decode_step(const swa_cache *c, const void *k_new, const void *v_new, const void *q, float *out, void *ws,
                size_t ws_bytes, void *stream);

/* One decode step in one call: kv_append of one token per sequence, then
 * the INT8 decode of that sequence's query ([KV-Loop] §三: write at the
 * current position, then attend; [WitCert], section SGLang 生产级落地: one
 * fused pass per step).  INT8 kinds only.  The result is bit for bit that
 * of kv_append(c, k_new, v_new, 1) followed by decode_attn_int8_witness_tv
 * (INT8) or decode_attn_int8_dither (INT8_DITHER) with the same arguments.
 * The append and the decode are one kernel launch: for each (b, h) one
 * work-group appends the token (quantizing the block it completes, in the
 * work-group whose split decodes that block), then every work-group decodes
 * its split; the last work-group of a sequence to finish, counted in the
 * cache's step_sync, advances next_position.  A plan with several splits per
 * (b, h) adds the merge launch, as the decode entry points do.
 *  k_new, v_new  [B][H][1][D] bf16
 *  q, out, cmax, tv, gate, tau  as for decode_attn_int8_witness_tv; cmax is
 *                the certificate for INT8_DITHER
 *  delta         INT8_DITHER failure budget, in (0, 1]; ignored for INT8
 *  ws            as for decode_attn
 * Errors: descriptor errors, SWA_EUNSUPPORTED for a non-INT8 kind,
 * SWA_ENULL (also for a NULL step_sync), SWA_EALIGN, SWA_EINVAL (NaN tau;
 * delta outside (0, 1] for INT8_DITHER), SWA_EWORKSPACE, SWA_EHIP. */
int decode_step_int8(const swa_cache *c, const void *k_new, const void *v_new, const void *q, float *out,
                     float *cmax, float *tv, int32_t *gate, float tau, float delta, void *ws, size_t ws_bytes,
                     void *stream);

/* decode_step_int8 for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks and results (bit for bit) as
 * decode_step_int8, without ws and ws_bytes: the split partials live in a
 * static device array of the library, 16 MiB per GPU, held until the
 * process ends.  Its device address is looked up on the first call on each
 * device (make that first call outside graph capture; later calls can be
 * captured).  The call allocates nothing and needs nothing cleared: the merge
 * reads only partials written in the same call.  All calls on one GPU share
 * that GPU's array, so calls that overlap on one GPU (on different streams,
 * or from several threads without ordering) race and give wrong results;
 * order them on one stream.
 * Errors: those of decode_step_int8, and SWA_EWORKSPACE when the shape
 * needs more than 16 MiB of partials (swa_workspace_bytes(c) > 16 MiB). */
int decode_step_int8_static(const swa_cache *c, const void *k_new, const void *v_new, const void *q, float *out,
                            float *cmax, float *tv, int32_t *gate, float tau, float delta, void *stream);

/* Workspace bytes the decode entry points need for this cache shape: the
 * split partials, B*H*nsplit*(D+4) floats, padded to 256 bytes (nsplit is
 * the largest number of context splits any (b, h) can need under the
 * library's split plan).  0 for an invalid descriptor. */
size_t swa_workspace_bytes(const swa_cache *c);

/* Zero-fill a workspace (optional: the decode entry points overwrite every
 * partial they read).  Errors: SWA_ENULL, SWA_EALIGN, SWA_EHIP. */
int swa_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Prefix reuse ([Prefix-Reuse], sections 哪些東西必須一起裁剪 and
 * 為什麼滑窗部分命中必須回退): truncate sequence b to its first cut[b] tokens,
 * so the next appended token gets position cut[b] -- when that is exact.
 * It is exact iff every row of the shorter history's window is still
 * stored: 0 <= cut <= n and (n <= W, or cut == n, or cut == 0); an INT8 (either kind) cache
 * also needs cut % 16 == 0 or cut >= 16*(n/16) (committed blocks keep only
 * codes).  Exact: slots holding positions >= cut become empty (pos = -1)
 * and next_position[b] = cut.  Otherwise sequence b is left unchanged and the
 * caller must recompute it.
 *  cut  [B] device int32
 *  ok   NULL, or [B] device int32: 1 truncated (or nothing to do), 0 fall back
 * Errors: SWA_ENULL, SWA_EALIGN, descriptor errors, SWA_EHIP. */
int kv_truncate(const swa_cache *c, const int32_t *cut, int32_t *ok, void *stream);

/* Debug check of the position invariant ([Lean-SWA] §3.2 PositionInvariant,
 * §6.3 the invariant as a runtime assertion): adds to *violations (device
 * int32, caller zeroes it) the number of slots whose pos differs from the
 * newest position p < n (INT8 kinds: p < 16*(n/16)) with p mod W == slot, or -1;
 * PAGED: also each live slot whose block_table entry is outside [0, P). */
int swa_validate(const swa_cache *c, int32_t *violations, void *stream);

/* Static text for a status code. */
const char *swa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
