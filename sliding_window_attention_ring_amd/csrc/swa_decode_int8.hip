// INT8 decode attention with the fused witness bound (head_dim 128).
//
// Page "WitCert：运行时误差仪表盘，把崩溃的KV量化从22.8拉回79.7":
// * section 频带酉性与双层证书: the logit error of a token with key residual
//   r_t is |q.r_t|/sqrt(d) <= c_t = (1/sqrt(d)) sum_b ||q_b|| w_{t,b}, with
//   w_{t,b} the stored band norms (16 bands of 8 dims, fp16);
// * section SGLang 生产级落地: with one scale per block the scale is a scalar
//   for every token of the block, so the key scale multiplies the finished
//   dot product and the value scale multiplies the softmax weight -- no
//   per-element dequantization multiply.
//
// Visible tokens for the query of step t = n-1 (n = next_position, len =
// min(W, n)) are the positions [n-len, n-1].  Those below 16*(n/16) sit in
// committed blocks of the ring: blocks k0..nb-1 with k0 = (n-len)/16, block k
// in slots [16k mod W, +16); in block k0 the positions below n-len are masked.
// The newest n mod 16 tokens are exact bf16 rows in the staging area and
// carry c_t = 0; the last stage (finish_int8) folds them in.
//
// Layout of the work: grid (split, h, b) (paged pools: (split, b, h), see
// grid_head below), NW waves; a split owns `cb`
// consecutive blocks; a wave takes UB blocks per iteration.  When the plan
// has one split per (b, h) (FINAL), the work-group runs the last stage
// itself.  Otherwise every split writes a partial (m, l, cmax, acc[D]) and
// a second kernel merges the splits of each (b, h) -- the kernel boundary
// makes the partials visible across the XCDs' L2 caches without any
// device-wide fence.  Per block a
// lane loads 2x16 B of key codes and 2x16 B of value codes (8 lanes per
// 128-byte row, rows g and g+8) and 8 B of witness (4 lanes per token).
//
// Tier B (DITHER; same page, section 频带酉性与双层证书, second tier): the
// codes carry a subtractive dither u = 1/2 - (m + 1/2)/256 that is
// regenerated here from the Philox stream the write path used (key = the
// request id, counter = (position, channel / 16, head, layer); section SGLang
// 生产级落地 for the five-tuple).  A token is read as s * (code - u), with no
// witness.  The lane that holds dims [16*(lane%8), +16) of rows g and g+8
// needs exactly one Philox block per row, shared by the key and the value.
// With t = 256 code + m, a signed 16-bit integer that one byte permute
// builds from the code byte and the dither byte as Philox returns it (two
// elements per permute), code - u = (t - 127.5)/256.  So the key dot is
// (1/256) sum q t - (127.5/256) sum q, and the value sum gets (p s_V/256) t
// per element, with -(127.5/256) times the running weight sum added once
// at the end.  The bound is probabilistic: with probability at
// least 1 - delta every visible logit error is at most
// cert = (S / sqrt(D)) (||q||_2 sqrt(ln(2 n_q / delta) / 6) + ||q||_1 beta),
// where S is the largest key scale of a visible block and n_q the number of
// visible quantized tokens.  Per channel the residual is uniform on 256 grid
// points: variance proxy 1/12, |mean| <= beta = 2^-9 + 2^-16 in code
// units.  A union bound over the n_q tokens gives the ln term.  The kernel
// tracks S as its running maximum.
#include <type_traits>

#include "swa_commit.h"
#include "swa_device.h"
#include "swa_launch.h"

namespace swa {
namespace {

// Waves per work-group and 16-token blocks per wave iteration.
#ifndef SWA_INT8_NW
#define SWA_INT8_NW 4
#endif
#ifndef SWA_INT8_UB
#define SWA_INT8_UB 2
#endif

constexpr int D = 128;
constexpr int PF = D + 4;          // m, l, cmax, pad, acc[D]
constexpr float kNegBig = -1e30f;
// Relative pad on the reported bound: covers the float32 rounding of the
// band norms of q, the 16-term sum and 1/sqrt(D) (each well below 2^-20).
constexpr float kBoundPad = 1.0f + 0x1p-12f;

// One 16-token block in flight: codes, witness and the two block scales
// (loaded with the codes so their latency is hidden by the prefetch too).
struct Blk {
  uint4 k0, k1, v0, v1;
  uint2 w;
  float sk, sv;
};

// Dot product of this lane's 16 query dims with 16 int8 key codes, in
// base-2 logit units before the block scale.  Each code converts with one
// sign-extending byte convert; the query is pre-scaled by log2(e)/sqrt(D).
struct KeyDot {
  float qf[16];
  __device__ __forceinline__ void init(const uint4* qv, float qscale) {
    float t8[8];
    unpack8(qv[0], t8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = t8[e] * qscale;
    unpack8(qv[1], t8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[8 + e] = t8[e] * qscale;
  }
  __device__ __forceinline__ float dot(const uint4 c) const {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) d = fmaf(qf[4 * i + j], s8(cw[i], j), d);
    return d;
  }
};

// Tier B element values t = 256 code + m for the 4 codes of word cw and
// the 4 dither bytes of word mw: bytes (m0, c0, m1, c1) and (m2, c2, m3, c3)
// as two signed 16-bit halves each (a byte permute takes bytes 0-3 from its
// second operand and 4-7 from its first).
__device__ __forceinline__ void dither_t(uint32_t cw, uint32_t mw, float (&t)[4]) {
  const uint32_t lo = __builtin_amdgcn_perm(cw, mw, 0x05010400u);
  const uint32_t hi = __builtin_amdgcn_perm(cw, mw, 0x07030602u);
  t[0] = s16lo(lo); t[1] = s16hi(lo);
  t[2] = s16lo(hi); t[3] = s16hi(hi);
}

// Tier B key dot of 16 dims: sum q (code - u) = (1/256) sum q t -
// (127.5/256) sum q, the query pre-scaled by log2(e)/sqrt(D) (q/256 is
// exact).
struct DitherKeyDot {
  float qt[16], qc;
  __device__ __forceinline__ void init(const uint4* qv, float qscale) {
    float t8[8], qf[16];
    unpack8(qv[0], t8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = t8[e] * qscale;
    unpack8(qv[1], t8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[8 + e] = t8[e] * qscale;
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      qt[e] = qf[e] * (1.0f / 256.0f);
      sum += qf[e];
    }
    qc = sum * (-127.5f / 256.0f);
  }
  // m: the dither bytes of the row
  __device__ __forceinline__ float dot(const uint4 c, const uint4 m) const {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    const uint32_t mw[4] = {m.x, m.y, m.z, m.w};
    float d = qc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float t[4];
      dither_t(cw[i], mw[i], t);
#pragma unroll
      for (int j = 0; j < 4; ++j) d = fmaf(qt[4 * i + j], t[j], d);
    }
    return d;
  }
};

// Bias bound of the dither residual in code units (grid half-step plus the
// float32 roundings that can move the rounding threshold).
constexpr float kDitherBeta = 0x1p-9f + 0x1p-16f;

// Last stage of one (b, h), run by >= 256 threads of a work-group (thread t
// < D owns output dim t and holds the merged M, L, A of the committed
// blocks; CM is their max c_t): fold in the exact staging tokens
// (positions 16*(n/16) .. n-1, row = position mod 16, c_t = 0), normalize,
// and write out, cmax and the optional TV bound and gate.
// Optional epilogue (tv != null): every visible logit moved by at most
// E = cmax, so the attention weights moved by at most tanh(E/2) in total
// variation (page "WitCert", section 为什么在线监控 KV 误差如此困难 gives the
// looser tanh(E) form); gate = tv > tau.
//
// DITHER: CM is the largest key scale S of the visible blocks, and the bound
// written to cmax_out is the Tier B certificate built from S, the query
// norms, n_q and delta (see the top of this file).
// The staging-tail inputs of the last stage, loaded ahead (by the merge
// kernel before the split partials, by a one-split work-group before its
// wave merge) so that their latencies overlap:
// thread t (< 256)'s 8 dims of staged key row t/16 and of q, and for t < D
// the staged values of dim t.  All 16 staging rows are allocated, so the
// loads need no guard (rows at or past the staged count are read but not
// used), which lets them all be in flight at once.
struct StageRows {
  uint4 k, q;
  float v[15];
};

__device__ __forceinline__ void load_stage(StageRows& st, int t, int64_t bh, const uint16_t* kst,
                                           const uint16_t* vst, const uint16_t* q) {
  const int tok = t >> 4, v16 = t & 15;
  if (t < 256) {
    st.k = reinterpret_cast<const uint4*>(kst + (bh * 16 + tok) * D)[v16];
    st.q = reinterpret_cast<const uint4*>(q + bh * D)[v16];
  }
  if (t < D) {
#pragma unroll
    for (int i = 0; i < 15; ++i) st.v[i] = bf16_to_f32(vst[(bh * 16 + i) * D + t]);
  }
}

template <bool DITHER>
__device__ __forceinline__ void finish_int8(int t, int64_t bh, int n, float M, float L, float A, float CM,
                                            float* sm_s, const uint16_t* __restrict__ kst,
                                            const uint16_t* __restrict__ vst, const uint16_t* __restrict__ q,
                                            float* __restrict__ out, float* __restrict__ cmax_out,
                                            float* __restrict__ tv, int32_t* __restrict__ gate, float tau,
                                            int W, float delta, const StageRows* pre = nullptr) {
  const float qscale = kLog2e / sqrtf((float)D);
  const int ns = n - (n / 16) * 16;
  if (ns > 0) {
    // Scores: 16 lanes per staged token, 8 bf16 each (threads 0..255 = 16 tokens).
    const int tok = t >> 4, v16 = t & 15;
    float d = 0.f;
    if (tok < ns) {
      float f[8], qv[8];
      unpack8(pre ? pre->k : reinterpret_cast<const uint4*>(kst + (bh * 16 + tok) * D)[v16], f);
      unpack8(pre ? pre->q : reinterpret_cast<const uint4*>(q + bh * D)[v16], qv);
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qv[e] * qscale, f[e], d);
    }
    d = group_sum<16>(d);
    if (v16 == 0 && tok < 16) sm_s[tok] = tok < ns ? d : -INFINITY;
    __syncthreads();
    if (t < D) {
      float ms = -INFINITY;
      for (int i = 0; i < ns; ++i) ms = fmaxf(ms, sm_s[i]);
      const float Mn = fmaxf(M, ms);
      const float sc = exp2_fast(M - Mn);
      L *= sc;
      A *= sc;
      if (pre) {
#pragma unroll
        for (int i = 0; i < 15; ++i) {
          if (i < ns) {
            const float p = exp2_fast(sm_s[i] - Mn);
            L += p;
            A = fmaf(p, pre->v[i], A);
          }
        }
      } else {
        for (int i = 0; i < ns; ++i) {
          const float p = exp2_fast(sm_s[i] - Mn);
          L += p;
          A = fmaf(p, bf16_to_f32(vst[(bh * 16 + i) * D + t]), A);
        }
      }
    }
  }
  if (t < D) out[bh * D + t] = L > 0.f ? A / L : 0.f;
  if constexpr (DITHER) {
    // ||q||_1 and ||q||_2^2 over the 128 dims: two per lane of the first wave.
    float a1 = 0.f, a2 = 0.f;
    if (t < 64) {
      const float f0 = bf16_to_f32(q[bh * D + t]), f1 = bf16_to_f32(q[bh * D + t + 64]);
      a1 = fabsf(f0) + fabsf(f1);
      a2 = fmaf(f0, f0, f1 * f1);
    }
    a1 = group_sum<64>(a1);
    a2 = group_sum<64>(a2);
    const int len = n < W ? n : W;
    const int nq = (n / 16) * 16 - (n - len);  // visible tokens in committed blocks
    if (nq > 0) {
      const float lg = logf(2.0f * (float)nq) - logf(delta);
      CM *= (sqrtf(a2) * sqrtf(lg * (1.0f / 6.0f)) + a1 * kDitherBeta) / sqrtf((float)D);
    } else {
      CM = 0.f;
    }
  }
  if (t == 0) {
    const float cm = CM * kBoundPad;
    cmax_out[bh] = cm;
    if (tv != nullptr) {
      // tanhf is within a few ulp; the 2^-20 pad keeps the value an upper bound.
      const float bnd = fminf(tanhf(0.5f * cm) * (1.0f + 0x1p-20f), 1.0f);
      tv[bh] = bnd;
      if (gate != nullptr) gate[bh] = bnd > tau ? 1 : 0;
    }
  }
}

// Grid order.  A paged pool keeps the fp32 block scales of every head of a
// page in one [P][H] line.  The hardware hands work-groups to the XCDs in
// turn, so with the grid (split, h, b) the heads of a sequence spread over
// all XCDs and each XCD's L2 fetches every scale line; with (split, b, h)
// all heads of a sequence share one XCD (B a multiple of 8 keeps the XCDs
// evenly loaded) and the line is fetched once.
#ifndef SWA_INT8_PAGED_SEQ_MAJOR
#define SWA_INT8_PAGED_SEQ_MAJOR 1
#endif
#ifndef SWA_INT8_RING_SEQ_MAJOR
#define SWA_INT8_RING_SEQ_MAJOR 0
#endif
template <bool PAGED>
constexpr bool kSeqMajor = PAGED ? SWA_INT8_PAGED_SEQ_MAJOR : SWA_INT8_RING_SEQ_MAJOR;
template <bool PAGED>
__device__ __forceinline__ int grid_head() {
  return kSeqMajor<PAGED> ? (int)blockIdx.z : (int)blockIdx.y;
}
template <bool PAGED>
__device__ __forceinline__ int grid_seq() {
  return kSeqMajor<PAGED> ? (int)blockIdx.y : (int)blockIdx.z;
}
inline dim3 int8_grid(const swa_cache& c, int nsplit) {
  const bool seq_major = c.layout == SWA_LAYOUT_PAGED ? kSeqMajor<true> : kSeqMajor<false>;
  return seq_major ? dim3(nsplit, c.B, c.H) : dim3(nsplit, c.H, c.B);
}

// The decode of one (split, h, b) work-group, called by decode_int8_kernel
// and by the fused step kernel; n is next_position[b] as this decode sees
// it.  APPEND (fused step): block kb_new, unless -1, was committed by this
// work-group in this launch, and its two scales are taken from sk_new /
// sv_new, not from memory -- a scalar-cache line holding them may have been
// filled before the commit (lines are shared across heads).  The pointers
// carry no restrict qualifier because the fused step writes the same
// buffers first.
template <int NW, int UB, bool PAGED, bool FINAL, bool DITHER, bool APPEND>
__device__ __forceinline__ void decode_int8_wg(
    int n, int kb_new, float sk_new, float sv_new, const int8_t* Kc, const int8_t* Vc, const float* ksc,
    const float* vsc, const uint16_t* wit, const int32_t* table, int64_t num_pages, const uint16_t* q,
    float* c_all, float* part, int H, int W, int cb, int nsplit_max, const uint16_t* kst, const uint16_t* vst,
    float* out, float* cmax_out, float* tv, int32_t* gate, float tau, const uint64_t* req, uint32_t layer,
    float delta) {
  static_assert(NW * 64 >= 256, "the staging fold needs 256 threads");
  __shared__ float sm_m[NW], sm_l[NW], sm_c[NW];
  __shared__ float sm_acc[NW][D];
  __shared__ float sm_s[16];

  const int split = blockIdx.x, h = grid_head<PAGED>(), b = grid_seq<PAGED>();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const int len = n < W ? n : W;
  const int nb = n / 16;                 // committed blocks
  const int p0 = n - len;                // oldest visible position
  const int k0 = p0 / 16;
  const int nbr = nb > k0 ? nb - k0 : 0; // ring blocks holding visible tokens
  int nsplit = (nbr + cb - 1) / cb;
  if (nsplit < 1) nsplit = 1;
  if (split >= nsplit) return;
  const int blo = k0 + split * cb;
  const int bhi = (blo + cb < nb) ? blo + cb : nb;
  const int wblocks = W / 16;

  const float qscale = kLog2e / sqrtf((float)D);
  const float rsd = 1.0f / sqrtf((float)D);

  // Key-dot mapping: lane covers dims [16*(lane%8), +16) of row lane/8 (+8).
  const int g = lane >> 3, vq = lane & 7;
  typename std::conditional<DITHER, DitherKeyDot, KeyDot>::type kd;
  kd.init(reinterpret_cast<const uint4*>(q + bh * D) + 2 * vq, qscale);
  // Tier B Philox key: the request id of this sequence (wave-uniform).
  uint32_t rk0 = 0, rk1 = 0;
  if constexpr (DITHER) {
    const uint64_t rid = req[b];
    rk0 = __builtin_amdgcn_readfirstlane((uint32_t)rid);
    rk1 = __builtin_amdgcn_readfirstlane((uint32_t)(rid >> 32));
  }
  // Witness mapping: lane covers bands [4*(lane%4), +4) of token lane/4.
  // nq[i] = ||q_band|| / sqrt(D) for those bands.
  const int wt = lane >> 2, wq = lane & 3;
  float nq[4];
  {
    const uint4* qv = reinterpret_cast<const uint4*>(q + bh * D) + 4 * wq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f[8];
      unpack8(qv[i], f);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
      nq[i] = sqrtf(ss) * rsd;
    }
  }

  float m = kNegBig, l = 0.f, cm = 0.f, su = 0.f, acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

  // Per-(b,h) regions are below 4 GiB: 32-bit byte offsets from wave-uniform bases.
  const char* Kbh = reinterpret_cast<const char*>(Kc + bh * (int64_t)W * D);
  const char* Vbh = reinterpret_cast<const char*>(Vc + bh * (int64_t)W * D);
  const char* Wbh = reinterpret_cast<const char*>(wit + bh * (int64_t)W * 16);
  const float* ksbh = ksc + bh * wblocks;
  const float* vsbh = vsc + bh * wblocks;
  // Paged cache: block kb lives in page table[b][kb mod W/16]; this split's
  // pages are staged in LDS once.
  extern __shared__ int32_t sm_pages[];
  if constexpr (PAGED) {
    const int32_t* tb = table + (int64_t)b * wblocks;
    for (int i = threadIdx.x; i < bhi - blo; i += NW * 64)
      sm_pages[i] = (int32_t)clamp_page(tb[(blo + i) % wblocks], num_pages);
    __syncthreads();
  }
  // Byte offset of the first row of block kb in the code arrays, and the
  // index of its scale.
  // Page of block kb (wave-uniform, so the address math stays scalar).
  auto block_page = [&](int kb) -> int64_t {
    return (int64_t)__builtin_amdgcn_readfirstlane(sm_pages[kb - blo]);
  };

  auto load = [&](Blk (&bk)[UB], int kb0) {
    // Paged: all page ids first.  Their LDS reads share a wait counter with
    // the scalar loads of the block scales, so reading them before any scale
    // load keeps the address of the next block from waiting on a scale.
    int64_t pis[UB];
    if constexpr (PAGED) {
#pragma unroll
      for (int ub = 0; ub < UB; ++ub) {
        const int kb = kb0 + ub < bhi ? kb0 + ub : bhi - 1;
        pis[ub] = block_page(kb) * H + h;  // (page, head) index
      }
    }
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      int kb = kb0 + ub;
      kb = kb < bhi ? kb : bhi - 1;  // past the end: re-read a live block, masked below
      if constexpr (PAGED) {
        const int64_t pi = pis[ub];
        const char* kp = reinterpret_cast<const char*>(Kc) + pi * (16 * D);
        const char* vp = reinterpret_cast<const char*>(Vc) + pi * (16 * D);
        const char* wp = reinterpret_cast<const char*>(wit) + pi * (16 * 32);
        bk[ub].k0 = load_stream(reinterpret_cast<const uint4*>(kp + lane * 16));
        bk[ub].k1 = load_stream(reinterpret_cast<const uint4*>(kp + 1024 + lane * 16));
        bk[ub].v0 = load_stream(reinterpret_cast<const uint4*>(vp + lane * 16));
        bk[ub].v1 = load_stream(reinterpret_cast<const uint4*>(vp + 1024 + lane * 16));
        if constexpr (!DITHER) bk[ub].w = load_stream(reinterpret_cast<const uint2*>(wp + lane * 8));
        bk[ub].sk = ksc[pi];
        bk[ub].sv = vsc[pi];
      } else {
        const uint32_t sb = (uint32_t)(kb % wblocks) * 16u;  // first slot of the block
        const uint32_t ok = sb * D + (uint32_t)lane * 16u;
        bk[ub].k0 = load_stream(reinterpret_cast<const uint4*>(Kbh + ok));
        bk[ub].k1 = load_stream(reinterpret_cast<const uint4*>(Kbh + ok + 1024u));
        bk[ub].v0 = load_stream(reinterpret_cast<const uint4*>(Vbh + ok));
        bk[ub].v1 = load_stream(reinterpret_cast<const uint4*>(Vbh + ok + 1024u));
        if constexpr (!DITHER)
          bk[ub].w = load_stream(reinterpret_cast<const uint2*>(Wbh + sb * 32u + (uint32_t)lane * 8u));
        bk[ub].sk = ksbh[kb % wblocks];
        bk[ub].sv = vsbh[kb % wblocks];
      }
    }
  };

  auto step = [&](const Blk (&cur)[UB], int kb0) {
    float s[2 * UB], sv[UB];
    uint4 dm[2 * UB];  // Tier B dither bytes of rows g and g+8 of each block
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      const int kb = kb0 + ub;
      const bool live = kb < bhi;
      const int kbc = live ? kb : bhi - 1;
      const int sbk = kbc % wblocks;
      float sk = cur[ub].sk;
      sv[ub] = cur[ub].sv;
      if constexpr (APPEND) {
        if (kb == kb_new) { sk = sk_new; sv[ub] = sv_new; }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // kbc, not kb: a past-the-end block index times 16 could pass 2^31
        // near the position limit; such rows are masked by !live anyway.
        const int pos = kbc * 16 + g + 8 * half;
        float d;
        if constexpr (DITHER) {
          const uint4 r = philox4x32_10(make_uint4((uint32_t)(kbc * 16 + g + 8 * half), (uint32_t)vq,
                                                   (uint32_t)h, layer), rk0, rk1);
          dm[2 * ub + half] = r;
          d = kd.dot(half ? cur[ub].k1 : cur[ub].k0, dm[2 * ub + half]);
          d = group_sum<8>(d) * sk;
        } else {
          d = kd.dot(half ? cur[ub].k1 : cur[ub].k0);
          d = group_sum<8>(d) * sk;  // key scale folded into the finished dot
        }
        s[2 * ub + half] = (live && pos >= p0) ? d : -INFINITY;
      }
      if constexpr (DITHER) {
        // every live block holds at least one visible token
        if (live) cm = fmaxf(cm, sk);
      } else {
        // Witness bound of token wt of this block.
        const uint2 w = cur[ub].w;
        float cp = nq[0] * f16_to_f32((uint16_t)(w.x & 0xffff));
        cp = fmaf(nq[1], f16_to_f32((uint16_t)(w.x >> 16)), cp);
        cp = fmaf(nq[2], f16_to_f32((uint16_t)(w.y & 0xffff)), cp);
        cp = fmaf(nq[3], f16_to_f32((uint16_t)(w.y >> 16)), cp);
        cp = group_sum<4>(cp);
        const int pos = kbc * 16 + wt;
        if (live && pos >= p0) {
          cm = fmaxf(cm, cp);
          if (c_all != nullptr && wq == 0) c_all[bh * W + (int64_t)sbk * 16 + wt] = cp * kBoundPad;
        }
      }
    }
    float mx = m;
#pragma unroll
    for (int i = 0; i < 2 * UB; ++i) mx = fmaxf(mx, s[i]);
    const float alpha = exp2_fast(m - mx);
    l *= alpha;
    if constexpr (DITHER) su *= alpha;
#pragma unroll
    for (int e2 = 0; e2 < 16; ++e2) acc[e2] *= alpha;
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float p = exp2_fast(s[2 * ub + half] - mx);
        l += p;
        const float pv = p * sv[ub];  // value scale folded into the weight
        const uint4 c = half ? cur[ub].v1 : cur[ub].v0;
        const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
        if constexpr (DITHER) {
          const uint4 mm = dm[2 * ub + half];
          const uint32_t mw[4] = {mm.x, mm.y, mm.z, mm.w};
          const float pvt = pv * (1.0f / 256.0f);
          su += pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float t[4];
            dither_t(cw[i], mw[i], t);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[4 * i + j] = fmaf(pvt, t[j], acc[4 * i + j]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[4 * i + j] = fmaf(pv, s8(cw[i], j), acc[4 * i + j]);
        }
      }
    }
    m = mx;
  };

  // Two register buffers in turn; the prefetch inside the loop is
  // unconditional so each wait only covers the older buffer.
  const int stride = NW * UB;
  int kb0 = blo + wave * UB;
  if (kb0 < bhi) {
    Blk ba[UB], bb[UB];
    load(ba, kb0);
    while (true) {
      if (kb0 + stride >= bhi) { step(ba, kb0); break; }
      load(bb, kb0 + stride);
      step(ba, kb0);
      kb0 += stride;
      if (kb0 + stride >= bhi) { step(bb, kb0); break; }
      load(ba, kb0 + stride);
      step(bb, kb0);
      kb0 += stride;
    }
  }

  // FINAL: the staging rows and the query for the fold in finish_int8, all
  // requested at once, while the waves merge (one memory round trip instead
  // of one per staged token).
  StageRows st;
  if constexpr (FINAL) load_stage(st, t, bh, kst, vst, q);

  if constexpr (DITHER) {
    // the -(127.5/256) sum p s_V term of every element (code - u = (t - 127.5)/256)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = fmaf(su, -127.5f / 256.0f, acc[e]);
  }
  // Merge the 8 lane groups of the wave (lanes with equal lane%8 share dims).
  float mw = m;
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) mw = fmaxf(mw, __shfl_xor(mw, o));
  {
    const float sc = exp2_fast(m - mw);
    l *= sc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] *= sc;
  }
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) {
    l += __shfl_xor(l, o);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] += __shfl_xor(acc[e], o);
  }
  cm = group_max<64>(cm);
  if (lane < 8) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sm_acc[wave][lane * 16 + e] = acc[e];
    if (lane == 0) { sm_m[wave] = mw; sm_l[wave] = l; sm_c[wave] = cm; }
  }
  __syncthreads();

  float M = kNegBig, L = 0.f, A = 0.f, CM = 0.f;
  if (t < D) {
#pragma unroll
    for (int w = 0; w < NW; ++w) { M = fmaxf(M, sm_m[w]); CM = fmaxf(CM, sm_c[w]); }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = exp2_fast(sm_m[w] - M);
      L = fmaf(sm_l[w], sc, L);
      A = fmaf(sm_acc[w][t], sc, A);
    }
  }

  if constexpr (FINAL) {
    finish_int8<DITHER>(t, bh, n, M, L, A, CM, sm_s, kst, vst, q, out, cmax_out, tv, gate, tau, W, delta, &st);
  } else {
    float* my = part + (bh * nsplit_max + split) * PF;
    if (t < D) my[4 + t] = A;
    if (t == 0) { my[0] = M; my[1] = L; my[2] = CM; }
  }
}

// FINAL: every (b, h) has a single split (the host plan has nsplit_max ==
// 1), so the work-group finishes the (b, h) itself and no merge kernel runs.
template <int NW, int UB, bool PAGED, bool FINAL, bool DITHER>
__global__ __launch_bounds__(NW * 64) void decode_int8_kernel(
    const int8_t* __restrict__ Kc, const int8_t* __restrict__ Vc, const float* __restrict__ ksc,
    const float* __restrict__ vsc, const uint16_t* __restrict__ wit, const int32_t* __restrict__ np,
    const int32_t* __restrict__ table, int64_t num_pages, const uint16_t* __restrict__ q,
    float* __restrict__ c_all, float* __restrict__ part, int H, int W, int cb, int nsplit_max,
    const uint16_t* __restrict__ kst, const uint16_t* __restrict__ vst, float* __restrict__ out,
    float* __restrict__ cmax_out, float* __restrict__ tv, int32_t* __restrict__ gate, float tau,
    const uint64_t* __restrict__ req, uint32_t layer, float delta) {
  decode_int8_wg<NW, UB, PAGED, FINAL, DITHER, false>(np[grid_seq<PAGED>()], -1, 0.f, 0.f, Kc, Vc, ksc, vsc, wit, table,
                                                      num_pages, q, c_all, part, H, W, cb, nsplit_max, kst, vst,
                                                      out, cmax_out, tv, gate, tau, req, layer, delta);
}

// Fused decode step (one token per sequence): the decode's grid.  First the token is appended: into the staging rows (by split
// 0), or -- when the token completes a 16-token block -- by quantizing that
// block (waves 0 and 1 of the split that owns the block, exactly as
// kv_append does).  After a barrier every work-group decodes its split with
// next_position + 1; the rows written are private to their (b, h) and read
// only by the work-group that wrote them (the staging rows only by the last
// stage, FINAL or the merge kernel), and the new block's scales come through
// LDS (see decode_int8_wg).  next_position[b] is shared by the work-groups
// of sequence b: each reads it first, and the sequence's counter in the
// cache's step_sync elects the last of them to finish, which writes
// next_position + 1 and clears the counter.  Every work-group of b has read
// next_position before it counts, so none reads the new value; the merge
// kernel and the next launch do.  A negative next_position (a violated
// precondition) appends nothing and advances nothing, as kv_append.
template <int NW, int UB, bool PAGED, bool FINAL, bool DITHER>
__global__ __launch_bounds__(NW * 64) void decode_step_int8_kernel(
    int8_t* Kc, int8_t* Vc, float* ksc, float* vsc, uint16_t* wit, int32_t* np, int32_t* pos, int32_t* cnt,
    RowMap map, const uint16_t* k_new, const uint16_t* v_new, Dither dz, const int32_t* table, int64_t num_pages,
    const uint16_t* q, float* part, int H, int W, int cb, int nsplit_max, uint16_t* kst, uint16_t* vst, float* out,
    float* cmax_out, float* tv, int32_t* gate, float tau, float delta) {
  __shared__ float sm_scale[2];
  const int split = blockIdx.x, h = grid_head<PAGED>(), b = grid_seq<PAGED>();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)b * H + h;
  const int n0 = np[b];
  int n = n0, kb_new = -1;
  if (n0 >= 0) {
    n = n0 + 1;
    if ((n0 & 15) == 15) {  // this token completes block n0 / 16
      // The split that decodes block n0 / 16 (blocks k0.. of the new window,
      // cb per split) commits it.
      const int len = n < W ? n : W;
      const int owner = ((n0 >> 4) - (n - len) / 16) / cb;
      if (split == owner) {
        kb_new = n0 >> 4;
        if (wave < 2) {
          const bool key = wave == 0;
          const float s = commit_block_wave(lane, key, key ? k_new : v_new, key ? kst : vst, n0, 1, kb_new, b, h,
                                            map, key ? Kc : Vc, key ? ksc : vsc, wit,
                                            (key && h == 0) ? pos + (int64_t)b * W : nullptr, dz);
          if (lane == 0) sm_scale[wave] = s;
        }
      }
    } else if (split == 0 && threadIdx.x < 32) {  // staging row n0 mod 16: 16 vectors of 16 B per tensor
      const int v16 = threadIdx.x & 15;
      const bool key = threadIdx.x < 16;
      const uint4* src = reinterpret_cast<const uint4*>(key ? k_new : v_new) + bh * 16 + v16;
      uint4* dst = reinterpret_cast<uint4*>(key ? kst : vst) + (bh * 16 + (n0 & 15)) * 16 + v16;
      store_stream(dst, *src);
    }
  }
  __syncthreads();
  const float sk_new = kb_new >= 0 ? sm_scale[0] : 0.f;
  const float sv_new = kb_new >= 0 ? sm_scale[1] : 0.f;
  decode_int8_wg<NW, UB, PAGED, FINAL, DITHER, true>(n, kb_new, sk_new, sv_new, Kc, Vc, ksc, vsc, wit, table,
                                                     num_pages, q, nullptr, part, H, W, cb, nsplit_max, kst, vst,
                                                     out, cmax_out, tv, gate, tau, dz.req, dz.layer, delta);
  if (threadIdx.x == 0 && n0 >= 0) {
    int32_t* c = cnt + (int64_t)b * kCounterStride;
    if (atomicAdd(c, 1) == H * (int)gridDim.x - 1) {
      atomicExch(c, 0);
      np[b] = n0 + 1;
    }
  }
}

// Merge of one (b, h): log-sum-exp over the split partials, then the
// staging fold, normalization and bound epilogue of finish_int8.  256
// threads; thread t < D owns output dim t.
template <bool DITHER>
__global__ __launch_bounds__(256) void merge_int8_kernel(
    const int32_t* __restrict__ np, const float* __restrict__ part, const uint16_t* __restrict__ kst,
    const uint16_t* __restrict__ vst, const uint16_t* __restrict__ q, float* __restrict__ out,
    float* __restrict__ cmax_out, float* __restrict__ tv, int32_t* __restrict__ gate, float tau, int H, int W,
    int cb, int nsplit_max, float delta) {
  __shared__ float sm_s[16];
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const int n = np[b];
  const int len = n < W ? n : W;
  const int nb = n / 16;
  const int k0 = (n - len) / 16;
  const int nbr = nb > k0 ? nb - k0 : 0;
  int nsplit = (nbr + cb - 1) / cb;
  if (nsplit < 1) nsplit = 1;
  StageRows st;
  load_stage(st, t, bh, kst, vst, q);  // issued before the partial loads
  float M = kNegBig, L = 0.f, A = 0.f, CM = 0.f;
  if (t < D) {
    const float* pp = part + bh * nsplit_max * PF;
    merge_partials<PF, true>(pp, nsplit, t, M, L, A, &CM);
  }
  finish_int8<DITHER>(t, bh, n, M, L, A, CM, sm_s, kst, vst, q, out, cmax_out, tv, gate, tau, W, delta, &st);
}

__global__ void fill_zero_f32(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// The second launch of a plan with several splits per (b, h).
hipError_t launch_merge_int8(const swa_cache& c, const void* q, float* out, float* cmax, float* tv, int32_t* gate,
                             float tau, float delta, const float* part, const SplitPlan& plan, hipStream_t s) {
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
  const uint16_t* kst = reinterpret_cast<const uint16_t*>(c.k_stage);
  const uint16_t* vst = reinterpret_cast<const uint16_t*>(c.v_stage);
  if (c.kind == SWA_KV_INT8_DITHER)
    hipLaunchKernelGGL(merge_int8_kernel<true>, dim3(c.H, c.B), dim3(256), 0, s, c.next_position, part, kst, vst,
                       q16, out, cmax, tv, gate, tau, c.H, c.W, plan.unit_per_split, plan.nsplit_max, delta);
  else
    hipLaunchKernelGGL(merge_int8_kernel<false>, dim3(c.H, c.B), dim3(256), 0, s, c.next_position, part, kst, vst,
                       q16, out, cmax, tv, gate, tau, c.H, c.W, plan.unit_per_split, plan.nsplit_max, delta);
  return hipGetLastError();
}

}  // namespace

int decode_int8_round_blocks() { return SWA_INT8_NW * SWA_INT8_UB; }

hipError_t launch_decode_step_int8(const swa_cache& c, const void* k_new, const void* v_new, const void* q,
                                   float* out, float* cmax, float* tv, int32_t* gate, float tau, float delta,
                                   void* ws, const SplitPlan& plan, hipStream_t s) {
  constexpr int NW = SWA_INT8_NW, UB = SWA_INT8_UB;
  const bool paged = c.layout == SWA_LAYOUT_PAGED;
  const bool dither = c.kind == SWA_KV_INT8_DITHER;
  const bool final_pass = plan.nsplit_max == 1;
  const Dither dz{dither ? c.request_id : nullptr, c.layer};
  float* part = reinterpret_cast<float*>(ws);
  int32_t* cnt = c.step_sync;
  const dim3 grid = int8_grid(c, plan.nsplit_max), block(NW * 64);
  const size_t lds = paged ? ((size_t)plan.unit_per_split + 1) * sizeof(int32_t) : 0;
  const int32_t* table = paged ? c.block_table : nullptr;
  const int64_t npages = paged ? c.num_pages : 0;
#define SWA_STEP_LAUNCH(P, F, DI)                                                                                \
  hipLaunchKernelGGL((decode_step_int8_kernel<NW, UB, P, F, DI>), grid, block, lds, s,                          \
                     reinterpret_cast<int8_t*>(c.k), reinterpret_cast<int8_t*>(c.v), c.k_scale, c.v_scale,      \
                     c.witness, c.next_position, c.pos, cnt, row_map(c),                                         \
                     reinterpret_cast<const uint16_t*>(k_new), reinterpret_cast<const uint16_t*>(v_new), dz,    \
                     table, npages, reinterpret_cast<const uint16_t*>(q), part, c.H, c.W, plan.unit_per_split,  \
                     plan.nsplit_max, reinterpret_cast<uint16_t*>(c.k_stage),                                    \
                     reinterpret_cast<uint16_t*>(c.v_stage), out, cmax, tv, gate, tau, delta)
#define SWA_STEP_LAUNCH_F(P, DI)                                                  \
  if (final_pass) SWA_STEP_LAUNCH(P, true, DI); else SWA_STEP_LAUNCH(P, false, DI);
  if (paged) {
    if (dither) { SWA_STEP_LAUNCH_F(true, true) } else { SWA_STEP_LAUNCH_F(true, false) }
  } else {
    if (dither) { SWA_STEP_LAUNCH_F(false, true) } else { SWA_STEP_LAUNCH_F(false, false) }
  }
#undef SWA_STEP_LAUNCH_F
#undef SWA_STEP_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || final_pass) return e;
  return launch_merge_int8(c, q, out, cmax, tv, gate, tau, delta, part, plan, s);
}

hipError_t launch_decode_int8(const swa_cache& c, const void* q, float* out, float* cmax, float* c_all,
                              float* tv, int32_t* gate, float tau, float delta, void* ws, const SplitPlan& plan,
                              hipStream_t s) {
  const bool dither = c.kind == SWA_KV_INT8_DITHER;
  if (dither) c_all = nullptr;
  constexpr int NW = SWA_INT8_NW, UB = SWA_INT8_UB;
  if (c_all != nullptr) {
    const int64_t n = (int64_t)c.B * c.H * c.W;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1 << 16) blocks = 1 << 16;
    hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)blocks), dim3(256), 0, s, c_all, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  float* part = reinterpret_cast<float*>(ws);
  const dim3 grid = int8_grid(c, plan.nsplit_max), block(NW * 64);
  const bool paged = c.layout == SWA_LAYOUT_PAGED;
  const size_t lds = paged ? ((size_t)plan.unit_per_split + 1) * sizeof(int32_t) : 0;
  const int8_t* kc = reinterpret_cast<const int8_t*>(c.k);
  const int8_t* vc = reinterpret_cast<const int8_t*>(c.v);
  const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q);
  const uint16_t* kst = reinterpret_cast<const uint16_t*>(c.k_stage);
  const uint16_t* vst = reinterpret_cast<const uint16_t*>(c.v_stage);
  const int32_t* table = paged ? c.block_table : nullptr;
  const int64_t npages = paged ? c.num_pages : 0;
  const uint64_t* req = dither ? c.request_id : nullptr;
#define SWA_INT8_LAUNCH(P, F, DI)                                                                                \
  hipLaunchKernelGGL((decode_int8_kernel<NW, UB, P, F, DI>), grid, block, lds, s, kc, vc, c.k_scale, c.v_scale, \
                     c.witness, c.next_position, table, npages, q16, c_all, part, c.H, c.W, plan.unit_per_split, \
                     plan.nsplit_max, kst, vst, out, cmax, tv, gate, tau, req, c.layer, delta)
#define SWA_INT8_LAUNCH_PF(DI)                                                              \
  if (paged) {                                                                              \
    if (final_pass) SWA_INT8_LAUNCH(true, true, DI); else SWA_INT8_LAUNCH(true, false, DI);    \
  } else {                                                                                  \
    if (final_pass) SWA_INT8_LAUNCH(false, true, DI); else SWA_INT8_LAUNCH(false, false, DI);  \
  }
  const bool final_pass = plan.nsplit_max == 1;
  if (dither) {
    SWA_INT8_LAUNCH_PF(true)
  } else {
    SWA_INT8_LAUNCH_PF(false)
  }
#undef SWA_INT8_LAUNCH_PF
#undef SWA_INT8_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || final_pass) return e;
  return launch_merge_int8(c, q, out, cmax, tv, gate, tau, delta, part, plan, s);
}

}  // namespace swa
