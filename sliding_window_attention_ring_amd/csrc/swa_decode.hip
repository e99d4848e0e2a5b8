// Single-query decode attention over the ring (bf16 or fp32 rows).
//
// What is computed (page "【AI 工业核题 D4】KV Cache 自回归生成推理", §三 decode
// step; page "用Lean4形式化验证滑动窗口KV Cache的正确性", §2.1): for the query of
// step t = n-1 (n = next_position), scores q.k_j / sqrt(D) over the visible
// tokens, a max-subtracted softmax and the weighted sum of V.  After n
// appends the visible tokens are exactly the rows in slots [0, min(W, n)):
// while unfilled, slots 0..n-1; once full, every slot holds one of the last W
// positions.  Softmax-weighted V is a function of the set of (k, v) pairs, so
// slot order never matters (§3.3 keeps attention separate from the cache
// order).
//
// Layout of the work (gfx950, wave64):
// * grid (split, h, b); a work-group of NW waves owns `chunk` consecutive
//   slots of one (b, h); splits beyond the live length exit at once;
// * a row of D elements is read by LPR lanes, 16 bytes each, so one wave
//   load instruction covers 64/LPR consecutive rows (1 KiB, coalesced);
// * each lane keeps U loads of K and U of V in flight for the next
//   iteration while it computes on the current one (register double
//   buffering);
// * dot products are reduced inside each LPR-lane group with DPP row ops;
//   the online softmax keeps a running (max, sum, acc) per lane group in
//   base 2;
// * lane groups, then waves (through LDS) are merged with the log-sum-exp
//   rule; a (b, h) served by one split writes its output directly, otherwise
//   each split writes a partial (m, l, acc[D]) and a small second kernel
//   merges the splits and normalizes.  The kernel boundary makes the
//   partials visible across the XCDs' separate L2 caches, so no work-group
//   needs a device-wide fence (each would write back and invalidate its L2);
//   the fused step with up to 63 heads merges in its own launch instead,
//   through device-coherent stores and loads (decode_rows_wg, INMERGE).
#include "swa_device.h"
#include "swa_launch.h"

namespace swa {
namespace {

// Row formats.  bf16 keys use the packed bf16 dot product (exact products,
// fp32 accumulate) with the raw query, scaled once per row afterwards; fp32
// rows use plain fused multiply-adds with a pre-scaled query.
template <typename T>
struct RowFmt;
template <>
struct RowFmt<uint16_t> {  // bf16
  static constexpr int kEpv = 8;
  struct Q { uint32_t w[4]; };
  static __device__ __forceinline__ Q load_q(const uint4 v, float) { return Q{{v.x, v.y, v.z, v.w}}; }
  static __device__ __forceinline__ float dot(const Q& q, const uint4 k) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    float d = 0.f;
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q.w[0]), __builtin_bit_cast(bf2, k.x), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q.w[1]), __builtin_bit_cast(bf2, k.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q.w[2]), __builtin_bit_cast(bf2, k.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q.w[3]), __builtin_bit_cast(bf2, k.w), d, false);
    return d;
  }
  static constexpr bool kPostScale = true;
  static __device__ __forceinline__ void unpack(const uint4 v, float (&f)[8]) { unpack8(v, f); }
};
template <>
struct RowFmt<float> {
  static constexpr int kEpv = 4;
  struct Q { float f[4]; };
  static __device__ __forceinline__ Q load_q(const uint4 v, float scale) {
    Q q;
    unpack4(v, q.f);
#pragma unroll
    for (int e = 0; e < 4; ++e) q.f[e] *= scale;
    return q;
  }
  static __device__ __forceinline__ float dot(const Q& q, const uint4 k) {
    float f[4];
    unpack4(k, f);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) d = fmaf(q.f[e], f[e], d);
    return d;
  }
  static constexpr bool kPostScale = false;
  static __device__ __forceinline__ void unpack(const uint4 v, float (&f)[4]) { unpack4(v, f); }
};

constexpr float kNegBig = -1e30f;  // finite start value of the running max

// Waves per work-group and row loads per lane per iteration.
#ifndef SWA_ROW_NW
#define SWA_ROW_NW 4
#endif
#ifndef SWA_ROW_U
#define SWA_ROW_U 4
#endif

// Grid order: (split, h, b), or (split, b, h) for paged pools, so that the
// hardware's turn-by-turn hand-out of work-groups to the XCDs puts all heads
// of a sequence on one XCD, whose L2 then reads the sequence's block-table
// lines once, and whose reads of a page's heads (adjacent in the pool) come
// together.
#ifndef SWA_ROW_PAGED_SEQ_MAJOR
#define SWA_ROW_PAGED_SEQ_MAJOR 1
#endif
#ifndef SWA_ROW_RING_SEQ_MAJOR
#define SWA_ROW_RING_SEQ_MAJOR 0
#endif
template <bool PAGED>
constexpr bool kRowSeqMajor = PAGED ? SWA_ROW_PAGED_SEQ_MAJOR : SWA_ROW_RING_SEQ_MAJOR;
template <bool PAGED>
__device__ __forceinline__ int row_grid_head() {
  return kRowSeqMajor<PAGED> ? (int)blockIdx.z : (int)blockIdx.y;
}
template <bool PAGED>
__device__ __forceinline__ int row_grid_seq() {
  return kRowSeqMajor<PAGED> ? (int)blockIdx.y : (int)blockIdx.z;
}
inline dim3 row_grid(const swa_cache& c, int nsplit) {
  const bool seq_major = c.layout == SWA_LAYOUT_PAGED ? kRowSeqMajor<true> : kRowSeqMajor<false>;
  return seq_major ? dim3(nsplit, c.B, c.H) : dim3(nsplit, c.H, c.B);
}

// The decode of one (split, h, b) work-group, called by decode_kernel and
// by the fused step kernel; n is next_position[b] as this decode sees it.
// FINAL: the host plan has one split per (b, h), so the work-group writes
// the output itself (zeros for an empty sequence) and no merge kernel runs.
// INMERGE (fused step, several splits): the splits of a (b, h) publish
// their partials with device-coherent stores and count themselves on
// pair_cnt (zero between launches); the last to arrive merges them, so no
// merge kernel runs either.  Each wave waits for its partial stores to
// complete before the count, and the merge reads them with device-coherent
// loads, so no L2 write-back or invalidation is needed.
// No restrict qualifiers: the fused step writes a row of K and V first.
template <typename T, int D, int NW, int U, bool PAGED, bool FINAL, bool INMERGE = false>
__device__ __forceinline__ void decode_rows_wg(int n, const uint4* K, const uint4* V, const int32_t* table,
                                               int64_t num_pages, const uint4* q, float* out, float* part, int H,
                                               int W, int chunk, int nsplit_max, int32_t* pair_cnt = nullptr) {
  using F = RowFmt<T>;
  constexpr int EPV = F::kEpv;
  constexpr int VPR = D / EPV;          // 16-byte vectors per row
  constexpr int LPR = VPR;              // lanes per row
  constexpr int RPL = 64 / LPR;         // rows per wave load
  constexpr int RPI = RPL * U;          // rows per wave iteration
  constexpr int PF = D + 4;             // floats per split partial
  // A row spans 2..64 lanes.  A wave load covers RPL rows: up to 16 rows
  // (one page, wave-uniform), or 32 rows of two pages (bf16 D = 16), whose
  // page is then looked up per lane.
  static_assert(LPR >= 2 && LPR <= 64, "row must span 2..64 lanes");
  static_assert(16 % RPL == 0 || RPL == 32, "a wave load spans at most two 16-row pages");
  constexpr bool kLanePage = RPL > 16;

  __shared__ float sm_m[NW], sm_l[NW];
  __shared__ float sm_acc[NW][D];
  __shared__ int sm_last;

  const int split = blockIdx.x, h = row_grid_head<PAGED>(), b = row_grid_seq<PAGED>();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)b * H + h;
  const int len = n < W ? n : W;
  if (len <= 0) {  // empty cache: zeros, written here (split 0) or by the merge kernel
    if constexpr (FINAL || INMERGE) {
      if (split == 0)
        for (int t = threadIdx.x; t < D; t += NW * 64) out[bh * D + t] = 0.f;
    }
    return;
  }
  const int nsplit = (len + chunk - 1) / chunk;
  if (split >= nsplit) return;
  const int r0 = split * chunk;
  const int r1 = (r0 + chunk < len) ? r0 + chunk : len;

  const int g = lane / LPR;      // row within a wave load
  const int vec = lane % LPR;    // 16-byte vector within the row
  // Per-(b,h) regions are below 4 GiB, so rows are addressed by 32-bit byte
  // offsets from a wave-uniform base.
  const char* Kbh = reinterpret_cast<const char*>(K + bh * (int64_t)W * VPR);
  const char* Vbh = reinterpret_cast<const char*>(V + bh * (int64_t)W * VPR);
  // Paged rows: the pages of this split's 16-slot blocks, staged in LDS once.
  extern __shared__ int32_t sm_pages[];
  const int pb0 = r0 >> 4;
  if constexpr (PAGED) {
    const int npb = ((r1 + 15) >> 4) - pb0;
    const int32_t* tb = table + (int64_t)b * (W / 16) + pb0;
    for (int i = threadIdx.x; i < npb; i += NW * 64) sm_pages[i] = (int32_t)clamp_page(tb[i], num_pages);
    __syncthreads();
  }

  const float qscale = kLog2e / sqrtf((float)D);  // base-2 softmax of q.k/sqrt(D)
  const typename F::Q qv = F::load_q(q[bh * VPR + vec], qscale);

  float m = kNegBig, l = 0.f, acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.f;

  auto load = [&](uint4 (&kb)[U], uint4 (&vb)[U], int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int row = base + u * RPL + g;
      row = row < r1 ? row : r1 - 1;  // past the end: re-read a live row, masked below
      if constexpr (PAGED) {
        // The RPL rows of load u lie in one 16-row page when RPL divides 16
        // (the split starts on a page), also after clamping at the end, so the
        // page is wave-uniform: a scalar base plus a 32-bit lane offset.
        // With 32 rows per load each lane looks its own page up.
        int64_t page;
        if constexpr (kLanePage) {
          page = sm_pages[(row >> 4) - pb0];
        } else {
          int first = base + u * RPL;
          first = first < r1 ? first : r1 - 1;
          page = __builtin_amdgcn_readfirstlane(sm_pages[(first >> 4) - pb0]);
        }
        const int64_t pbase = (page * H + h) * (16 * VPR * 16);
        const uint32_t off = (uint32_t)((row & 15) * VPR + vec) * 16u;
        kb[u] = load_stream(reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(K) + pbase + off));
        vb[u] = load_stream(reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(V) + pbase + off));
      } else {
        const uint32_t off = (uint32_t)(row * VPR + vec) * 16u;
        kb[u] = load_stream(reinterpret_cast<const uint4*>(Kbh + off));
        vb[u] = load_stream(reinterpret_cast<const uint4*>(Vbh + off));
      }
    }
  };
  auto step = [&](const uint4 (&kb)[U], const uint4 (&vb)[U], int base) {
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d = group_sum<LPR>(F::dot(qv, kb[u]));
      if constexpr (F::kPostScale) d *= qscale;
      const int row = base + u * RPL + g;
      s[u] = row < r1 ? d : -INFINITY;
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u]);
    const float alpha = exp2_fast(m - mx);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = exp2_fast(s[u] - mx);
      l += p;
      float f[EPV];
      F::unpack(vb[u], f);
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] = fmaf(p, f[e], acc[e]);
    }
    m = mx;
  };

  // Two register buffers in turn: while one is consumed the other's loads
  // are in flight.  Inside the loop the prefetch is unconditional, so the
  // wait before each use only covers the older buffer.
  const int stride = NW * RPI;
  int base = r0 + wave * RPI;
  if (base < r1) {
    uint4 ka[U], va[U], kb[U], vb[U];
    load(ka, va, base);
    while (true) {
      if (base + stride >= r1) { step(ka, va, base); break; }
      load(kb, vb, base + stride);
      step(ka, va, base);
      base += stride;
      if (base + stride >= r1) { step(kb, vb, base); break; }
      load(ka, va, base + stride);
      step(kb, vb, base);
      base += stride;
    }
  }

  // Merge the lane groups of this wave (lanes with equal `vec` hold the same dims).
  float mw = m;
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) mw = fmaxf(mw, __shfl_xor(mw, o));
  {
    const float sc = exp2_fast(m - mw);
    l *= sc;
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] *= sc;
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
    l += __shfl_xor(l, o);
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] += __shfl_xor(acc[e], o);
  }
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) sm_acc[wave][lane * EPV + e] = acc[e];
    if (lane == 0) { sm_m[wave] = mw; sm_l[wave] = l; }
  }
  __syncthreads();

  // Merge the waves: thread t owns output dim t.
  const int t = threadIdx.x;
  float M = kNegBig, L = 0.f, A = 0.f;
  if (t < D) {
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w]);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = exp2_fast(sm_m[w] - M);
      L = fmaf(sm_l[w], sc, L);
      A = fmaf(sm_acc[w][t], sc, A);
    }
  }
  if (nsplit == 1) {
    if (t < D) out[bh * D + t] = A / L;
    return;
  }

  float* my = part + (bh * nsplit_max + split) * PF;
  if constexpr (INMERGE) {
    // Publish this split's partial; the last split of the (b, h) to arrive merges.
    if (t < D) store_coherent(my + 4 + t, A);
    if (t == 0) { store_coherent(my, M); store_coherent(my + 1, L); }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
    __syncthreads();
    if (t == 0) {
      const int last = atomicAdd(pair_cnt, 1) == nsplit - 1;
      if (last) atomicExch(pair_cnt, 0);
      sm_last = last;
    }
    __syncthreads();
    if (sm_last && t < D) {
      float M2, L2, A2;
      merge_partials<PF, false, true>(part + bh * nsplit_max * PF, nsplit, t, M2, L2, A2);
      out[bh * D + t] = A2 / L2;
    }
  } else {
    // Publish this split's partial for the merge kernel.
    if (t < D) my[4 + t] = A;
    if (t == 0) { my[0] = M; my[1] = L; }
  }
}

template <typename T, int D, int NW, int U, bool PAGED, bool FINAL>
__global__ __launch_bounds__(NW * 64) void decode_kernel(
    const uint4* __restrict__ K, const uint4* __restrict__ V, const int32_t* __restrict__ np,
    const int32_t* __restrict__ table, int64_t num_pages, const uint4* __restrict__ q, float* __restrict__ out,
    float* __restrict__ part, int H, int W, int chunk, int nsplit_max) {
  decode_rows_wg<T, D, NW, U, PAGED, FINAL>(np[row_grid_seq<PAGED>()], K, V, table, num_pages, q, out, part, H, W, chunk,
                                            nsplit_max);
}

// Fused decode step (one token per sequence) for row caches: grid (split,
// h, b) as the decode's.  INMERGE (several splits per (b, h), H <= 63): the
// splits of a (b, h) merge in this launch, counted on int [b][1 + h] of the
// cache's step_sync line of sequence b (int [b][0] counts the sequence's
// work-groups).  The work-group of the split whose slots hold slot
// next_position mod W writes its token's key and value rows there (and, for
// h == 0, the slot's position); after a barrier every work-group decodes its
// split with next_position + 1.  The rows are read only by the work-group
// that wrote them.  next_position[b] is advanced by the last of the work-groups
// of sequence b to finish, elected by the sequence's counter in the cache's
// step_sync, as in the INT8 step kernel.  A negative next_position (a
// violated precondition) appends nothing and advances nothing.
template <typename T, int D, int NW, int U, bool PAGED, bool FINAL, bool INMERGE>
__global__ __launch_bounds__(NW * 64) void decode_step_rows_kernel(
    uint4* K, uint4* V, int32_t* np, int32_t* pos, int32_t* cnt, RowMap map, const uint4* k_new,
    const uint4* v_new, int64_t num_pages, const uint4* q, float* out, float* part, int H, int W, int chunk,
    int nsplit_max) {
  constexpr int VPR = D / RowFmt<T>::kEpv;
  const int split = blockIdx.x, h = row_grid_head<PAGED>(), b = row_grid_seq<PAGED>();
  const int64_t bh = (int64_t)b * H + h;
  const int n0 = np[b];
  if (n0 >= 0) {
    const int64_t slot = n0 % W;
    if (slot / chunk == split) {
      const int64_t row = map.row(b, h, slot);
      for (int i = threadIdx.x; i < 2 * VPR; i += NW * 64) {
        if (i < VPR) store_stream(K + row * VPR + i, k_new[bh * VPR + i]);
        else store_stream(V + row * VPR + (i - VPR), v_new[bh * VPR + (i - VPR)]);
      }
      if (h == 0 && threadIdx.x == 0) pos[(int64_t)b * W + slot] = n0;
    }
  }
  __syncthreads();
  decode_rows_wg<T, D, NW, U, PAGED, FINAL, INMERGE>(n0 >= 0 ? n0 + 1 : n0, K, V, map.table, num_pages, q, out, part,
                                                     H, W, chunk, nsplit_max,
                                                     INMERGE ? cnt + (int64_t)b * kCounterStride + 1 + h : nullptr);
  if (threadIdx.x == 0 && n0 >= 0) {
    int32_t* c = cnt + (int64_t)b * kCounterStride;
    if (atomicAdd(c, 1) == H * (int)gridDim.x - 1) {
      atomicExch(c, 0);
      np[b] = n0 + 1;
    }
  }
}

// Log-sum-exp merge of the split partials of one (b, h); thread t owns dim t.
// A (b, h) served by a single split already has its output; an empty cache
// gets zeros.
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(const int32_t* __restrict__ np,
                                                  const float* __restrict__ part, float* __restrict__ out,
                                                  int H, int W, int chunk, int nsplit_max) {
  constexpr int PF = D + 4;
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const int n = np[b];
  const int len = n < W ? n : W;
  if (len <= 0) { out[bh * D + t] = 0.f; return; }
  const int nsplit = (len + chunk - 1) / chunk;
  if (nsplit == 1) return;
  float M, L, A;
  merge_partials<PF>(part + bh * nsplit_max * PF, nsplit, t, M, L, A);
  out[bh * D + t] = A / L;
}

// The second launch of a plan with several splits per (b, h).
template <int D>
hipError_t launch_merge(const swa_cache& c, float* out, const float* part, const SplitPlan& plan, hipStream_t s) {
  hipLaunchKernelGGL((merge_kernel<D>), dim3(c.H, c.B), dim3(D), 0, s, c.next_position, part, out, c.H, c.W,
                     plan.unit_per_split, plan.nsplit_max);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_one(const swa_cache& c, const void* q, float* out, void* ws, const SplitPlan& plan,
                      hipStream_t s) {
  constexpr int NW = SWA_ROW_NW, U = SWA_ROW_U;
  float* part = reinterpret_cast<float*>(ws);
  const dim3 grid = row_grid(c, plan.nsplit_max), block(NW * 64);
  const bool paged = c.layout == SWA_LAYOUT_PAGED;
  // paged: one int per 16-slot block of a split, plus slack
  const size_t lds = paged ? ((size_t)plan.unit_per_split / 16 + 2) * sizeof(int32_t) : 0;
  const uint4* kp = reinterpret_cast<const uint4*>(c.k);
  const uint4* vp = reinterpret_cast<const uint4*>(c.v);
  const uint4* qp = reinterpret_cast<const uint4*>(q);
  const int32_t* table = paged ? c.block_table : nullptr;
  const int64_t npages = paged ? c.num_pages : 0;
#define SWA_ROW_LAUNCH(P, F)                                                                                     \
  hipLaunchKernelGGL((decode_kernel<T, D, NW, U, P, F>), grid, block, lds, s, kp, vp, c.next_position, table,    \
                     npages, qp, out, part, c.H, c.W, plan.unit_per_split, plan.nsplit_max)
  const bool final_pass = plan.nsplit_max == 1;
  if (paged) {
    if (final_pass) SWA_ROW_LAUNCH(true, true); else SWA_ROW_LAUNCH(true, false);
  } else {
    if (final_pass) SWA_ROW_LAUNCH(false, true); else SWA_ROW_LAUNCH(false, false);
  }
#undef SWA_ROW_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || final_pass) return e;
  return launch_merge<D>(c, out, part, plan, s);
}

template <typename T, int D>
hipError_t launch_step_one(const swa_cache& c, const void* k_new, const void* v_new, const void* q, float* out,
                           void* ws, const SplitPlan& plan, hipStream_t s) {
  constexpr int NW = SWA_ROW_NW, U = SWA_ROW_U;
  const bool paged = c.layout == SWA_LAYOUT_PAGED;
  const bool final_pass = plan.nsplit_max == 1;
  // Several splits per (b, h): merged in the step kernel when each head has
  // a counter in its sequence's step_sync line, else by the merge kernel.
  const bool inmerge = !final_pass && c.H <= kCounterStride - 1;
  const size_t lds = paged ? ((size_t)plan.unit_per_split / 16 + 2) * sizeof(int32_t) : 0;
  const dim3 grid = row_grid(c, plan.nsplit_max), block(NW * 64);
  float* part = reinterpret_cast<float*>(ws);
  int32_t* cnt = c.step_sync;
#define SWA_ROW_STEP(P, F, M)                                                                                     \
  hipLaunchKernelGGL((decode_step_rows_kernel<T, D, NW, U, P, F, M>), grid, block, lds, s,                        \
                     reinterpret_cast<uint4*>(c.k), reinterpret_cast<uint4*>(c.v), c.next_position, c.pos, cnt,    \
                     row_map(c), reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),    \
                     paged ? c.num_pages : 0, reinterpret_cast<const uint4*>(q), out, part, c.H, c.W,               \
                     plan.unit_per_split, plan.nsplit_max)
  if (paged) {
    if (final_pass) SWA_ROW_STEP(true, true, false);
    else if (inmerge) SWA_ROW_STEP(true, false, true);
    else SWA_ROW_STEP(true, false, false);
  } else {
    if (final_pass) SWA_ROW_STEP(false, true, false);
    else if (inmerge) SWA_ROW_STEP(false, false, true);
    else SWA_ROW_STEP(false, false, false);
  }
#undef SWA_ROW_STEP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || final_pass || inmerge) return e;
  return launch_merge<D>(c, out, part, plan, s);
}

}  // namespace

hipError_t launch_decode_step_rows(const swa_cache& c, const void* k_new, const void* v_new, const void* q,
                                   float* out, void* ws, const SplitPlan& plan, hipStream_t s) {
  if (c.kind == SWA_KV_BF16) {
    switch (c.D) {
      case 16: return launch_step_one<uint16_t, 16>(c, k_new, v_new, q, out, ws, plan, s);
      case 32: return launch_step_one<uint16_t, 32>(c, k_new, v_new, q, out, ws, plan, s);
      case 64: return launch_step_one<uint16_t, 64>(c, k_new, v_new, q, out, ws, plan, s);
      case 128: return launch_step_one<uint16_t, 128>(c, k_new, v_new, q, out, ws, plan, s);
      case 256: return launch_step_one<uint16_t, 256>(c, k_new, v_new, q, out, ws, plan, s);
    }
  } else if (c.kind == SWA_KV_FP32) {
    switch (c.D) {
      case 16: return launch_step_one<float, 16>(c, k_new, v_new, q, out, ws, plan, s);
      case 32: return launch_step_one<float, 32>(c, k_new, v_new, q, out, ws, plan, s);
      case 64: return launch_step_one<float, 64>(c, k_new, v_new, q, out, ws, plan, s);
      case 128: return launch_step_one<float, 128>(c, k_new, v_new, q, out, ws, plan, s);
      case 256: return launch_step_one<float, 256>(c, k_new, v_new, q, out, ws, plan, s);
    }
  }
  return hipErrorInvalidValue;
}

// Rows of one work-group iteration round (all NW waves): the split size is a
// multiple of it so that every wave does the same number of iterations.
int decode_round_rows(const swa_cache& c) {
  const int esz = c.kind == SWA_KV_FP32 ? 4 : 2;
  const int lpr = c.D * esz / 16;
  return SWA_ROW_NW * (64 / lpr) * SWA_ROW_U;
}

hipError_t launch_decode(const swa_cache& c, const void* q, float* out, void* ws, const SplitPlan& plan,
                         hipStream_t s) {
  if (c.kind == SWA_KV_BF16) {
    switch (c.D) {
      case 16: return launch_one<uint16_t, 16>(c, q, out, ws, plan, s);
      case 32: return launch_one<uint16_t, 32>(c, q, out, ws, plan, s);
      case 64: return launch_one<uint16_t, 64>(c, q, out, ws, plan, s);
      case 128: return launch_one<uint16_t, 128>(c, q, out, ws, plan, s);
      case 256: return launch_one<uint16_t, 256>(c, q, out, ws, plan, s);
    }
  } else if (c.kind == SWA_KV_FP32) {
    switch (c.D) {
      case 16: return launch_one<float, 16>(c, q, out, ws, plan, s);
      case 32: return launch_one<float, 32>(c, q, out, ws, plan, s);
      case 64: return launch_one<float, 64>(c, q, out, ws, plan, s);
      case 128: return launch_one<float, 128>(c, q, out, ws, plan, s);
      case 256: return launch_one<float, 256>(c, q, out, ws, plan, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace swa
