// Append kernels: write new K/V rows into the ring of W slots.
//
// Ring rule (page "用Lean4形式化验证滑动窗口KV Cache的正确性", §3.4): the token
// with absolute position p is stored in slot p mod W and overwrites the
// oldest; each slot also records p (§3.2, cells carry their position).
// next_position advances with the rows (page "LLM 機制實驗（五）", section
// 哪些東西必須一起裁剪).  The position is read from next_position on the
// device, so a decode loop needs no host round trip.  The advance is a
// separate launch ordered after the writes, so no work-group can read an
// already-advanced value.
#include "swa_commit.h"
#include "swa_device.h"
#include "swa_launch.h"

namespace swa {
namespace {

// One thread per 16-byte vector of the last Tw = min(T, W) new tokens.
// A chunk longer than W writes only its last W tokens: the earlier ones
// would be overwritten inside the same chunk, so skipping them keeps every
// slot written by exactly one thread.
__global__ void append_rows_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                                   uint4* __restrict__ K, uint4* __restrict__ V,
                                   int32_t* __restrict__ pos, const int32_t* __restrict__ np, RowMap map,
                                   int B, int H, int W, int T, int Tw, int vpr) {
  const int64_t total = (int64_t)B * H * Tw * vpr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int vec = (int)(i % vpr);
    int64_t r = i / vpr;
    const int jj = (int)(r % Tw);
    r /= Tw;
    const int h = (int)(r % H);
    const int b = (int)(r / H);
    const int j = T - Tw + jj;
    const int64_t n0 = np[b];
    if (n0 < 0) continue;  // precondition violated: write nothing (swa_validate reports it)
    const int64_t p = n0 + j;
    const int64_t slot = p % W;
    const int64_t bh = (int64_t)b * H + h;
    const int64_t src = (bh * T + j) * vpr + vec;
    const int64_t dst = map.row(b, h, slot) * vpr + vec;
    K[dst] = k_new[src];
    V[dst] = v_new[src];
    if (h == 0 && vec == 0) pos[(int64_t)b * W + slot] = (int32_t)p;
  }
}

__global__ void advance_kernel(int32_t* __restrict__ np, int B, int T) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) np[b] += T;
}

// Chunks up to this many tokens take the single-launch path.
constexpr int kSmallT = 16;

// INT8 commit of complete 16-token blocks (commit_block_wave, swa_commit.h).
// Grid (blocks, H, B), 128 threads: wave 0 commits the key block (with
// witness), wave 1 the value block.  Rows come from the staging area for
// positions below the old next_position and from the new chunk otherwise.
__global__ __launch_bounds__(128) void append_int8_blocks_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ k_stage, const uint16_t* __restrict__ v_stage,
    int8_t* __restrict__ Kc, int8_t* __restrict__ Vc, float* __restrict__ k_scale,
    float* __restrict__ v_scale, uint16_t* __restrict__ witness, int32_t* __restrict__ pos,
    const int32_t* __restrict__ np, RowMap map, int H, int W, int T, Dither dz) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int64_t n0 = np[b];
  if (n0 < 0) return;  // precondition violated: write nothing (swa_validate reports it)
  const int64_t n1 = n0 + T;
  const int64_t kb_hi = n1 / 16;
  int64_t kb_lo = n0 / 16;
  if (kb_hi - W / 16 > kb_lo) kb_lo = kb_hi - W / 16;
  const int64_t kb = kb_lo + blockIdx.x;
  if (kb >= kb_hi) return;
  const bool key = (threadIdx.x >> 6) == 0;
  commit_block_wave(threadIdx.x & 63, key, key ? k_new : v_new, key ? k_stage : v_stage, n0, T, kb, b, h, map,
                    key ? Kc : Vc, key ? k_scale : v_scale, witness,
                    h == 0 ? pos + (int64_t)b * W : nullptr, dz);
}

// Decode-sized INT8 append (T <= 16) in one launch: one work-group of 16
// waves per sequence commits the (at most one) block the chunk completes
// -- 2H wave tasks, keys and values of every head -- then stages the tokens
// of the new incomplete block, then advances next_position.  Only this
// work-group reads or writes next_position[b], and the barriers order the
// staging reads of the commit before the staging writes.
__global__ __launch_bounds__(1024) void append_int8_small_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_stage,
    uint16_t* __restrict__ v_stage, int8_t* __restrict__ Kc, int8_t* __restrict__ Vc,
    float* __restrict__ k_scale, float* __restrict__ v_scale, uint16_t* __restrict__ witness,
    int32_t* __restrict__ pos, int32_t* __restrict__ np, RowMap map, int H, int W, int T, Dither dz) {
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n0 = np[b];
  if (n0 < 0) return;  // precondition violated: write nothing (swa_validate reports it)
  const int64_t n1 = n0 + T;
  const int64_t kb_hi = n1 / 16;
  int64_t kb_lo = n0 / 16;
  if (kb_hi - W / 16 > kb_lo) kb_lo = kb_hi - W / 16;
  for (int64_t kb = kb_lo; kb < kb_hi; ++kb) {
    for (int task = wave; task < 2 * H; task += 16) {
      const int h = task >> 1;
      const bool key = (task & 1) == 0;
      commit_block_wave(lane, key, key ? k_new : v_new, key ? k_stage : v_stage, n0, T, kb, b, h, map,
                        key ? Kc : Vc, key ? k_scale : v_scale, witness,
                        h == 0 ? pos + (int64_t)b * W : nullptr, dz);
    }
  }
  __syncthreads();
  int64_t lo = kb_hi * 16;
  if (lo < n0) lo = n0;
  const int cnt = (int)(n1 - lo);
  constexpr int vpr = kD8 * 2 / 16;
  const int total = H * cnt * vpr;
  const uint4* kn = reinterpret_cast<const uint4*>(k_new);
  const uint4* vn = reinterpret_cast<const uint4*>(v_new);
  uint4* ks = reinterpret_cast<uint4*>(k_stage);
  uint4* vs = reinterpret_cast<uint4*>(v_stage);
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int vec = i % vpr;
    const int j = (i / vpr) % cnt;
    const int h = i / (vpr * cnt);
    const int64_t p = lo + j;
    const int64_t bh = (int64_t)b * H + h;
    ks[(bh * 16 + (p & 15)) * vpr + vec] = kn[(bh * T + (p - n0)) * vpr + vec];
    vs[(bh * 16 + (p & 15)) * vpr + vec] = vn[(bh * T + (p - n0)) * vpr + vec];
  }
  __syncthreads();
  if (threadIdx.x == 0) np[b] = (int32_t)n1;
}

// Decode-sized row append (T <= 16) in one launch: one work-group per
// sequence writes the rows and positions, then advances next_position.
__global__ __launch_bounds__(256) void append_rows_small_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new, uint4* __restrict__ K,
    uint4* __restrict__ V, int32_t* __restrict__ pos, int32_t* __restrict__ np, RowMap map, int H, int W, int T,
    int Tw, int vpr) {
  const int b = blockIdx.x;
  const int64_t n0 = np[b];
  if (n0 < 0) return;  // precondition violated: write nothing (swa_validate reports it)
  const int total = H * Tw * vpr;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int vec = i % vpr;
    const int jj = (i / vpr) % Tw;
    const int h = i / (vpr * Tw);
    const int j = T - Tw + jj;
    const int64_t p = n0 + j;
    const int64_t slot = p % W;
    const int64_t bh = (int64_t)b * H + h;
    const int64_t dst = map.row(b, h, slot) * vpr + vec;
    K[dst] = k_new[(bh * T + j) * vpr + vec];
    V[dst] = v_new[(bh * T + j) * vpr + vec];
    if (h == 0 && vec == 0) pos[(int64_t)b * W + slot] = (int32_t)p;
  }
  __syncthreads();
  if (threadIdx.x == 0) np[b] = (int32_t)(n0 + T);
}

// Tokens of the new, still incomplete block go to the staging rows (row
// index = position mod 16).  Runs after the commit kernel, which may read
// staging rows of the block it completes.
__global__ void append_int8_stage_kernel(const uint4* __restrict__ k_new,
                                         const uint4* __restrict__ v_new,
                                         uint4* __restrict__ k_stage, uint4* __restrict__ v_stage,
                                         const int32_t* __restrict__ np, int H, int T, int vpr) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int64_t n0 = np[b];
  if (n0 < 0) return;
  const int64_t n1 = n0 + T;
  int64_t lo = (n1 / 16) * 16;
  if (lo < n0) lo = n0;
  const int64_t cnt = n1 - lo;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int j = idx / vpr, vec = idx % vpr;
  if (j >= cnt) return;
  const int64_t p = lo + j;
  const int64_t bh = (int64_t)b * H + h;
  const int64_t src = (bh * T + (p - n0)) * vpr + vec;
  const int64_t dst = (bh * 16 + (p & 15)) * vpr + vec;
  k_stage[dst] = k_new[src];
  v_stage[dst] = v_new[src];
}

}  // namespace

hipError_t launch_append_rows(const swa_cache& c, const void* k_new, const void* v_new, int T,
                              hipStream_t s, bool* advanced) {
  const int esz = c.kind == SWA_KV_FP32 ? 4 : 2;
  const int vpr = c.D * esz / 16;
  const int Tw = T < c.W ? T : c.W;
  if (T <= kSmallT) {
    hipLaunchKernelGGL(append_rows_small_kernel, dim3(c.B), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),
                       reinterpret_cast<uint4*>(c.k), reinterpret_cast<uint4*>(c.v), c.pos, c.next_position,
                       row_map(c), c.H, c.W, T, Tw, vpr);
    *advanced = true;
    return hipGetLastError();
  }
  *advanced = false;
  const int64_t total = (int64_t)c.B * c.H * Tw * vpr;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 1 << 20) blocks = 1 << 20;
  hipLaunchKernelGGL(append_rows_kernel, dim3((unsigned)blocks), dim3(threads), 0, s,
                     reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),
                     reinterpret_cast<uint4*>(c.k), reinterpret_cast<uint4*>(c.v), c.pos,
                     c.next_position, row_map(c), c.B, c.H, c.W, T, Tw, vpr);
  return hipGetLastError();
}

hipError_t launch_append_int8(const swa_cache& c, const void* k_new, const void* v_new, int T,
                              hipStream_t s, bool* advanced) {
  const Dither dz{c.kind == SWA_KV_INT8_DITHER ? c.request_id : nullptr, c.layer};
  if (T <= kSmallT) {
    hipLaunchKernelGGL(append_int8_small_kernel, dim3(c.B), dim3(1024), 0, s,
                       reinterpret_cast<const uint16_t*>(k_new), reinterpret_cast<const uint16_t*>(v_new),
                       reinterpret_cast<uint16_t*>(c.k_stage), reinterpret_cast<uint16_t*>(c.v_stage),
                       reinterpret_cast<int8_t*>(c.k), reinterpret_cast<int8_t*>(c.v), c.k_scale, c.v_scale,
                       c.witness, c.pos, c.next_position, row_map(c), c.H, c.W, T, dz);
    *advanced = true;
    return hipGetLastError();
  }
  *advanced = false;
  // At most ceil(T/16) blocks complete, and only the newest W/16 are kept.
  int nblk = (T + 15) / 16;
  if (nblk > c.W / 16) nblk = c.W / 16;
  hipLaunchKernelGGL(append_int8_blocks_kernel, dim3(nblk, c.H, c.B), dim3(128), 0, s,
                     reinterpret_cast<const uint16_t*>(k_new), reinterpret_cast<const uint16_t*>(v_new),
                     reinterpret_cast<const uint16_t*>(c.k_stage),
                     reinterpret_cast<const uint16_t*>(c.v_stage), reinterpret_cast<int8_t*>(c.k),
                     reinterpret_cast<int8_t*>(c.v), c.k_scale, c.v_scale, c.witness, c.pos,
                     c.next_position, row_map(c), c.H, c.W, T, dz);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int vpr = c.D * 2 / 16;
  const int tok = T < 16 ? T : 16;
  const int threads = 256;
  const int blocks = (tok * vpr + threads - 1) / threads;
  hipLaunchKernelGGL(append_int8_stage_kernel, dim3(blocks, c.H, c.B), dim3(threads), 0, s,
                     reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),
                     reinterpret_cast<uint4*>(c.k_stage), reinterpret_cast<uint4*>(c.v_stage),
                     c.next_position, c.H, T, vpr);
  return hipGetLastError();
}

hipError_t launch_advance(const swa_cache& c, int T, hipStream_t s) {
  hipLaunchKernelGGL(advance_kernel, dim3((c.B + 255) / 256), dim3(256), 0, s, c.next_position, c.B, T);
  return hipGetLastError();
}

}  // namespace swa
