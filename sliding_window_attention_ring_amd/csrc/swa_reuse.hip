// Prefix reuse: truncate each sequence of the cache to a common prefix, or
// report that it must fall back to recomputation.
//
// Page "LLM 機制實驗（五）：改了歷史，能否只重算變化的後綴？": the reusable part of a cache is the
// leading run of unchanged tokens; K, V and positions of the first `cut`
// rows are kept and the next token gets position `cut` (section
// 哪些東西必須一起裁剪); a window cache that already evicted rows of that
// prefix must be recomputed instead (section 為什麼滑窗部分命中必須回退).
//
// On the ring the truncation is exact iff every row the shorter history's
// window needs is still stored: 0 <= cut <= n and (n <= W, or cut == n, or
// cut == 0).  An INT8 cache (either kind) also needs cut on a 16-token block boundary or
// inside the exact staging tail (cut >= 16*(n/16)), since committed blocks
// keep only codes.
#include "swa_device.h"
#include "swa_launch.h"

namespace swa {
namespace {

// One work-group per sequence.  Slots holding positions >= cut are marked
// empty, then next_position becomes cut; every thread has read
// next_position before the barrier that precedes the write.
__global__ __launch_bounds__(256) void truncate_kernel(int32_t* __restrict__ pos, int32_t* __restrict__ np,
                                                       const int32_t* __restrict__ cut, int32_t* __restrict__ ok,
                                                       int W, int int8) {
  const int b = blockIdx.x;
  const int64_t n = np[b];
  const int64_t c = cut[b];
  bool valid = c >= 0 && c <= n && (n <= W || c == 0 || c == n);
  if (int8) valid = valid && (c % 16 == 0 || c >= 16 * (n / 16));
  if (!valid || c == n) {
    if (threadIdx.x == 0 && ok != nullptr) ok[b] = valid ? 1 : 0;
    return;
  }
  int32_t* pb = pos + (int64_t)b * W;
  for (int s = threadIdx.x; s < W; s += blockDim.x)
    if (pb[s] >= c) pb[s] = -1;
  __syncthreads();
  if (threadIdx.x == 0) {
    np[b] = (int32_t)c;
    if (ok != nullptr) ok[b] = 1;
  }
}

}  // namespace

hipError_t launch_truncate(const swa_cache& c, const int32_t* cut, int32_t* ok, hipStream_t s) {
  hipLaunchKernelGGL(truncate_kernel, dim3(c.B), dim3(256), 0, s, c.pos, c.next_position, cut, ok, c.W,
                     (c.kind == SWA_KV_INT8 || c.kind == SWA_KV_INT8_DITHER) ? 1 : 0);
  return hipGetLastError();
}

}  // namespace swa
