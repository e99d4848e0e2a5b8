// C ABI entry points (declared in include/swa.h): host-side argument
// checks, the split policy of the decode kernels, and the small
// maintenance kernels (reset, workspace fill, position-invariant check).
#include <stdlib.h>

#include <mutex>

#include "swa_device.h"
#include "swa_launch.h"

namespace swa {

int decode_round_rows(const swa_cache& c);
int decode_int8_round_blocks();

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool is_int8(int kind) { return kind == SWA_KV_INT8 || kind == SWA_KV_INT8_DITHER; }

bool head_dim_valid(int D) { return D == 16 || D == 32 || D == 64 || D == 128 || D == 256; }

// Descriptor checks common to every entry point.
int check_cache(const swa_cache* c) {
  if (c == nullptr) return SWA_ENULL;
  if (c->kind != SWA_KV_BF16 && c->kind != SWA_KV_FP32 && !is_int8(c->kind)) return SWA_EUNSUPPORTED;
  if (c->B < 1 || c->H < 1 || c->W < 1) return SWA_EINVAL;
  if (c->layout != SWA_LAYOUT_RING && c->layout != SWA_LAYOUT_PAGED) return SWA_EINVAL;
  if (c->B > 65535 || c->H > 65535) return SWA_EINVAL;  // grid y/z limits
  if (!head_dim_valid(c->D)) return SWA_EINVAL;
  // The INT8 kinds keep 16 bands of 8 dims per key (32 witness bytes).
  if (is_int8(c->kind) && c->D != 128) return SWA_EUNSUPPORTED;
  if (is_int8(c->kind) && c->W % 16 != 0) return SWA_EINVAL;
  // The decode kernels address one (b, h) region with 32-bit byte offsets.
  const int64_t esz = c->kind == SWA_KV_FP32 ? 4 : c->kind == SWA_KV_BF16 ? 2 : 1;
  if ((int64_t)c->W * c->D * esz >= ((int64_t)1 << 32)) return SWA_EINVAL;
  if (c->k == nullptr || c->v == nullptr || c->pos == nullptr || c->next_position == nullptr)
    return SWA_ENULL;
  if (!aligned16(c->k) || !aligned16(c->v)) return SWA_EALIGN;
  if (((uintptr_t)c->pos & 3u) || ((uintptr_t)c->next_position & 3u)) return SWA_EALIGN;
  if (c->layout == SWA_LAYOUT_PAGED) {
    if (c->W % 16 != 0 || c->num_pages < 1) return SWA_EINVAL;
    if (c->block_table == nullptr) return SWA_ENULL;
    if ((uintptr_t)c->block_table & 3u) return SWA_EALIGN;
  }
  if (is_int8(c->kind)) {
    if (!c->k_scale || !c->v_scale || !c->k_stage || !c->v_stage) return SWA_ENULL;
    if (!aligned16(c->k_stage) || !aligned16(c->v_stage)) return SWA_EALIGN;
    if (((uintptr_t)c->k_scale & 3u) || ((uintptr_t)c->v_scale & 3u)) return SWA_EALIGN;
  }
  if (c->kind == SWA_KV_INT8) {
    if (!c->witness) return SWA_ENULL;
    if (!aligned16(c->witness)) return SWA_EALIGN;
  }
  if (c->kind == SWA_KV_INT8_DITHER) {
    if (!c->request_id) return SWA_ENULL;
    if ((uintptr_t)c->request_id & 7u) return SWA_EALIGN;
  }
  if ((uintptr_t)c->step_sync & 3u) return SWA_EALIGN;
  return SWA_OK;
}

// Target number of decode work-groups per launch: one per compute unit of
// the device (256 on MI355X); the split size is then rounded to whole
// iteration rounds and capped at the window, so shapes with many (b, h)
// pairs still get one split per pair (512 work-groups at B*H = 512).
// Measured on MI355X, fewer and longer splits stream HBM better than many
// short ones: each split pays a query load, its pipeline fill and a partial
// write, and the merge reads every partial.  The dithered INT8 decode is the
// exception: it carries about 1.5x the VALU work per byte of the witness
// decode, and 4 work-groups per CU (two splits per (b, h) at B*H = 512) ran
// its fused step up to 0.6% faster than 1 per CU on MI355X; 8 per CU was
// 5% slower on some parts.  SWA_TARGET_WGS overrides the target for every
// kind; it is read once per process so workspace sizes stay consistent.
int target_wgs(int kind) {
  static int env = [] {
    const char* s = getenv("SWA_TARGET_WGS");
    const int x = s ? atoi(s) : 0;
    return x > 0 ? x : 0;
  }();
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  if (env > 0) return env;
  return kind == SWA_KV_INT8_DITHER ? 4 * cus : cus;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

__global__ void reset_kernel(int32_t* __restrict__ pos, int32_t* __restrict__ np, float* __restrict__ ks,
                             float* __restrict__ vs, int32_t* __restrict__ sync, int B, int H, int W, int int8) {
  const int64_t npos = (int64_t)B * W;
  const int64_t nsc = int8 ? (int64_t)B * H * (W / 16) : 0;
  const int64_t nsync = sync != nullptr ? (int64_t)B * kCounterStride : 0;
  int64_t total = npos > nsc ? npos : nsc;
  total = total > nsync ? total : nsync;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (i < npos) pos[i] = -1;
    if (i < B) np[i] = 0;
    if (i < nsc) { ks[i] = 0.f; vs[i] = 0.f; }
    if (i < nsync) sync[i] = 0;
  }
}

__global__ void fill_zero_u32(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Slot s must hold the newest position p < lim with p mod W == s, or -1.
// lim = n for row caches, 16*(n/16) for INT8 (only committed blocks).  A
// paged cache must also map every live slot to a page of the pool.
__global__ void validate_kernel(const int32_t* __restrict__ pos, const int32_t* __restrict__ np,
                                const int32_t* __restrict__ table, int64_t num_pages,
                                int32_t* __restrict__ violations, int B, int W, int int8) {
  const int64_t total = (int64_t)B * W;
  int bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(i / W), s = (int)(i % W);
    const int64_t n = np[b];
    if (n < 0) { bad += 1; continue; }
    const int64_t lim = int8 ? (n / 16) * 16 : n;
    const int64_t expect = (lim <= s) ? -1 : s + (int64_t)W * ((lim - 1 - s) / W);
    bad += (pos[i] != expect);
    if (table != nullptr && expect >= 0) {
      const int64_t page = table[(int64_t)b * (W / 16) + s / 16];
      bad += (page < 0 || page >= num_pages);
    }
  }
  if (bad) atomicAdd(violations, bad);
}

unsigned grid_for(int64_t n, int threads, int64_t cap) {
  int64_t b = (n + threads - 1) / threads;
  if (b < 1) b = 1;
  return (unsigned)(b > cap ? cap : b);
}

}  // namespace

SplitPlan plan_decode(const swa_cache& c) {
  SplitPlan p;
  const int64_t tgt = target_wgs(c.kind);
  if (is_int8(c.kind)) {
    const int64_t rb = decode_int8_round_blocks();
    const int64_t wb = c.W / 16;
    int64_t cb = round_up(((int64_t)c.B * c.H * wb + tgt - 1) / tgt, rb);
    if (cb > round_up(wb, rb)) cb = round_up(wb, rb);
    p.unit_per_split = (int)cb;
    p.nsplit_max = (int)((wb + cb - 1) / cb);
  } else {
    const int64_t rr = decode_round_rows(c);
    int64_t ch = round_up(((int64_t)c.B * c.H * c.W + tgt - 1) / tgt, rr);
    if (ch > round_up(c.W, rr)) ch = round_up(c.W, rr);
    p.unit_per_split = (int)ch;
    p.nsplit_max = (int)((c.W + ch - 1) / ch);
  }
  if (p.nsplit_max < 1) p.nsplit_max = 1;
  return p;
}

hipError_t launch_reset(const swa_cache& c, hipStream_t s) {
  int64_t n = (int64_t)c.B * c.W > (int64_t)c.B * c.H * (c.W / 16) ? (int64_t)c.B * c.W
                                                                    : (int64_t)c.B * c.H * (c.W / 16);
  if (n < (int64_t)c.B * kCounterStride) n = (int64_t)c.B * kCounterStride;
  // Pools of a paged cache may be shared with other caches: leave them alone.
  const int clear_scales = is_int8(c.kind) && c.layout == SWA_LAYOUT_RING ? 1 : 0;
  hipLaunchKernelGGL(reset_kernel, dim3(grid_for(n, 256, 1 << 16)), dim3(256), 0, s, c.pos, c.next_position,
                     c.k_scale, c.v_scale, c.step_sync, c.B, c.H, c.W, clear_scales);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 4);
  hipLaunchKernelGGL(fill_zero_u32, dim3(grid_for(n, 256, 1 << 16)), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

hipError_t launch_validate(const swa_cache& c, int32_t* violations, hipStream_t s) {
  hipLaunchKernelGGL(validate_kernel, dim3(grid_for((int64_t)c.B * c.W, 256, 1 << 16)), dim3(256), 0, s,
                     c.pos, c.next_position, c.layout == SWA_LAYOUT_PAGED ? c.block_table : nullptr,
                     c.num_pages, violations, c.B, c.W, is_int8(c.kind) ? 1 : 0);
  return hipGetLastError();
}

}  // namespace swa

using namespace swa;

namespace {

// Scratch of decode_step_int8_static: the split partials of a step live in
// this file-scope device array instead of a caller's workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code
// never passes the array's name to a kernel (in host code the name is a
// host-side stand-in, not a device address): the device address is looked
// up once per device with hipGetSymbolAddress, with that device current, and
// that pointer is what the kernels get.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (SWA_OK), or SWA_EHIP /
// SWA_EUNSUPPORTED when it cannot be found.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SWA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SWA_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SWA_EHIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return SWA_OK;
}

// Argument checks of the fused INT8 step, common to decode_step_int8 and
// decode_step_int8_static (everything but the workspace).
int check_step_int8(const swa_cache* c, const void* k_new, const void* v_new, const void* q, const float* out,
                    const float* cmax, const float* tv, const int32_t* gate, float tau, float delta) {
  const int st = check_cache(c);
  if (st != SWA_OK) return st;
  if (!is_int8(c->kind)) return SWA_EUNSUPPORTED;
  if (k_new == nullptr || v_new == nullptr || q == nullptr || out == nullptr || cmax == nullptr ||
      c->step_sync == nullptr)
    return SWA_ENULL;
  if (gate != nullptr && tv == nullptr) return SWA_ENULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(out)) return SWA_EALIGN;
  if (((uintptr_t)cmax & 3u) || ((uintptr_t)tv & 3u) || ((uintptr_t)gate & 3u)) return SWA_EALIGN;
  if (!(tau == tau)) return SWA_EINVAL;
  if (c->kind == SWA_KV_INT8_DITHER && !(delta > 0.f && delta <= 1.f)) return SWA_EINVAL;
  return SWA_OK;
}

}  // namespace

extern "C" {

const char* swa_status_string(int status) {
  switch (status) {
    case SWA_OK: return "ok";
    case SWA_EINVAL: return "invalid size or descriptor field";
    case SWA_ENULL: return "required pointer is NULL";
    case SWA_EALIGN: return "pointer not aligned (16 bytes for K/V/q/out/staging/workspace)";
    case SWA_EUNSUPPORTED: return "kind or head_dim not supported by this entry point";
    case SWA_EWORKSPACE:
      return "workspace smaller than swa_workspace_bytes() (decode_step_int8_static: the shape needs more "
             "than its 16 MiB scratch)";
    case SWA_EHIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

size_t swa_workspace_bytes(const swa_cache* c) {
  if (check_cache(c) != SWA_OK) return 0;
  return workspace_bytes_for(*c, plan_decode(*c));
}

int swa_cache_reset(const swa_cache* c, void* stream) {
  int st = check_cache(c);
  if (st != SWA_OK) return st;
  return launch_reset(*c, (hipStream_t)stream) == hipSuccess ? SWA_OK : SWA_EHIP;
}

int swa_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (ws == nullptr) return SWA_ENULL;
  if (!aligned16(ws)) return SWA_EALIGN;
  if (ws_bytes == 0) return SWA_OK;
  return launch_fill_zero(ws, ws_bytes, (hipStream_t)stream) == hipSuccess ? SWA_OK : SWA_EHIP;
}

int kv_append(const swa_cache* c, const void* k_new, const void* v_new, int32_t T, void* stream) {
  int st = check_cache(c);
  if (st != SWA_OK) return st;
  if (T < 1) return SWA_EINVAL;
  if (k_new == nullptr || v_new == nullptr) return SWA_ENULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return SWA_EALIGN;
  const hipStream_t s = (hipStream_t)stream;
  bool advanced = false;
  hipError_t e = is_int8(c->kind) ? launch_append_int8(*c, k_new, v_new, T, s, &advanced)
                                   : launch_append_rows(*c, k_new, v_new, T, s, &advanced);
  if (e == hipSuccess && !advanced) e = launch_advance(*c, T, s);
  return e == hipSuccess ? SWA_OK : SWA_EHIP;
}

int decode_attn(const swa_cache* c, const void* q, float* out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cache(c);
  if (st != SWA_OK) return st;
  if (is_int8(c->kind)) return SWA_EUNSUPPORTED;
  if (q == nullptr || out == nullptr || ws == nullptr) return SWA_ENULL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws)) return SWA_EALIGN;
  if (ws_bytes < swa_workspace_bytes(c)) return SWA_EWORKSPACE;
  const SplitPlan p = plan_decode(*c);
  return launch_decode(*c, q, out, ws, p, (hipStream_t)stream) == hipSuccess ? SWA_OK : SWA_EHIP;
}

int decode_attn_int8_witness_tv(const swa_cache* c, const void* q, float* out, float* cmax, float* tv,
                                int32_t* gate, float tau, float* c_all, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cache(c);
  if (st != SWA_OK) return st;
  if (c->kind != SWA_KV_INT8) return SWA_EUNSUPPORTED;
  if (q == nullptr || out == nullptr || cmax == nullptr || ws == nullptr) return SWA_ENULL;
  if (gate != nullptr && tv == nullptr) return SWA_ENULL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws)) return SWA_EALIGN;
  if (((uintptr_t)cmax & 3u) || ((uintptr_t)c_all & 3u) || ((uintptr_t)tv & 3u) || ((uintptr_t)gate & 3u))
    return SWA_EALIGN;
  if (!(tau == tau)) return SWA_EINVAL;  // NaN threshold
  if (ws_bytes < swa_workspace_bytes(c)) return SWA_EWORKSPACE;
  const SplitPlan p = plan_decode(*c);
  return launch_decode_int8(*c, q, out, cmax, c_all, tv, gate, tau, 1.0f, ws, p, (hipStream_t)stream) == hipSuccess
             ? SWA_OK
             : SWA_EHIP;
}

int decode_attn_int8_dither(const swa_cache* c, const void* q, float* out, float* cert, float* tv, int32_t* gate,
                            float tau, float delta, void* ws, size_t ws_bytes, void* stream) {
  int st = check_cache(c);
  if (st != SWA_OK) return st;
  if (c->kind != SWA_KV_INT8_DITHER) return SWA_EUNSUPPORTED;
  if (q == nullptr || out == nullptr || cert == nullptr || ws == nullptr) return SWA_ENULL;
  if (gate != nullptr && tv == nullptr) return SWA_ENULL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws)) return SWA_EALIGN;
  if (((uintptr_t)cert & 3u) || ((uintptr_t)tv & 3u) || ((uintptr_t)gate & 3u)) return SWA_EALIGN;
  if (!(tau == tau)) return SWA_EINVAL;                 // NaN threshold
  if (!(delta > 0.f && delta <= 1.f)) return SWA_EINVAL;  // also rejects NaN
  if (ws_bytes < swa_workspace_bytes(c)) return SWA_EWORKSPACE;
  const SplitPlan p = plan_decode(*c);
  return launch_decode_int8(*c, q, out, cert, nullptr, tv, gate, tau, delta, ws, p, (hipStream_t)stream) ==
                 hipSuccess
             ? SWA_OK
             : SWA_EHIP;
}

int decode_attn_int8_witness(const swa_cache* c, const void* q, float* out, float* cmax, float* c_all,
                             void* ws, size_t ws_bytes, void* stream) {
  return decode_attn_int8_witness_tv(c, q, out, cmax, nullptr, nullptr, 0.f, c_all, ws, ws_bytes, stream);
}

int decode_step(const swa_cache* c, const void* k_new, const void* v_new, const void* q, float* out, void* ws,
                size_t ws_bytes, void* stream) {
  int st = check_cache(c);
  if (st != SWA_OK) return st;
  if (is_int8(c->kind)) return SWA_EUNSUPPORTED;
  if (k_new == nullptr || v_new == nullptr || q == nullptr || out == nullptr || ws == nullptr ||
      c->step_sync == nullptr)
    return SWA_ENULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(q) || !aligned16(out) || !aligned16(ws))
    return SWA_EALIGN;
  if (ws_bytes < swa_workspace_bytes(c)) return SWA_EWORKSPACE;
  const SplitPlan p = plan_decode(*c);
  return launch_decode_step_rows(*c, k_new, v_new, q, out, ws, p, (hipStream_t)stream) == hipSuccess ? SWA_OK
                                                                                                      : SWA_EHIP;
}

int decode_step_int8(const swa_cache* c, const void* k_new, const void* v_new, const void* q, float* out,
                     float* cmax, float* tv, int32_t* gate, float tau, float delta, void* ws, size_t ws_bytes,
                     void* stream) {
  int st = check_step_int8(c, k_new, v_new, q, out, cmax, tv, gate, tau, delta);
  if (st != SWA_OK) return st;
  if (ws == nullptr) return SWA_ENULL;
  if (!aligned16(ws)) return SWA_EALIGN;
  if (ws_bytes < swa_workspace_bytes(c)) return SWA_EWORKSPACE;
  const SplitPlan p = plan_decode(*c);
  return launch_decode_step_int8(*c, k_new, v_new, q, out, cmax, tv, gate, tau,
                                 c->kind == SWA_KV_INT8_DITHER ? delta : 1.0f, ws, p, (hipStream_t)stream) == hipSuccess
             ? SWA_OK
             : SWA_EHIP;
}

int decode_step_int8_static(const swa_cache* c, const void* k_new, const void* v_new, const void* q, float* out,
                            float* cmax, float* tv, int32_t* gate, float tau, float delta, void* stream) {
  // The argument checks of decode_step_int8, then the partials' size against
  // the static scratch, before any HIP call; nothing is allocated.
  const int st = check_step_int8(c, k_new, v_new, q, out, cmax, tv, gate, tau, delta);
  if (st != SWA_OK) return st;
  if (swa_workspace_bytes(c) > kScratchBytes) return SWA_EWORKSPACE;
  void* ws = nullptr;
  const int sst = current_scratch(&ws);
  if (sst != SWA_OK) return sst;
  return decode_step_int8(c, k_new, v_new, q, out, cmax, tv, gate, tau, delta, ws, kScratchBytes, stream);
}

int kv_truncate(const swa_cache* c, const int32_t* cut, int32_t* ok, void* stream) {
  int st = check_cache(c);
  if (st != SWA_OK) return st;
  if (cut == nullptr) return SWA_ENULL;
  if (((uintptr_t)cut & 3u) || ((uintptr_t)ok & 3u)) return SWA_EALIGN;
  return launch_truncate(*c, cut, ok, (hipStream_t)stream) == hipSuccess ? SWA_OK : SWA_EHIP;
}

int swa_validate(const swa_cache* c, int32_t* violations, void* stream) {
  int st = check_cache(c);
  if (st != SWA_OK) return st;
  if (violations == nullptr) return SWA_ENULL;
  if ((uintptr_t)violations & 3u) return SWA_EALIGN;
  return launch_validate(*c, violations, (hipStream_t)stream) == hipSuccess ? SWA_OK : SWA_EHIP;
}

}  // extern "C"
