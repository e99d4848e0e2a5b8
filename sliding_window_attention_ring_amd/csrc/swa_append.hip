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

// INT8 commit of complete 16-token blocks.  Grid (blocks, H, B), 128 threads:
// wave 0 quantizes the key block and writes its witness, wave 1 the value
// block.  Lane l handles token l/4 of the block and dims [32*(l%4), +32).
// Rows come from the staging area for positions below the old
// next_position and from the new chunk otherwise.
//
// Quantization (page "WitCert：运行时误差仪表盘", section SGLang 生产级落地:
// one scale per block): s = f32(absmax / 127) with IEEE division, code =
// rint(x / s) (IEEE division, ties to even) clamped to +-127; s = 0 gives zero
// codes.  Witness (section 频带酉性与双层证书): the Euclidean norm of each
// 8-dim band of the key residual k - s*code, stored as fp16 rounded toward
// +infinity after a 2^-18 relative pad that covers the float32 rounding of
// the residual and the norm, so the stored value is never below the exact
// norm.
constexpr int kD8 = 128;
// Chunks up to this many tokens take the single-launch path.
constexpr int kSmallT = 16;

// Tier B subtractive dither (page "WitCert", section 频带酉性与双层证书,
// second tier; section SGLang 生产级落地 for the Philox five-tuple).  req ==
// nullptr selects Tier A (plain rounding plus the witness).  Otherwise the
// element of channel c of the token at position p in head h gets
// u = (m + 1/2)/256 - 1/2, m = byte c mod 16 of Philox-4x32-10 with key
// (req[b] low word, high word) and counter (p, c / 16, h, layer), words in
// order, least significant byte first; code = rint(f32(x / s) + u).  Since
// |u| <= 1/2 - 2^-9 the sum stays inside +-127.5 and the clamp never acts.
// Keys and values use the same u, and no witness is written.
struct Dither {
  const uint64_t* req;
  uint32_t layer;
};

// One wave quantizes one 16-token block (index kb) of one tensor of one
// (b, h).  Lane l handles token l/4 of the block and dims [32*(l%4), +32).
// Rows come from the staging area for positions below n0 (the old
// next_position) and from the new chunk otherwise.  For keys it also writes
// the witness and, if pos_b is not null, the slot positions.
__device__ __forceinline__ void commit_block_wave(int lane, bool key, const uint16_t* __restrict__ src_new,
                                                  const uint16_t* __restrict__ src_stage, int64_t n0, int T,
                                                  int64_t kb, int b, int h, const RowMap& map,
                                                  int8_t* __restrict__ codes, float* __restrict__ scale,
                                                  uint16_t* __restrict__ witness, int32_t* __restrict__ pos_b,
                                                  Dither dz) {
  const int W = map.W;
  const int64_t bh = (int64_t)b * map.H + h;
  const int r = lane >> 2;        // token within the block
  const int part = lane & 3;      // 32-dim quarter of the row
  const int64_t p = kb * 16 + r;
  const uint16_t* row = (p < n0) ? src_stage + (bh * 16 + (p & 15)) * kD8
                                 : src_new + (bh * T + (p - n0)) * kD8;
  const uint4* rv = reinterpret_cast<const uint4*>(row + part * 32);
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[8];
    unpack8(rv[i], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i * 8 + e] = f[e];
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = group_max<64>(amax);
  const float s = __fdiv_rn(amax, 127.0f);

  // Dither bytes of this lane's 32 channels: Philox blocks 2*part and 2*part+1.
  const bool dith = dz.req != nullptr;
  uint32_t dw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (dith) {
    const uint64_t rid = dz.req[b];
    const uint32_t k0 = (uint32_t)rid, k1 = (uint32_t)(rid >> 32);
    const uint4 d0 = philox4x32_10(make_uint4((uint32_t)p, 2u * part, (uint32_t)h, dz.layer), k0, k1);
    const uint4 d1 = philox4x32_10(make_uint4((uint32_t)p, 2u * part + 1u, (uint32_t)h, dz.layer), k0, k1);
    dw[0] = d0.x; dw[1] = d0.y; dw[2] = d0.z; dw[3] = d0.w;
    dw[4] = d1.x; dw[5] = d1.y; dw[6] = d1.z; dw[7] = d1.w;
  }
  int8_t cq[32];
  float cf[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    float c = 0.f;
    if (s > 0.f) {
      float y = __fdiv_rn(x[e], s);
      if (dith) y = y + fmaf(u8f(dw[e >> 2], e & 3), 1.0f / 256.0f, -255.0f / 512.0f);  // u is exact
      c = fminf(fmaxf(rintf(y), -127.f), 127.f);
    }
    cf[e] = c;
    cq[e] = (int8_t)(int)c;
  }
  const int64_t slot = (kb * 16) % W + r;
  const int64_t row_idx = map.row(b, h, slot);
  int8_t* dst = codes + row_idx * kD8 + part * 32;
  uint4 packed[2];
  uint32_t* pw = reinterpret_cast<uint32_t*>(packed);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pw[i] = (uint32_t)(uint8_t)cq[4 * i] | ((uint32_t)(uint8_t)cq[4 * i + 1] << 8) |
            ((uint32_t)(uint8_t)cq[4 * i + 2] << 16) | ((uint32_t)(uint8_t)cq[4 * i + 3] << 24);
  }
  reinterpret_cast<uint4*>(dst)[0] = packed[0];
  reinterpret_cast<uint4*>(dst)[1] = packed[1];
  if (lane == 0) scale[map.block(b, h, slot)] = s;
  if (key && pos_b != nullptr && part == 0) pos_b[slot] = (int32_t)p;
  if (key && !dith) {
    uint16_t wb[4];
#pragma unroll
    for (int band = 0; band < 4; ++band) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float res = fmaf(-s, cf[band * 8 + e], x[band * 8 + e]);
        ss = fmaf(res, res, ss);
      }
      const float nrm = sqrtf(ss) * (1.0f + 0x1p-18f);
      wb[band] = f32_to_f16_up(nrm);
    }
    uint2 o;
    o.x = (uint32_t)wb[0] | ((uint32_t)wb[1] << 16);
    o.y = (uint32_t)wb[2] | ((uint32_t)wb[3] << 16);
    reinterpret_cast<uint2*>(witness + row_idx * (kD8 / 8))[part] = o;
  }
}

// Grid (blocks, H, B), 128 threads: wave 0 commits the key block (with
// witness), wave 1 the value block.
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
