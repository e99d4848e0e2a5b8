// Device helpers shared by the gfx950 kernels: wave64 lane-group reductions
// on DPP row operations, bf16/fp16 unpacking and directed rounding to fp16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

constexpr int kWave = 64;
// log2(e): scores are kept in base 2 so the softmax uses the native exp2.
constexpr float kLog2e = 1.4426950408889634f;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane of a group ends with the group total.  Steps: swap neighbours,
// swap pairs (quad permutes), mirror within half-rows of 8, mirror within
// rows of 16, then cross-row exchanges.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (G >= 4) x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x += dpp_f32<0x141>(x);  // row_half_mirror
  if constexpr (G >= 16) x += dpp_f32<0x140>(x); // row_mirror
  if constexpr (G >= 32) x += __shfl_xor(x, 16);
  if constexpr (G >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int G>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (G >= 2) x = fmaxf(x, dpp_f32<0xB1>(x));
  if constexpr (G >= 4) x = fmaxf(x, dpp_f32<0x4E>(x));
  if constexpr (G >= 8) x = fmaxf(x, dpp_f32<0x141>(x));
  if constexpr (G >= 16) x = fmaxf(x, dpp_f32<0x140>(x));
  if constexpr (G >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (G >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 is the high half of an fp32: unpacking is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Eight fp32 from a 16-byte vector of eight bf16 (element order kept).
__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Four fp32 from a 16-byte vector of four fp32.
__device__ __forceinline__ void unpack4(const uint4 v, float (&f)[4]) {
  f[0] = __builtin_bit_cast(float, v.x); f[1] = __builtin_bit_cast(float, v.y);
  f[2] = __builtin_bit_cast(float, v.z); f[3] = __builtin_bit_cast(float, v.w);
}

// Signed byte j of a 32-bit word as fp32 (one sign-extending convert).
__device__ __forceinline__ float s8(uint32_t w, int j) {
  return (float)(int32_t)(int8_t)(w >> (8 * j));
}

// Unsigned byte j of a 32-bit word as fp32 (one byte convert).
__device__ __forceinline__ float u8f(uint32_t w, int j) { return (float)((w >> (8 * j)) & 0xffu); }

// Signed low / high 16-bit half of a word as fp32.
__device__ __forceinline__ float s16lo(uint32_t w) { return (float)(int32_t)(int16_t)(w & 0xffffu); }
__device__ __forceinline__ float s16hi(uint32_t w) { return (float)((int32_t)w >> 16); }

// Philox-4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011).  Each round forms the 64-bit
// products M0*c0 and M1*c2 and maps the counter to
// (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
// then advances by the Weyl constants.  With a wave-uniform key the key
// schedule stays in scalar registers; each three-way xor is one gfx950
// three-input bit operation (truth table 0x96).
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4(__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96), (uint32_t)p1,
                   __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96), (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Nonnegative fp32 -> fp16 bits, rounded toward +infinity (never below x).
__device__ __forceinline__ uint16_t f32_to_f16_up(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  uint16_t bits = __builtin_bit_cast(uint16_t, h);
  if ((float)h < x) bits = (uint16_t)(bits + 1);  // next fp16 toward +inf (x >= 0)
  return bits;
}

// Streaming 16-byte load that does not keep the line in the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

// Non-temporal vector store, for the few rows a decode step writes: a line
// left dirty in L2 would be written back in the middle of the step's read
// stream, and each such write costs DRAM a read/write turnaround.
__device__ __forceinline__ void store_stream(uint4* p, const uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_stream(uint2* p, const uint2 v) {
  const u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}

// A page id read from a caller-filled block table, clamped into the pool so
// that a bad entry can never address memory outside it (swa_validate
// reports such entries).
__device__ __forceinline__ int64_t clamp_page(int32_t page, int64_t num_pages) {
  const int64_t p = page < 0 ? 0 : page;
  return p < num_pages ? p : num_pages - 1;
}

// Where row `slot` of (b, h) lives: the contiguous ring [B][H][W] (table
// null) or row slot%16 of page block_table[b][slot/16] in a pool
// [pages][H][16].  row() is in units of rows; block() indexes per-block
// values ([B][H][W/16] or [pages][H]).
struct RowMap {
  const int32_t* table;
  int64_t num_pages;
  int H, W;
  __device__ __forceinline__ int64_t page(int b, int64_t slot) const {
    return clamp_page(table[(int64_t)b * (W / 16) + (slot >> 4)], num_pages);
  }
  __device__ __forceinline__ int64_t row(int b, int h, int64_t slot) const {
    if (table == nullptr) return ((int64_t)b * H + h) * W + slot;
    return (page(b, slot) * H + h) * 16 + (slot & 15);
  }
  __device__ __forceinline__ int64_t block(int b, int h, int64_t slot) const {
    if (table == nullptr) return ((int64_t)b * H + h) * (W / 16) + (slot >> 4);
    return page(b, slot) * H + h;
  }
};

// A partial published inside one launch for a work-group on another XCD:
// device-scope (agent) atomic stores and loads, which are served where the
// device is coherent, past the XCD-local L2 caches (no L2 write-back or
// invalidation, which a release/acquire fence would cost for the whole L2).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Log-sum-exp merge of split partials laid out as [nsplit][PF] floats with
// m at 0, l at 1 and acc at 4.. (base-2 scores): M = max m_s, L = sum
// 2^(m_s-M) l_s, A = sum 2^(m_s-M) acc_s[t]; with CMAX also CM = max of the
// floats at 2.  One pass: eight splits' values are loaded together (a
// short last group re-reads its last split, masked out of the sums, so
// every load is unconditional and the waits stay exact), then folded in
// with a running maximum.  Up to eight splits cost one memory round trip.
// COHERENT: the partials were written in the same launch by other
// work-groups (store_coherent), so they are read with load_coherent; the
// arithmetic is the same either way, and so are the results.
template <int PF, bool CMAX = false, bool COHERENT = false>
__device__ __forceinline__ void merge_partials(const float* __restrict__ pp, int nsplit, int t, float& M,
                                               float& L, float& A, float* CM = nullptr) {
  auto ld = [](const float* p) { return COHERENT ? load_coherent(p) : *p; };
  M = -1e30f;
  L = 0.f;
  A = 0.f;
  float cm = 0.f;
  for (int sp = 0; sp < nsplit; sp += 8) {
    const int n = nsplit - sp < 8 ? nsplit - sp : 8;
    float m8[8], l8[8], a8[8], c8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float* pi = pp + (sp + (i < n ? i : n - 1)) * PF;
      m8[i] = ld(pi);
      l8[i] = ld(pi + 1);
      a8[i] = ld(pi + 4 + t);
      if constexpr (CMAX) c8[i] = ld(pi + 2);
    }
    float mc = M;
#pragma unroll
    for (int i = 0; i < 8; ++i) mc = fmaxf(mc, m8[i]);
    const float r = exp2_fast(M - mc);
    L *= r;
    A *= r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sc = i < n ? exp2_fast(m8[i] - mc) : 0.f;
      L = fmaf(l8[i], sc, L);
      A = fmaf(a8[i], sc, A);
      if constexpr (CMAX) cm = fmaxf(cm, c8[i]);
    }
    M = mc;
  }
  if constexpr (CMAX) *CM = cm;
}

}  // namespace swa
