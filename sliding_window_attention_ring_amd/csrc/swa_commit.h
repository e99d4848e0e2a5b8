// Block commit of the INT8 cache kinds, shared by the append kernels and
// the fused decode step: one wave quantizes one 16-token block of one
// tensor of one (b, h).
#pragma once

#include "swa_device.h"

namespace swa {

// Quantization (page "WitCert：运行时误差仪表盘", section SGLang 生产级落地:
// one scale per block): s = f32(absmax / 127) with IEEE division, code =
// rint(x / s) (IEEE division, ties to even) clamped to +-127; s = 0 gives zero
// codes.  Witness (section 频带酉性与双层证书): the Euclidean norm of each
// 8-dim band of the key residual k - s*code, stored as fp16 rounded toward
// +infinity after a 2^-18 relative pad that covers the float32 rounding of
// the residual and the norm, so the stored value is never below the exact
// norm.
constexpr int kD8 = 128;

// Tier B subtractive dither (page "WitCert", section 频带酉性与双层证书,
// second tier; section SGLang 生产级落地 for the Philox five-tuple).  req ==
// nullptr selects Tier A (plain rounding plus the witness).  Otherwise the
// element of channel c of the token at position p in head h gets
// u = 1/2 - (m + 1/2)/256, m = byte c mod 16 of Philox-4x32-10 with key
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
// the witness and, if pos_b is not null, the slot positions.  Returns the
// block scale (the same in every lane).
__device__ __forceinline__ float commit_block_wave(int lane, bool key, const uint16_t* __restrict__ src_new,
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
      if (dith) y = y + fmaf(u8f(dw[e >> 2], e & 3), -1.0f / 256.0f, 255.0f / 512.0f);  // u is exact
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
  store_stream(reinterpret_cast<uint4*>(dst), packed[0]);
  store_stream(reinterpret_cast<uint4*>(dst) + 1, packed[1]);
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
    store_stream(reinterpret_cast<uint2*>(witness + row_idx * (kD8 / 8)) + part, o);
  }
  return s;
}

}  // namespace swa
