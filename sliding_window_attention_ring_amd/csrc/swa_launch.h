// Host-side launch interface between the C-ABI layer and the kernel files.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/swa.h"
#include "swa_device.h"

namespace swa {

// Decode split policy: tokens (bf16/fp32) or 16-token blocks (INT8) per
// work-group, and the largest split count any (b, h) can need.
struct SplitPlan {
  int unit_per_split;  // rows (bf16/fp32) or blocks (INT8) per work-group
  int nsplit_max;
};

SplitPlan plan_decode(const swa_cache& c);

inline RowMap row_map(const swa_cache& c) {
  return RowMap{c.layout == SWA_LAYOUT_PAGED ? c.block_table : nullptr, c.num_pages, c.H, c.W};
}

// Floats per split partial: m, l, cmax, pad, acc[D].
inline int partial_floats(int D) { return D + 4; }


// *advanced is set when the launch also advanced next_position (the
// single-launch path for short chunks); otherwise launch_advance must follow.
hipError_t launch_append_rows(const swa_cache& c, const void* k_new, const void* v_new, int T,
                              hipStream_t s, bool* advanced);
hipError_t launch_append_int8(const swa_cache& c, const void* k_new, const void* v_new, int T,
                              hipStream_t s, bool* advanced);
hipError_t launch_advance(const swa_cache& c, int T, hipStream_t s);

hipError_t launch_decode(const swa_cache& c, const void* q, float* out, void* ws,
                         const SplitPlan& plan, hipStream_t s);
// INT8 kinds; delta is the Tier B failure budget (ignored for SWA_KV_INT8).
hipError_t launch_decode_int8(const swa_cache& c, const void* q, float* out, float* cmax,
                              float* c_all, float* tv, int32_t* gate, float tau, float delta, void* ws,
                              const SplitPlan& plan, hipStream_t s);

// One decode step (kv_append of one token, then the INT8 decode) in one
// launch, plus the merge launch when the plan has several splits per (b, h).
hipError_t launch_decode_step_int8(const swa_cache& c, const void* k_new, const void* v_new, const void* q,
                                   float* out, float* cmax, float* tv, int32_t* gate, float tau, float delta,
                                   void* ws, const SplitPlan& plan, hipStream_t s);

// The same for the bf16 / fp32 row kinds (kv_append of one token + decode_attn).
hipError_t launch_decode_step_rows(const swa_cache& c, const void* k_new, const void* v_new, const void* q,
                                   float* out, void* ws, const SplitPlan& plan, hipStream_t s);

// Workspace layout: the split partials, B*H*nsplit_max*(D+4) floats,
// padded to 256 bytes.  Nothing else: the fused step's per-sequence
// completion counters live in the cache (step_sync), so a workspace carries
// no state from one call to the next and any caches may share one.
// Counters are one per 256-byte line: atomics on one line are serialized,
// so sequences sharing a line would queue behind each other as their
// work-groups finish together.
constexpr int kCounterStride = 64;  // int32 per step_sync line
inline size_t workspace_bytes_for(const swa_cache& c, const SplitPlan& p) {
  const size_t b = (size_t)c.B * c.H * (size_t)p.nsplit_max * partial_floats(c.D) * sizeof(float);
  return (b + 255) / 256 * 256;
}

hipError_t launch_reset(const swa_cache& c, hipStream_t s);
hipError_t launch_truncate(const swa_cache& c, const int32_t* cut, int32_t* ok, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_validate(const swa_cache& c, int32_t* violations, hipStream_t s);

}  // namespace swa
