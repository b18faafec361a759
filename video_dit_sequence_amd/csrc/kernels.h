// Internal launchers of the ltxa HIP kernels.  Each assumes its arguments
// already passed the checks in validate.h and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "validate.h"

namespace ltxa {

// Per-pair rotary table built on the host: pair i turns by pos[axis[i]] * coef[i];
// axis[i] < 0 marks a pair that is left as it is.
struct RopeTable {
  float coef[128];
  int32_t axis[128];
};

hipError_t launch_perm(const void* src, void* dst, const PermPlan& plan, int world_size,
                       bool to_packed, hipStream_t stream);

hipError_t launch_rope(uint16_t* x, const int32_t* pos, int64_t n_tokens, int32_t axes,
                       int64_t batch, int32_t heads, int32_t head_dim, const RopeTable& table,
                       hipStream_t stream);

hipError_t launch_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t batch, int32_t heads, int32_t head_dim, int64_t nq, int64_t nk_pad,
                       int64_t nk_valid, float scale, hipStream_t stream);

}  // namespace ltxa
