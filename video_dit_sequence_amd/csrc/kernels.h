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

hipError_t launch_pack_rope(const uint16_t* src, uint16_t* dst, const int32_t* pos, int64_t n_tokens,
                            int32_t axes, int64_t batch, int32_t heads, int32_t head_dim, int32_t ranks,
                            const RopeTable& table, hipStream_t stream);

// Attention over [batch, nq, heads, head_dim] operands.  The output row of
// (batch entry bb, token n, head h) is written at head slot
// (bb / out_batch) * heads + h of token n of output batch entry
// bb % out_batch in an [out_batch, nq, out_heads, head_dim] tensor: with
// out_batch = batch and out_heads = heads that is the operands' own layout;
// with batch = P * out_batch and out_heads = P * heads it is the token-major
// layout the per-rank shards came from.
hipError_t launch_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t batch, int32_t heads, int32_t head_dim, int64_t nq, int64_t nk_pad,
                       int64_t nk_valid, float scale, int64_t out_batch, int32_t out_heads,
                       hipStream_t stream);

}  // namespace ltxa
