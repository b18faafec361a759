// Internal launchers of the ltxa HIP kernels.  Each assumes its arguments
// already passed the checks in validate.h and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "validate.h"

namespace ltxa {

// Per-pair rotary table of the head-shared grid, built on the host in fp64:
// pair i turns by (pos[axis[i]] + mid) * coef[i]; axis[i] < 0 marks a pair
// that is left as it is.  The fp32 path rounds coef[i] to fp32.
struct RopeTable {
  double coef[128];
  int32_t axis[128];
};

// Grid over the inner dimension of grid_heads heads: global pair gp turns by
// (pos[gp / n_ax] + mid) * theta^(-(gp % n_ax) / n_ax) / max_pos[gp / n_ax]
// while gp / n_ax < axes; the tensor's head h is grid head head_offset + h.
struct RopeInner {
  double theta;
  double max_pos[3];
  int32_t n_ax;
  int32_t head_offset;
};

struct RopeMode {
  bool split;   // pairs (i, i + head_dim/2) instead of (2i, 2i+1)
  bool inner;   // RopeInner grid instead of the shared RopeTable
  bool f64;     // angles and sin/cos in fp64
  double mid;   // 0, or 0.5 for cell-middle positions
  float out_scale = 1.0f;   // every output value is the rotated value times this
  float out_scale2 = 1.0f;  // the same, for the second tensor of a two-tensor launch
};

hipError_t launch_perm(const void* src, void* dst, const PermPlan& plan, int world_size,
                       bool to_packed, hipStream_t stream);

// Rotary embedding of src [batch, n_tokens, heads, head_dim] into dst
// [ranks, batch, n_tokens, heads/ranks, head_dim]; ranks = 1 with dst = src
// rotates in place.  A non-null src2 is a second tensor of the same shape
// and positions, rotated into dst2 (scaled by mode.out_scale2) by the same
// launch, which computes the angles once for both.
hipError_t launch_rope_any(const uint16_t* src, uint16_t* dst, const uint16_t* src2, uint16_t* dst2,
                           const int32_t* pos, int64_t n_tokens, int32_t axes, int64_t batch, int32_t heads,
                           int32_t head_dim, int32_t ranks, const RopeMode& mode, const RopeTable& table,
                           const RopeInner& inner, hipStream_t stream);

// Angle table of the head-shared grid: table_out[n][i] = (cos, sin) of pair i
// of token n, fp32, head_dim/2 pairs per token (mode.f64 and mode.mid as for
// launch_rope_any; the split, inner and out_scale fields are not used).
hipError_t launch_rope_angles(const int32_t* pos, float* table_out, int64_t n_tokens, int32_t axes,
                              int32_t head_dim, const RopeMode& mode, const RopeTable& table,
                              hipStream_t stream);

// launch_rope_any's pack (ranks head shards) with the angles taken from such a
// table, each (cos, sin) multiplied by out_scale.  With src2 (else null), a
// second tensor of the same shape goes to dst2 in the same launch, its
// (cos, sin) multiplied by out_scale2.
hipError_t launch_rope_pack_table(const uint16_t* src, uint16_t* dst, const uint16_t* src2, uint16_t* dst2,
                                  const float* table, int64_t n_tokens, int64_t batch, int32_t heads,
                                  int32_t head_dim, int32_t ranks, bool split, float out_scale, float out_scale2,
                                  hipStream_t stream);

// Attention over [batch, nq, heads, head_dim] operands.  The output row of
// (batch entry bb, token n, head h) is written at head slot
// (bb / out_batch) * heads + h of token n of output batch entry
// bb % out_batch in an [out_batch, nq, out_heads, head_dim] tensor: with
// out_batch = batch and out_heads = heads that is the operands' own layout;
// with batch = P * out_batch and out_heads = P * heads it is the token-major
// layout the per-rank shards came from.
// q_log2: q already holds the log2-domain operands bf16(scale * log2(e) * q)
// and is used as given (scale is then unused).
hipError_t launch_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t batch, int32_t heads, int32_t head_dim, int64_t nq, int64_t nk_pad,
                       int64_t nk_valid, float scale, int64_t out_batch, int32_t out_heads,
                       hipStream_t stream, bool q_log2 = false);

}  // namespace ltxa
