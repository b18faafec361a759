// Host-only argument checks for the ltxa C ABI.  Pure integer arithmetic: no
// HIP calls, so every error path can be exercised without a GPU.
#pragma once

#include <cmath>
#include <cstdint>

#include "ltxa.h"

namespace ltxa {

constexpr int64_t kMaxBytes = INT64_C(1) << 52;  // keeps every byte offset far from overflow

// a * b, or -1 if it would exceed kMaxBytes.
inline int64_t mul_capped(int64_t a, int64_t b) {
  if (a < 0 || b < 0) return -1;
  if (a == 0 || b == 0) return 0;
  if (a > kMaxBytes / b) return -1;
  return a * b;
}

inline int64_t mul4_capped(int64_t a, int64_t b, int64_t c, int64_t d) {
  int64_t ab = mul_capped(a, b);
  if (ab < 0) return -1;
  int64_t abc = mul_capped(ab, c);
  if (abc < 0) return -1;
  return mul_capped(abc, d);
}

inline bool overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  auto pa = reinterpret_cast<uintptr_t>(a);
  auto pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + static_cast<uintptr_t>(b_bytes) && pb < pa + static_cast<uintptr_t>(a_bytes);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct PermPlan {
  int64_t bytes;  // bytes of each tensor
  int64_t rows;   // batch * n_tokens
  int64_t chunk;  // bytes of one (token, rank) head block: heads/P * head_dim * elem
};

inline int check_perm(const void* src, const void* dst, int64_t batch, int64_t n_tokens,
                      int32_t heads, int32_t head_dim, int32_t world_size,
                      int32_t elem_bytes, PermPlan* plan) {
  if (!src || !dst) return LTXA_E_NULL;
  if (batch < 1 || n_tokens < 1 || heads < 1 || head_dim < 1 || world_size < 1)
    return LTXA_E_SHAPE;
  if (!(elem_bytes == 1 || elem_bytes == 2 || elem_bytes == 4 || elem_bytes == 8))
    return LTXA_E_SHAPE;
  if (heads % world_size != 0 || n_tokens % world_size != 0) return LTXA_E_DIVISIBILITY;
  int64_t bytes = mul4_capped(batch, n_tokens, heads, mul_capped(head_dim, elem_bytes));
  if (bytes < 0) return LTXA_E_RANGE;
  int64_t chunk = static_cast<int64_t>(heads / world_size) * head_dim * elem_bytes;
  // Grid: one thread per vector (1 to 16 bytes), 256 per workgroup, at most
  // 2^31 - 1 workgroups: 2^38 bytes (256 GiB) per tensor always fits.
  if (world_size > 65535) return LTXA_E_RANGE;
  if (bytes > (INT64_C(1) << 38)) return LTXA_E_RANGE;
  if (overlap(src, bytes, dst, bytes)) return LTXA_E_ALIAS;
  plan->bytes = bytes;
  plan->rows = batch * n_tokens;
  plan->chunk = chunk;
  return LTXA_OK;
}

inline int check_rope_tensor(const void* x, const int32_t* pos, int64_t n, int32_t axes,
                             const double* max_pos, int32_t head_dim) {
  if (!pos || !max_pos) return LTXA_E_NULL;
  if (n < 1) return LTXA_E_SHAPE;
  if (axes < 1 || axes > 3 || axes > head_dim / 2) return LTXA_E_SHAPE;
  for (int a = 0; a < axes; ++a)
    if (!(std::isfinite(max_pos[a]) && max_pos[a] > 0.0)) return LTXA_E_SHAPE;
  if (!aligned16(x) || !aligned16(pos)) return LTXA_E_ALIGN;
  return LTXA_OK;
}

inline int check_rope(const void* q, const int32_t* q_pos, int64_t nq, int32_t q_axes,
                      const double* q_max_pos, const void* k, const int32_t* k_pos, int64_t nk,
                      int32_t k_axes, const double* k_max_pos, int64_t batch, int32_t heads,
                      int32_t head_dim, double theta) {
  if (!q && !k) return LTXA_E_NULL;
  if (batch < 1 || heads < 1) return LTXA_E_SHAPE;
  if (head_dim < 2 || head_dim > 256 || head_dim % 2 != 0) return LTXA_E_SHAPE;
  if (!(std::isfinite(theta) && theta > 0.0)) return LTXA_E_SHAPE;
  if ((head_dim * 2) % 16 != 0) return LTXA_E_ALIGN;
  int64_t qb = 0, kb = 0;
  if (q) {
    int rc = check_rope_tensor(q, q_pos, nq, q_axes, q_max_pos, head_dim);
    if (rc) return rc;
    qb = mul4_capped(batch, nq, heads, int64_t(head_dim) * 2);
    if (qb < 0 || mul_capped(nq, q_axes) < 0) return LTXA_E_RANGE;
  }
  if (k) {
    int rc = check_rope_tensor(k, k_pos, nk, k_axes, k_max_pos, head_dim);
    if (rc) return rc;
    kb = mul4_capped(batch, nk, heads, int64_t(head_dim) * 2);
    if (kb < 0 || mul_capped(nk, k_axes) < 0) return LTXA_E_RANGE;
  }
  if (q && k && overlap(q, qb, k, kb)) return LTXA_E_ALIAS;
  // Grid: one thread per (token, 4 pairs); x dimension holds it.
  if (nq > (INT64_C(1) << 40) || nk > (INT64_C(1) << 40)) return LTXA_E_RANGE;
  return LTXA_OK;
}

inline int check_attn(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, int64_t batch, int32_t heads, int32_t head_dim,
                      int64_t nq, int64_t nk_pad, int64_t nk_valid, float scale) {
  if (!q || !k || !v || !o) return LTXA_E_NULL;
  if (batch < 1 || heads < 1 || nq < 1 || nk_pad < 1) return LTXA_E_SHAPE;
  if (!(head_dim == 64 || head_dim == 128)) return LTXA_E_SHAPE;
  if (nk_valid < 1 || nk_valid > nk_pad) return LTXA_E_SHAPE;
  if (!(std::isfinite(scale) && scale > 0.0f)) return LTXA_E_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && !aligned16(lse)))
    return LTXA_E_ALIGN;
  int64_t qb = mul4_capped(batch, nq, heads, int64_t(head_dim) * 2);
  int64_t kb = mul4_capped(batch, nk_pad, heads, int64_t(head_dim) * 2);
  int64_t lb = mul4_capped(batch, heads, nq, 4);
  if (qb < 0 || kb < 0 || lb < 0) return LTXA_E_RANGE;
  // Per-tile element offsets inside the kernel are 32-bit: 64 token rows of
  // heads * head_dim elements must stay below 2^31.
  if (int64_t(heads) * head_dim * 64 >= (INT64_C(1) << 31)) return LTXA_E_RANGE;
  // Grid x = ceil(nq / rows per block) * batch * heads must stay below 2^31.
  int64_t qblocks = (nq + 63) / 64;
  if (mul_capped(qblocks, mul_capped(batch, heads)) < 0 ||
      qblocks * batch * heads >= (INT64_C(1) << 31))
    return LTXA_E_RANGE;
  if (overlap(o, qb, q, qb) || overlap(o, qb, k, kb) || overlap(o, qb, v, kb)) return LTXA_E_ALIAS;
  if (lse && (overlap(lse, lb, q, qb) || overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) ||
              overlap(lse, lb, o, qb)))
    return LTXA_E_ALIAS;
  return LTXA_OK;
}

// Fused pack + rotary: src [batch, n_tokens, heads, head_dim] bf16 ->
// dst [world_size, batch, n_tokens, heads/world_size, head_dim] bf16.
inline int check_pack_rope(const void* src, const void* dst, const int32_t* pos, int64_t n_tokens,
                           int32_t axes, const double* max_pos, int64_t batch, int32_t heads,
                           int32_t head_dim, int32_t world_size, double theta) {
  if (!src || !dst) return LTXA_E_NULL;
  if (batch < 1 || heads < 1 || world_size < 1) return LTXA_E_SHAPE;
  if (head_dim < 2 || head_dim > 256 || head_dim % 2 != 0) return LTXA_E_SHAPE;
  if (!(std::isfinite(theta) && theta > 0.0)) return LTXA_E_SHAPE;
  if ((head_dim * 2) % 16 != 0) return LTXA_E_ALIGN;
  int rc = check_rope_tensor(src, pos, n_tokens, axes, max_pos, head_dim);
  if (rc) return rc;
  if (!aligned16(dst)) return LTXA_E_ALIGN;
  if (heads % world_size != 0 || n_tokens % world_size != 0) return LTXA_E_DIVISIBILITY;
  const int64_t bytes = mul4_capped(batch, n_tokens, heads, int64_t(head_dim) * 2);
  if (bytes < 0 || mul_capped(n_tokens, axes) < 0) return LTXA_E_RANGE;
  if (n_tokens > (INT64_C(1) << 40)) return LTXA_E_RANGE;
  if (overlap(src, bytes, dst, bytes)) return LTXA_E_ALIAS;
  return LTXA_OK;
}

// Attention over world_size head shards [world_size, batch, n, heads/world_size,
// head_dim] with the output in the token-major [batch, nq, heads, head_dim]
// layout: the same checks as check_attn over a batch of world_size * batch
// entries with heads/world_size heads each.
inline int check_attn_unpack(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, int64_t batch, int32_t heads, int32_t head_dim,
                             int64_t nq, int64_t nk_pad, int64_t nk_valid, float scale,
                             int32_t world_size) {
  if (!q || !k || !v || !o) return LTXA_E_NULL;
  if (batch < 1 || heads < 1 || world_size < 1) return LTXA_E_SHAPE;
  if (heads % world_size != 0) return LTXA_E_DIVISIBILITY;
  if (mul_capped(batch, world_size) < 0) return LTXA_E_RANGE;
  return check_attn(q, k, v, o, lse, batch * world_size, heads / world_size, head_dim, nq, nk_pad,
                    nk_valid, scale);
}

// Output scale of the rotary calls (ltxa_rope_opts::out_scale when not 0):
// finite and positive.
inline int check_out_scale(float out_scale) {
  return std::isfinite(out_scale) && out_scale > 0.0f ? LTXA_OK : LTXA_E_SHAPE;
}

// Options of the rotary variants; opts may be NULL (all zero).
inline int check_rope_opts(const ltxa_rope_opts* opts, int32_t heads, int32_t head_dim, int32_t axes) {
  if (!opts) return LTXA_OK;
  if (!(opts->rope_type == LTXA_ROPE_INTERLEAVED || opts->rope_type == LTXA_ROPE_SPLIT)) return LTXA_E_SHAPE;
  if (!(opts->fp64_angles == 0 || opts->fp64_angles == 1)) return LTXA_E_SHAPE;
  if (!(opts->middle == 0 || opts->middle == 1)) return LTXA_E_SHAPE;
  if (opts->out_scale != 0.0f && check_out_scale(opts->out_scale) != LTXA_OK) return LTXA_E_SHAPE;
  if (opts->grid_heads < 0 || opts->head_offset < 0) return LTXA_E_SHAPE;
  if (opts->grid_heads > 0) {
    if (int64_t(opts->head_offset) + heads > opts->grid_heads) return LTXA_E_SHAPE;
    if (int64_t(opts->grid_heads) * (head_dim / 2) / axes < 1) return LTXA_E_SHAPE;
    if (int64_t(opts->grid_heads) * (head_dim / 2) >= (INT64_C(1) << 40)) return LTXA_E_RANGE;
    if (heads > 65535) return LTXA_E_RANGE;  // grid y of the per-head kernel
  }
  if (opts->rope_type == LTXA_ROPE_SPLIT && head_dim % 16 != 0) return LTXA_E_ALIGN;
  return LTXA_OK;
}

// Angle table of the shared grid: table fp32 [n_tokens, head_dim/2, 2].
// opts may be NULL; the table holds the unscaled angles of the head-shared
// grid, so opts->grid_heads and opts->out_scale must be 0 (rope_type does not
// change a pair's angle and is only checked for validity).
inline int check_rope_angles(const int32_t* pos, int64_t n_tokens, int32_t axes, const double* max_pos,
                             int32_t head_dim, double theta, const ltxa_rope_opts* opts, const float* table) {
  if (!table) return LTXA_E_NULL;
  if (head_dim < 2 || head_dim > 256 || head_dim % 2 != 0) return LTXA_E_SHAPE;
  if (!(std::isfinite(theta) && theta > 0.0)) return LTXA_E_SHAPE;
  if ((head_dim * 2) % 16 != 0) return LTXA_E_ALIGN;
  int rc = check_rope_tensor(table, pos, n_tokens, axes, max_pos, head_dim);
  if (rc) return rc;
  rc = check_rope_opts(opts, 1, head_dim, axes);
  if (rc) return rc;
  if (opts && (opts->grid_heads != 0 || opts->out_scale != 0.0f)) return LTXA_E_SHAPE;
  const int64_t bytes = mul_capped(n_tokens, int64_t(head_dim) * 4);
  if (bytes < 0 || mul_capped(n_tokens, axes) < 0) return LTXA_E_RANGE;
  // Grid: one thread per (token, pair), 256 per workgroup, below 2^31 workgroups.
  if (n_tokens * (head_dim / 2) >= (INT64_C(1) << 39)) return LTXA_E_RANGE;
  if (overlap(table, bytes, pos, mul_capped(n_tokens, axes) * 4)) return LTXA_E_ALIAS;
  return LTXA_OK;
}

// Pack + rotary from an angle table: src [batch, n_tokens, heads, head_dim]
// bf16 -> dst [world_size, batch, n_tokens, heads/world_size, head_dim] bf16,
// table fp32 [n_tokens, head_dim/2, 2].  out_scale 0 means 1.
inline int check_pack_rope_table(const void* src, const void* dst, const float* table, int64_t n_tokens,
                                 int64_t batch, int32_t heads, int32_t head_dim, int32_t world_size,
                                 int32_t rope_type, float out_scale) {
  if (!src || !dst || !table) return LTXA_E_NULL;
  if (n_tokens < 1 || batch < 1 || heads < 1 || world_size < 1) return LTXA_E_SHAPE;
  if (head_dim < 2 || head_dim > 256 || head_dim % 2 != 0) return LTXA_E_SHAPE;
  if (!(rope_type == LTXA_ROPE_INTERLEAVED || rope_type == LTXA_ROPE_SPLIT)) return LTXA_E_SHAPE;
  if (out_scale != 0.0f && check_out_scale(out_scale) != LTXA_OK) return LTXA_E_SHAPE;
  if ((head_dim * 2) % 16 != 0) return LTXA_E_ALIGN;
  if (rope_type == LTXA_ROPE_SPLIT && head_dim % 16 != 0) return LTXA_E_ALIGN;
  if (!aligned16(src) || !aligned16(dst) || !aligned16(table)) return LTXA_E_ALIGN;
  if (heads % world_size != 0 || n_tokens % world_size != 0) return LTXA_E_DIVISIBILITY;
  const int64_t bytes = mul4_capped(batch, n_tokens, heads, int64_t(head_dim) * 2);
  const int64_t tbytes = mul_capped(n_tokens, int64_t(head_dim) * 4);
  if (bytes < 0 || tbytes < 0) return LTXA_E_RANGE;
  // Grid: world_size * ceil(batch * n_tokens * groups / 256) workgroups below 2^31.
  const int64_t groups = head_dim / (rope_type == LTXA_ROPE_SPLIT ? 16 : 8);
  const int64_t threads = mul_capped(mul_capped(batch, n_tokens), groups);
  if (threads < 0 || mul_capped((threads + 255) / 256, world_size) < 0 ||
      (threads + 255) / 256 * world_size >= (INT64_C(1) << 31))
    return LTXA_E_RANGE;
  if (overlap(src, bytes, dst, bytes) || overlap(dst, bytes, table, tbytes)) return LTXA_E_ALIAS;
  return LTXA_OK;
}

// Q and K packed and rotated by one table in one launch: each pair as for
// check_pack_rope_table, a grid of twice the workgroups, and neither
// destination may overlap the other pair's tensors (the two sources may
// overlap: they are only read).
inline int check_pack_rope_qk_table(const void* q, const void* q_dst, float q_scale, const void* k,
                                    const void* k_dst, float k_scale, const float* table, int64_t n_tokens,
                                    int64_t batch, int32_t heads, int32_t head_dim, int32_t world_size,
                                    int32_t rope_type) {
  int rc = check_pack_rope_table(q, q_dst, table, n_tokens, batch, heads, head_dim, world_size, rope_type,
                                 q_scale);
  if (rc) return rc;
  rc = check_pack_rope_table(k, k_dst, table, n_tokens, batch, heads, head_dim, world_size, rope_type, k_scale);
  if (rc) return rc;
  // One launch: twice the workgroups of one tensor, still below 2^31.
  const int64_t groups = head_dim / (rope_type == LTXA_ROPE_SPLIT ? 16 : 8);
  const int64_t threads = mul_capped(mul_capped(batch, n_tokens), groups);
  if ((threads + 255) / 256 * world_size * 2 >= (INT64_C(1) << 31)) return LTXA_E_RANGE;
  const int64_t bytes = mul4_capped(batch, n_tokens, heads, int64_t(head_dim) * 2);
  if (overlap(q_dst, bytes, k, bytes) || overlap(q_dst, bytes, k_dst, bytes) || overlap(k_dst, bytes, q, bytes))
    return LTXA_E_ALIAS;
  return LTXA_OK;
}

// One tensor rotated in place: x [batch, n_tokens, heads, head_dim] bf16.
inline int check_rope_ex(const void* x, const int32_t* pos, int64_t n_tokens, int32_t axes,
                         const double* max_pos, int64_t batch, int32_t heads, int32_t head_dim, double theta,
                         const ltxa_rope_opts* opts) {
  if (!x) return LTXA_E_NULL;
  const int rc = check_rope(x, pos, n_tokens, axes, max_pos, nullptr, nullptr, 0, 0, nullptr, batch, heads,
                            head_dim, theta);
  if (rc) return rc;
  return check_rope_opts(opts, heads, head_dim, axes);
}

// Q and K rotated in place in one launch by the same positions and options:
// q as for check_rope_ex, k non-null and disjoint from q, k_scale 0 (none)
// or finite and > 0.
inline int check_rope_qk_ex(const void* q, const void* k, const int32_t* pos, int64_t n_tokens, int32_t axes,
                            const double* max_pos, int64_t batch, int32_t heads, int32_t head_dim, double theta,
                            const ltxa_rope_opts* opts, float k_scale) {
  if (!k) return LTXA_E_NULL;
  const int rc = check_rope_ex(q, pos, n_tokens, axes, max_pos, batch, heads, head_dim, theta, opts);
  if (rc) return rc;
  if (k_scale != 0.0f && check_out_scale(k_scale) != LTXA_OK) return LTXA_E_SHAPE;
  if (!aligned16(k)) return LTXA_E_ALIGN;
  const int64_t bytes = mul4_capped(batch, n_tokens, heads, int64_t(head_dim) * 2);
  if (overlap(q, bytes, k, bytes) || overlap(k, bytes, pos, mul_capped(n_tokens, axes) * 4)) return LTXA_E_ALIAS;
  return LTXA_OK;
}

}  // namespace ltxa
