// C ABI of libltxa.so (declared in include/ltxa.h): argument checks, then a
// launch on the caller's stream.  No allocation, no host synchronisation, no
// global mutable state.
#include <cmath>

#include "kernels.h"
#include "ltxa.h"
#include "validate.h"

#define LTXA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

int launch_status(hipError_t e) { return e == hipSuccess ? LTXA_OK : LTXA_E_HIP; }

// Frequencies of the head-shared rotary schedule, in fp64 on the host: with
// A axes and head_dim/2 pairs, axis a owns pairs [a*n_ax, (a+1)*n_ax), and
// pair a*n_ax + j turns by pos[a] * theta^(-j/n_ax) / max_pos[a]; the
// leftover highest pairs stay unrotated.
ltxa::RopeTable rope_table(int32_t head_dim, int32_t axes, const double* max_pos, double theta) {
  ltxa::RopeTable t;
  const int pairs = head_dim / 2;
  const int per_axis = pairs / axes;
  for (int i = 0; i < 128; ++i) {
    t.coef[i] = 0.0;
    t.axis[i] = -1;
  }
  for (int a = 0; a < axes; ++a)
    for (int j = 0; j < per_axis; ++j) {
      const int i = a * per_axis + j;
      t.coef[i] = std::pow(theta, -static_cast<double>(j) / per_axis) / max_pos[a];
      t.axis[i] = a;
    }
  return t;
}

// The same schedule laid over grid_heads * head_dim channels.
ltxa::RopeInner rope_inner(const ltxa_rope_opts* opts, int32_t head_dim, int32_t axes, const double* max_pos,
                           double theta) {
  ltxa::RopeInner g{};
  g.theta = theta;
  for (int a = 0; a < 3; ++a) g.max_pos[a] = a < axes ? max_pos[a] : 1.0;
  if (opts && opts->grid_heads > 0) {
    g.n_ax = static_cast<int32_t>(int64_t(opts->grid_heads) * (head_dim / 2) / axes);
    g.head_offset = opts->head_offset;
  }
  return g;
}

ltxa::RopeMode rope_mode(const ltxa_rope_opts* opts) {
  ltxa::RopeMode m{false, false, false, 0.0};
  if (opts) {
    m.split = opts->rope_type == LTXA_ROPE_SPLIT;
    m.inner = opts->grid_heads > 0;
    m.f64 = opts->fp64_angles != 0;
    m.mid = opts->middle ? 0.5 : 0.0;
    if (opts->out_scale != 0.0f) m.out_scale = opts->out_scale;
  }
  return m;
}

int rope_launch(const void* src, void* dst, const int32_t* pos, int64_t n_tokens, int32_t axes,
                const double* max_pos, int64_t batch, int32_t heads, int32_t head_dim, int32_t ranks,
                double theta, const ltxa_rope_opts* opts, void* stream, void* second = nullptr,
                float second_scale = 0.0f) {
  ltxa::RopeMode mode = rope_mode(opts);
  if (second_scale != 0.0f) mode.out_scale2 = second_scale;
  return launch_status(ltxa::launch_rope_any(
      static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), static_cast<const uint16_t*>(second),
      static_cast<uint16_t*>(second), pos, n_tokens, axes, batch, heads, head_dim, ranks, mode,
      rope_table(head_dim, axes, max_pos, theta), rope_inner(opts, head_dim, axes, max_pos, theta),
      static_cast<hipStream_t>(stream)));
}

// Q and K turn by the same angles when they share the position buffer, the
// token count and the per-axis extents (self-attention).
bool same_rotation(const int32_t* q_pos, int64_t nq, int32_t q_axes, const double* q_max_pos,
                   const int32_t* k_pos, int64_t nk, int32_t k_axes, const double* k_max_pos) {
  if (q_pos != k_pos || nq != nk || q_axes != k_axes) return false;
  for (int a = 0; a < q_axes; ++a)
    if (q_max_pos[a] != k_max_pos[a]) return false;
  return true;
}

}  // namespace

LTXA_EXPORT int ltxa_version(void) { return LTXA_VERSION; }

LTXA_EXPORT const char* ltxa_status_string(int status) {
  switch (status) {
    case LTXA_OK: return "ok";
    case LTXA_E_NULL: return "a required pointer is NULL";
    case LTXA_E_SHAPE: return "a size is out of range";
    case LTXA_E_DIVISIBILITY: return "heads or tokens are not divisible by world_size";
    case LTXA_E_ALIGN: return "a device pointer or row is not 16-byte aligned";
    case LTXA_E_ALIAS: return "buffers that must be distinct overlap";
    case LTXA_E_HIP: return "the HIP runtime reported a launch error";
    case LTXA_E_RANGE: return "a size overflows byte counts or grid limits";
    default: return "unknown ltxa status";
  }
}

LTXA_EXPORT int ltxa_sp_pack(const void* src, void* dst, int64_t batch, int64_t n_tokens,
                             int32_t heads, int32_t head_dim, int32_t world_size,
                             int32_t elem_bytes, void* stream) {
  ltxa::PermPlan plan;
  const int rc = ltxa::check_perm(src, dst, batch, n_tokens, heads, head_dim, world_size,
                                  elem_bytes, &plan);
  if (rc) return rc;
  return launch_status(ltxa::launch_perm(src, dst, plan, world_size, true,
                                         static_cast<hipStream_t>(stream)));
}

LTXA_EXPORT int ltxa_sp_unpack(const void* src, void* dst, int64_t batch, int64_t n_tokens,
                               int32_t heads, int32_t head_dim, int32_t world_size,
                               int32_t elem_bytes, void* stream) {
  ltxa::PermPlan plan;
  const int rc = ltxa::check_perm(src, dst, batch, n_tokens, heads, head_dim, world_size,
                                  elem_bytes, &plan);
  if (rc) return rc;
  return launch_status(ltxa::launch_perm(src, dst, plan, world_size, false,
                                         static_cast<hipStream_t>(stream)));
}

LTXA_EXPORT int ltxa_rope_qk(void* q, const int32_t* q_pos, int64_t nq, int32_t q_axes,
                             const double* q_max_pos, void* k, const int32_t* k_pos, int64_t nk,
                             int32_t k_axes, const double* k_max_pos, int64_t batch, int32_t heads,
                             int32_t head_dim, double theta, void* stream) {
  const int rc = ltxa::check_rope(q, q_pos, nq, q_axes, q_max_pos, k, k_pos, nk, k_axes, k_max_pos,
                                  batch, heads, head_dim, theta);
  if (rc) return rc;
  if (q && k && same_rotation(q_pos, nq, q_axes, q_max_pos, k_pos, nk, k_axes, k_max_pos))
    return rope_launch(q, q, q_pos, nq, q_axes, q_max_pos, batch, heads, head_dim, 1, theta, nullptr, stream, k);
  if (q) {
    const int r = rope_launch(q, q, q_pos, nq, q_axes, q_max_pos, batch, heads, head_dim, 1, theta, nullptr,
                              stream);
    if (r) return r;
  }
  if (k) return rope_launch(k, k, k_pos, nk, k_axes, k_max_pos, batch, heads, head_dim, 1, theta, nullptr, stream);
  return LTXA_OK;
}

LTXA_EXPORT int ltxa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t batch, int32_t heads, int32_t head_dim, int64_t nq,
                              int64_t nk_pad, int64_t nk_valid, float scale, void* stream) {
  const int rc = ltxa::check_attn(q, k, v, o, lse, batch, heads, head_dim, nq, nk_pad, nk_valid, scale);
  if (rc) return rc;
  return launch_status(ltxa::launch_attn(q, k, v, o, lse, batch, heads, head_dim, nq, nk_pad, nk_valid,
                                         scale, batch, heads, static_cast<hipStream_t>(stream)));
}

LTXA_EXPORT int ltxa_sp_pack_rope(const void* src, void* dst, const int32_t* pos, int64_t n_tokens,
                                  int32_t axes, const double* max_pos, int64_t batch, int32_t heads,
                                  int32_t head_dim, int32_t world_size, double theta, void* stream) {
  const int rc = ltxa::check_pack_rope(src, dst, pos, n_tokens, axes, max_pos, batch, heads, head_dim,
                                       world_size, theta);
  if (rc) return rc;
  return rope_launch(src, dst, pos, n_tokens, axes, max_pos, batch, heads, head_dim, world_size, theta, nullptr,
                     stream);
}

LTXA_EXPORT int ltxa_rope_ex(void* x, const int32_t* pos, int64_t n_tokens, int32_t axes, const double* max_pos,
                             int64_t batch, int32_t heads, int32_t head_dim, double theta,
                             const ltxa_rope_opts* opts, void* stream) {
  const int rc = ltxa::check_rope_ex(x, pos, n_tokens, axes, max_pos, batch, heads, head_dim, theta, opts);
  if (rc) return rc;
  return rope_launch(x, x, pos, n_tokens, axes, max_pos, batch, heads, head_dim, 1, theta, opts, stream);
}

LTXA_EXPORT int ltxa_rope_qk_ex(void* q, void* k, const int32_t* pos, int64_t n_tokens, int32_t axes,
                                const double* max_pos, int64_t batch, int32_t heads, int32_t head_dim,
                                double theta, const ltxa_rope_opts* opts, float k_scale, void* stream) {
  const int rc = ltxa::check_rope_qk_ex(q, k, pos, n_tokens, axes, max_pos, batch, heads, head_dim, theta, opts,
                                        k_scale);
  if (rc) return rc;
  return rope_launch(q, q, pos, n_tokens, axes, max_pos, batch, heads, head_dim, 1, theta, opts, stream, k,
                     k_scale);
}

LTXA_EXPORT int ltxa_sp_pack_rope_ex(const void* src, void* dst, const int32_t* pos, int64_t n_tokens,
                                     int32_t axes, const double* max_pos, int64_t batch, int32_t heads,
                                     int32_t head_dim, int32_t world_size, double theta,
                                     const ltxa_rope_opts* opts, void* stream) {
  int rc = ltxa::check_pack_rope(src, dst, pos, n_tokens, axes, max_pos, batch, heads, head_dim, world_size,
                                 theta);
  if (rc) return rc;
  rc = ltxa::check_rope_opts(opts, heads, head_dim, axes);
  if (rc) return rc;
  return rope_launch(src, dst, pos, n_tokens, axes, max_pos, batch, heads, head_dim, world_size, theta, opts,
                     stream);
}

LTXA_EXPORT int ltxa_rope_table(const int32_t* pos, int64_t n_tokens, int32_t axes, const double* max_pos,
                                int32_t head_dim, double theta, const ltxa_rope_opts* opts, float* table,
                                void* stream) {
  const int rc = ltxa::check_rope_angles(pos, n_tokens, axes, max_pos, head_dim, theta, opts, table);
  if (rc) return rc;
  return launch_status(ltxa::launch_rope_angles(pos, table, n_tokens, axes, head_dim, rope_mode(opts),
                                                rope_table(head_dim, axes, max_pos, theta),
                                                static_cast<hipStream_t>(stream)));
}

LTXA_EXPORT int ltxa_sp_pack_rope_table(const void* src, void* dst, const float* table, int64_t n_tokens,
                                        int64_t batch, int32_t heads, int32_t head_dim, int32_t world_size,
                                        int32_t rope_type, float out_scale, void* stream) {
  const int rc = ltxa::check_pack_rope_table(src, dst, table, n_tokens, batch, heads, head_dim, world_size,
                                             rope_type, out_scale);
  if (rc) return rc;
  return launch_status(ltxa::launch_rope_pack_table(
      static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), nullptr, nullptr, table, n_tokens, batch,
      heads, head_dim, world_size, rope_type == LTXA_ROPE_SPLIT, out_scale != 0.0f ? out_scale : 1.0f, 1.0f,
      static_cast<hipStream_t>(stream)));
}

LTXA_EXPORT int ltxa_sp_pack_rope_qk_table(const void* q, void* q_dst, float q_scale, const void* k, void* k_dst,
                                           float k_scale, const float* table, int64_t n_tokens, int64_t batch,
                                           int32_t heads, int32_t head_dim, int32_t world_size, int32_t rope_type,
                                           void* stream) {
  const int rc = ltxa::check_pack_rope_qk_table(q, q_dst, q_scale, k, k_dst, k_scale, table, n_tokens, batch,
                                                heads, head_dim, world_size, rope_type);
  if (rc) return rc;
  return launch_status(ltxa::launch_rope_pack_table(
      static_cast<const uint16_t*>(q), static_cast<uint16_t*>(q_dst), static_cast<const uint16_t*>(k),
      static_cast<uint16_t*>(k_dst), table, n_tokens, batch, heads, head_dim, world_size,
      rope_type == LTXA_ROPE_SPLIT, q_scale != 0.0f ? q_scale : 1.0f, k_scale != 0.0f ? k_scale : 1.0f,
      static_cast<hipStream_t>(stream)));
}

LTXA_EXPORT int ltxa_attn_fwd_log2q(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int64_t batch, int32_t heads, int32_t head_dim, int64_t nq, int64_t nk_pad,
                                    int64_t nk_valid, void* stream) {
  const int rc = ltxa::check_attn(q, k, v, o, lse, batch, heads, head_dim, nq, nk_pad, nk_valid, 1.0f);
  if (rc) return rc;
  return launch_status(ltxa::launch_attn(q, k, v, o, lse, batch, heads, head_dim, nq, nk_pad, nk_valid, 1.0f,
                                         batch, heads, static_cast<hipStream_t>(stream), true));
}

LTXA_EXPORT int ltxa_attn_fwd_unpack_log2q(const void* q, const void* k, const void* v, void* o, float* lse,
                                           int64_t batch, int32_t heads, int32_t head_dim, int64_t nq,
                                           int64_t nk_pad, int64_t nk_valid, int32_t world_size, void* stream) {
  const int rc = ltxa::check_attn_unpack(q, k, v, o, lse, batch, heads, head_dim, nq, nk_pad, nk_valid, 1.0f,
                                         world_size);
  if (rc) return rc;
  return launch_status(ltxa::launch_attn(q, k, v, o, lse, batch * world_size, heads / world_size, head_dim,
                                         nq, nk_pad, nk_valid, 1.0f, batch, heads,
                                         static_cast<hipStream_t>(stream), true));
}

LTXA_EXPORT int ltxa_attn_fwd_unpack(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int64_t batch, int32_t heads, int32_t head_dim, int64_t nq,
                                     int64_t nk_pad, int64_t nk_valid, float scale, int32_t world_size,
                                     void* stream) {
  const int rc = ltxa::check_attn_unpack(q, k, v, o, lse, batch, heads, head_dim, nq, nk_pad, nk_valid,
                                         scale, world_size);
  if (rc) return rc;
  return launch_status(ltxa::launch_attn(q, k, v, o, lse, batch * world_size, heads / world_size, head_dim,
                                         nq, nk_pad, nk_valid, scale, batch, heads,
                                         static_cast<hipStream_t>(stream)));
}
