// Interleaved rotary embedding applied in place to a bf16 [batch, tokens,
// heads, head_dim] tensor (FastVideo gemma page: LTXRopeType INTERLEAVED
// rotates channel pairs (2i, 2i+1); precompute_ltx_freqs_cis turns integer
// (t, x, y) positions, normalised by max_pos, into angles with base theta;
// apply_ltx_rotary_emb multiplies each pair by (cos, sin)).
//
// One thread owns one token and one group of 4 pairs (16 bytes of a head
// row).  It computes the 4 angles and their cos/sin once, in fp32, and
// applies them to that 16-byte slice of every head and batch entry, so the
// transcendentals are amortised over batch * heads rows.  Lanes of a wave
// cover consecutive 16-byte slices of consecutive tokens: each head row is
// read and written in full, once, with 16-byte accesses.
//
// Two kernels share that arithmetic: rope_kernel rotates a tensor in place;
// pack_rope_kernel reads the token-major tensor and writes the rotated rows
// straight into the per-rank head shards (the layout of ltxa_sp_pack), so
// the exchange and the rotation cost one pass over HBM instead of two.  Both
// compute every output with the same instructions, so they agree bit for
// bit.
#include "common.h"
#include "kernels.h"

namespace ltxa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsInFlight = 4;

__device__ __forceinline__ u32x4 rotate4(u32x4 w, const float (&c)[4], const float (&s)[4]) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = bf16lo_to_f32(w[i]);
    const float x1 = bf16hi_to_f32(w[i]);
    const float y0 = __builtin_fmaf(x0, c[i], -x1 * s[i]);
    const float y1 = __builtin_fmaf(x0, s[i], x1 * c[i]);
    r[i] = pack_bf16x2(y0, y1);
  }
  return r;
}

// cos and sin of the 4 pairs 4g..4g+3 of token n: phi = pos[axis] * coef.
__device__ __forceinline__ void pair_angles(const RopeTable& table, const int32_t* __restrict__ pos,
                                            int64_t n, int32_t axes, int g, float (&c)[4], float (&s)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pair = 4 * g + i;
    const int a = table.axis[pair];
    c[i] = 1.0f;
    s[i] = 0.0f;
    if (a >= 0) {
      const float phi = static_cast<float>(pos[n * axes + a]) * table.coef[pair];
      sincosf(phi, &s[i], &c[i]);
    }
  }
}

__global__ __launch_bounds__(kThreads) void rope_kernel(uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ pos,
                                                        int64_t n_tokens, int32_t axes, int64_t batch,
                                                        int32_t heads, int32_t head_dim, RopeTable table) {
  const int groups = head_dim >> 3;  // 8 channels = 4 pairs per thread
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t n = t / groups;
  const int g = static_cast<int>(t - n * groups);
  if (n >= n_tokens) return;

  float c[4], s[4];
  pair_angles(table, pos, n, axes, g, c, s);

  const int64_t rows = batch * heads;
  const int64_t row_stride = head_dim;            // elements between heads of one token
  const int64_t tok_stride = int64_t(heads) * head_dim;
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsInFlight) {
    u32x4 w[kRowsInFlight];
    u32x4* p[kRowsInFlight];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int64_t r = r0 + u;
      p[u] = nullptr;
      if (r < rows) {
        const int64_t b = r / heads, h = r - b * heads;
        uint16_t* row = x + (b * n_tokens + n) * tok_stride + h * row_stride + 8 * g;
        p[u] = reinterpret_cast<u32x4*>(row);
        w[u] = *p[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u)
      if (p[u]) *p[u] = rotate4(w[u], c, s);
  }
}

// src: token-major [batch, n_tokens, heads, head_dim]; dst: per-rank shards
// [ranks, batch, n_tokens, heads/ranks, head_dim].
__global__ __launch_bounds__(kThreads) void pack_rope_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst,
                                                             const int32_t* __restrict__ pos,
                                                             int64_t n_tokens, int32_t axes, int64_t batch,
                                                             int32_t heads, int32_t head_dim, int32_t ranks,
                                                             RopeTable table) {
  const int groups = head_dim >> 3;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t n = t / groups;
  const int g = static_cast<int>(t - n * groups);
  if (n >= n_tokens) return;

  float c[4], s[4];
  pair_angles(table, pos, n, axes, g, c, s);

  const int32_t hl = heads / ranks;
  const int64_t rows = batch * heads;
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsInFlight) {
    u32x4 w[kRowsInFlight];
    u32x4* out[kRowsInFlight];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int64_t r = r0 + u;
      out[u] = nullptr;
      if (r < rows) {
        const int64_t b = r / heads, h = r - b * heads;
        const int64_t p = h / hl, j = h - p * hl;
        w[u] = *reinterpret_cast<const u32x4*>(src + ((b * n_tokens + n) * heads + h) * head_dim + 8 * g);
        out[u] = reinterpret_cast<u32x4*>(dst + (((p * batch + b) * n_tokens + n) * hl + j) * head_dim + 8 * g);
      }
    }
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u)
      if (out[u]) *out[u] = rotate4(w[u], c, s);
  }
}

}  // namespace

hipError_t launch_pack_rope(const uint16_t* src, uint16_t* dst, const int32_t* pos, int64_t n_tokens,
                            int32_t axes, int64_t batch, int32_t heads, int32_t head_dim, int32_t ranks,
                            const RopeTable& table, hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's error
  const int64_t threads = n_tokens * (head_dim / 8);
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(pack_rope_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, src,
                     dst, pos, n_tokens, axes, batch, heads, head_dim, ranks, table);
  return hipGetLastError();
}

hipError_t launch_rope(uint16_t* x, const int32_t* pos, int64_t n_tokens, int32_t axes,
                       int64_t batch, int32_t heads, int32_t head_dim, const RopeTable& table,
                       hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's error
  const int64_t threads = n_tokens * (head_dim / 8);
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(rope_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, x,
                     pos, n_tokens, axes, batch, heads, head_dim, table);
  return hipGetLastError();
}

}  // namespace ltxa
