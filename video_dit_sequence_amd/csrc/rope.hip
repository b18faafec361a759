// Rotary position embedding on bf16 [batch, tokens, heads, head_dim] tensors
// (FastVideo gemma page: LTXRopeType names an INTERLEAVED pairing, channels
// (2i, 2i+1), and a SPLIT one, channels (i, i + head_dim/2);
// precompute_ltx_freqs_cis turns integer (t, x, y) positions, normalised by
// max_pos, into angles with base theta, optionally at cell middles and over
// the whole inner dimension of all heads; apply_ltx_rotary_emb multiplies
// each pair by (cos, sin)).
//
// Every kernel reads a token-major tensor and writes the rotated rows either
// back in place (ranks = 1, dst = src) or straight into the per-rank head
// shards [ranks, batch, tokens, heads/ranks, head_dim] that ltxa_sp_pack
// produces, so the exchange and the rotation cost one pass over HBM.  In
// place and packed outputs come from the same instructions, so they agree
// bit for bit.
//
// Two thread mappings, by where the angles vary:
//  * Shared grid (every head turns by the same angles).  One thread owns one
//    token and one group of 4 pairs (interleaved: 16 contiguous bytes) or 8
//    pairs (split: 16 bytes in each half of the head).  It computes the
//    cos/sin of its pairs once and applies them to every (batch, head) row
//    of that token, so the transcendentals are amortised over batch * heads
//    rows.  Lanes cover consecutive groups of consecutive tokens.  Loads and
//    stores are non-temporal: each byte is touched once.  (A mapping with
//    whole token rows per wave, which reads 1 KiB per instruction, measured
//    slower: it repeats the cos/sin for every head group.)
//    With few tokens (a short text or audio sequence) the rows of a token
//    are split over grid y, so that the launch still fills the chip.
//  * Inner grid (heads turn at different frequencies).  A workgroup owns one
//    head and a run of tokens; the head's frequencies are computed once per
//    workgroup (one fp64 pow per pair, shared through LDS), and one thread
//    owns one pair group of one token.  Lanes cover the groups of one head
//    row, then tokens.
// And a split of the shared grid into its two steps, as the page's
// precomputed frequencies split it: an angle table (cos, sin per token and
// pair) evaluated once, then a pack + rotation that reads it, for one tensor
// or for Q and K in one launch (the self-attention path).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ltxa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsInFlight = 4;
constexpr int kInnerTokensPerThread = 1;
// Threads that keep every CU busy (256 CUs x 512): a shared-grid launch with
// fewer (token, pair group) threads splits each token's rows over grid y.
constexpr int64_t kFillThreads = 256 * 512;

// cos/sin of the angle (pos + mid) * coef; fp32 or fp64 evaluation.
template <bool F64>
__device__ __forceinline__ void turn(int32_t p, double mid, double coef, float& c, float& s) {
  if constexpr (F64) {
    const double phi = (static_cast<double>(p) + mid) * coef;
    double sd, cd;
    sincos(phi, &sd, &cd);
    c = static_cast<float>(cd);
    s = static_cast<float>(sd);
  } else {
    const float phi = (static_cast<float>(p) + static_cast<float>(mid)) * static_cast<float>(coef);
    sincosf(phi, &s, &c);
  }
}

__device__ __forceinline__ void rot(float x0, float x1, float c, float s, float& y0, float& y1) {
  y0 = __builtin_fmaf(x0, c, -x1 * s);
  y1 = __builtin_fmaf(x0, s, x1 * c);
}

// Interleaved: one 16-byte word holds pairs 4g .. 4g+3 as (x0, x1) halves.
__device__ __forceinline__ u32x4 rotate_interleaved(u32x4 w, const float* c, const float* s) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y0, y1;
    rot(bf16lo_to_f32(w[i]), bf16hi_to_f32(w[i]), c[i], s[i], y0, y1);
    r[i] = pack_bf16x2(y0, y1);
  }
  return r;
}

// Split: lo holds x0 of pairs 8g .. 8g+7, hi holds their x1.
__device__ __forceinline__ void rotate_split(u32x4& lo, u32x4& hi, const float* c, const float* s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a0, a1, b0, b1;
    rot(bf16lo_to_f32(lo[i]), bf16lo_to_f32(hi[i]), c[2 * i], s[2 * i], a0, a1);
    rot(bf16hi_to_f32(lo[i]), bf16hi_to_f32(hi[i]), c[2 * i + 1], s[2 * i + 1], b0, b1);
    lo[i] = pack_bf16x2(a0, b0);
    hi[i] = pack_bf16x2(a1, b1);
  }
}

// Row base pointers of (batch entry b, token n, head h): source in the
// token-major layout, destination in the rank-sharded one (rank h / hl).
struct RowAddr {
  const uint16_t* src;
  uint16_t* dst;
};
__device__ __forceinline__ RowAddr row_addr(const uint16_t* src, uint16_t* dst, int64_t b, int64_t n,
                                            int64_t h, int64_t n_tokens, int32_t heads, int32_t hl,
                                            int64_t batch, int32_t head_dim) {
  const int64_t p = h / hl, j = h - p * hl;
  return {src + ((b * n_tokens + n) * heads + h) * head_dim,
          dst + (((p * batch + b) * n_tokens + n) * hl + j) * head_dim};
}

template <bool SPLIT>
__device__ __forceinline__ void rotate_rows(const RowAddr* a, int count, int g, int half, const float* c,
                                            const float* s) {
  if constexpr (SPLIT) {
    u32x4 lo[kRowsInFlight], hi[kRowsInFlight];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u)
      if (u < count) {
        lo[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a[u].src + 8 * g));
        hi[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a[u].src + half + 8 * g));
      }
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u)
      if (u < count) {
        rotate_split(lo[u], hi[u], c, s);
        __builtin_nontemporal_store(lo[u], reinterpret_cast<u32x4*>(a[u].dst + 8 * g));
        __builtin_nontemporal_store(hi[u], reinterpret_cast<u32x4*>(a[u].dst + half + 8 * g));
      }
  } else {
    u32x4 w[kRowsInFlight];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u)
      if (u < count) w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a[u].src + 8 * g));
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u)
      if (u < count)
        __builtin_nontemporal_store(rotate_interleaved(w[u], c, s), reinterpret_cast<u32x4*>(a[u].dst + 8 * g));
  }
}

template <bool SPLIT, bool F64>
__global__ __launch_bounds__(kThreads) void rope_shared_kernel(const uint16_t* src, uint16_t* dst,
                                                               const uint16_t* src2, uint16_t* dst2,
                                                               const int32_t* __restrict__ pos,
                                                               int64_t n_tokens, int32_t axes, int64_t batch,
                                                               int32_t heads, int32_t head_dim, int32_t ranks,
                                                               int32_t rows_per, double mid, float out_scale,
                                                               float out_scale2, RopeTable table) {
  constexpr int PPT = SPLIT ? 8 : 4;  // pairs per thread
  const int groups = head_dim / (2 * PPT);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t n = t / groups;
  const int g = static_cast<int>(t - n * groups);
  if (n >= n_tokens) return;

  float c[PPT], s[PPT], c2[PPT], s2[PPT];
#pragma unroll
  for (int e = 0; e < PPT; ++e) {
    const int pair = PPT * g + e;
    const int a = table.axis[pair];
    float cr = 1.0f, sr = 0.0f;
    if (a >= 0) turn<F64>(pos[n * axes + a], mid, table.coef[pair], cr, sr);
    // An output scale turns (cos, sin) into (k cos, k sin) once per token:
    // every row is then rotated and scaled with the same two fp32 operations
    // per value and rounded to bf16 once.  k = 1 leaves both exact.  The
    // second tensor has a scale of its own.
    c[e] = cr * out_scale;
    s[e] = sr * out_scale;
    c2[e] = cr * out_scale2;
    s2[e] = sr * out_scale2;
  }

  // This thread's chunk of the token's (batch, head) rows (grid y, rows_per
  // rows each), then (if given) the same rows of the second tensor.  Rows go
  // in (batch entry, head) order; a cursor keeps the source and destination
  // row pointers and the (b, h, rank, head-in-rank) counters up to date with
  // additions only (one divide per thread to place it at its first row).
  const int32_t hl = heads / ranks;
  const int64_t first = static_cast<int64_t>(blockIdx.y) * rows_per;
  const int64_t rows = batch * heads - first < rows_per ? batch * heads : first + rows_per;
  const int64_t row_stride = int64_t(heads) * head_dim;         // token stride of the source
  const int64_t rank_stride = batch * n_tokens * hl * head_dim;  // rank stride of the destination
  auto all_rows = [&](const uint16_t* from, uint16_t* to, const float* cs, const float* sn)
                      __attribute__((always_inline)) {
    int64_t b = first / heads;
    int32_t h = static_cast<int32_t>(first - b * heads);
    int32_t j = h % hl;
    RowAddr cur = row_addr(from, to, b, n, h, n_tokens, heads, hl, batch, head_dim);
    auto advance = [&]() __attribute__((always_inline)) {
      cur.src += head_dim;
      cur.dst += head_dim;
      if (++j == hl) {  // next rank's shard, same batch entry and token
        j = 0;
        cur.dst += rank_stride - int64_t(hl) * head_dim;
      }
      if (++h == heads) {  // next batch entry, first head
        h = 0;
        ++b;
        cur.src += (n_tokens - 1) * row_stride;
        cur.dst = to + (b * n_tokens + n) * hl * head_dim;
      }
    };
    for (int64_t r0 = first; r0 < rows; r0 += kRowsInFlight) {
      RowAddr a[kRowsInFlight];
      const int count = rows - r0 < kRowsInFlight ? static_cast<int>(rows - r0) : kRowsInFlight;
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        a[u] = cur;
        if (u < count) advance();
      }
      rotate_rows<SPLIT>(a, count, g, head_dim / 2, cs, sn);
    }
  };
  all_rows(src, dst, c, s);
  if (src2) all_rows(src2, dst2, c2, s2);
}

template <bool SPLIT, bool F64>
__global__ __launch_bounds__(kThreads) void rope_inner_kernel(const uint16_t* src, uint16_t* dst,
                                                              const uint16_t* src2, uint16_t* dst2,
                                                              const int32_t* __restrict__ pos,
                                                              int64_t n_tokens, int32_t axes, int64_t batch,
                                                              int32_t heads, int32_t head_dim, int32_t ranks,
                                                              double mid, float out_scale, float out_scale2,
                                                              RopeInner grid) {
  constexpr int PPT = SPLIT ? 8 : 4;
  const int groups = head_dim / (2 * PPT);
  const int lanes_per_token = groups;
  const int token_lanes = kThreads / lanes_per_token;
  const int g = threadIdx.x % groups;
  const int tl = threadIdx.x / groups;
  const int32_t h = blockIdx.y;

  // Frequencies of the head's pairs, one fp64 pow per pair, shared through
  // LDS: global pair gp of the grid's grid_heads * head_dim / 2 pairs has
  // axis gp / n_ax and index gp % n_ax.
  __shared__ double s_coef[128];
  __shared__ int s_axis[128];
  if (threadIdx.x < head_dim / 2) {
    const int64_t gp = (static_cast<int64_t>(grid.head_offset) + h) * (head_dim / 2) + threadIdx.x;
    const int64_t a = gp / grid.n_ax, k = gp - a * grid.n_ax;
    s_axis[threadIdx.x] = a < axes ? static_cast<int>(a) : -1;
    s_coef[threadIdx.x] =
        a < axes ? pow(grid.theta, -static_cast<double>(k) / grid.n_ax) / grid.max_pos[a < axes ? a : 0] : 0.0;
  }
  __syncthreads();
  if (tl >= token_lanes) return;
  double coef[PPT];
  int axis[PPT];
#pragma unroll
  for (int e = 0; e < PPT; ++e) {
    coef[e] = s_coef[PPT * g + e];
    axis[e] = s_axis[PPT * g + e];
  }

  const int32_t hl = heads / ranks;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kInnerTokensPerThread * token_lanes + tl;
  for (int i = 0; i < kInnerTokensPerThread; ++i) {
    const int64_t n = n0 + static_cast<int64_t>(i) * token_lanes;
    if (n >= n_tokens) break;
    float c[PPT], s[PPT], c2[PPT], s2[PPT];
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      float cr = 1.0f, sr = 0.0f;
      if (axis[e] >= 0) turn<F64>(pos[n * axes + axis[e]], mid, coef[e], cr, sr);
      c[e] = cr * out_scale;  // as in the shared-grid kernel
      s[e] = sr * out_scale;
      c2[e] = cr * out_scale2;
      s2[e] = sr * out_scale2;
    }
    // The head's rows of every batch entry; then, if given, the same rows of
    // the second tensor (K beside Q: the same angles, evaluated once).
    auto all_rows = [&](const uint16_t* from, uint16_t* to, const float* cs, const float* sn)
                        __attribute__((always_inline)) {
      for (int64_t b0 = 0; b0 < batch; b0 += kRowsInFlight) {
        RowAddr a[kRowsInFlight];
        const int count = batch - b0 < kRowsInFlight ? static_cast<int>(batch - b0) : kRowsInFlight;
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u)
          a[u] = row_addr(from, to, b0 + u, n, h, n_tokens, heads, hl, batch, head_dim);
        rotate_rows<SPLIT>(a, count, g, head_dim / 2, cs, sn);
      }
    };
    all_rows(src, dst, c, s);
    if (src2) all_rows(src2, dst2, c2, s2);
  }
}

// Angle table of the shared grid (the pages' precomputed frequencies,
// precompute_ltx_freqs_cis, applied later by apply_ltx_rotary_emb): entry
// (n, i) = (cos, sin) of pair i of token n, from the same turn() as the
// kernels above, unscaled, so a rotation read from the table equals the one
// computed in place bit for bit.  One thread per pair and block of
// kAngleTokens consecutive tokens: its schedule entry is read once and the
// block's position loads are all in flight together (one thread per (token,
// pair) waited for two dependent loads per entry: 9-10 us on a 32768-token,
// 64-pair table, where writing it takes ~2 us).
constexpr int kAngleTokens = 8;
template <bool F64>
__global__ __launch_bounds__(kThreads) void rope_angles_kernel(const int32_t* __restrict__ pos,
                                                               float2* __restrict__ out, int64_t n_tokens,
                                                               int32_t axes, int32_t half, int32_t log2_half,
                                                               double mid, RopeTable table) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  // A shift when half is a power of two (log2_half >= 0): 64-bit divides are
  // software loops.
  const int64_t blk = log2_half >= 0 ? t >> log2_half : t / half;
  const int i = static_cast<int>(t - blk * half);
  const int64_t n0 = blk * kAngleTokens;
  if (n0 >= n_tokens) return;
  const int count = n_tokens - n0 < kAngleTokens ? static_cast<int>(n_tokens - n0) : kAngleTokens;
  const int a = table.axis[i];
  float c[kAngleTokens], s[kAngleTokens];
  if (a >= 0) {
    const double coef = table.coef[i];
    int32_t p[kAngleTokens];
#pragma unroll
    for (int u = 0; u < kAngleTokens; ++u) p[u] = u < count ? pos[(n0 + u) * axes + a] : 0;
#pragma unroll
    for (int u = 0; u < kAngleTokens; ++u) turn<F64>(p[u], mid, coef, c[u], s[u]);
  } else {
#pragma unroll
    for (int u = 0; u < kAngleTokens; ++u) {
      c[u] = 1.0f;
      s[u] = 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < kAngleTokens; ++u)
    if (u < count) out[(n0 + u) * half + i] = float2{c[u], s[u]};
}

// Pack + rotary with the angles read from that table.  Layout of the plain
// pack rather than of the shared-grid kernel: one thread owns one pair group
// (16 bytes of each head row; split pairing: 16 bytes in each half) of one
// token row and rank, and rotates that rank's heads/ranks rows of it, so a
// wave reads and writes whole 16-byte columns of consecutive token rows.
// Workgroups are dealt so that the ranks of the same token rows are
// consecutive logical workgroups on one XCD, which then reads each table row
// into its L2 once (dealt round-robin, every XCD's L2 fetches the whole
// table: +9 % in a timing probe).  Measured on MI355X on the [1, 32768, 32,
// 128] -> 8 ranks tensor: 89.1-90.5 us, against 93.7-94.1 us for the
// shared-grid kernel, which computes its sin/cos itself; Q and K together in
// one launch 177 us (6.07 TB/s), against ~190 us for two shared-grid
// launches, and the table's build 6.8 us.
template <bool SPLIT, int ROW, int HL, bool TWO>
__global__ __launch_bounds__(kThreads) void rope_pack_table_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   const u32x4* __restrict__ src2,
                                                                   u32x4* __restrict__ dst2,
                                                                   const float4* __restrict__ tab,
                                                                   int64_t n_tokens, int64_t batch,
                                                                   int32_t heads, int32_t head_dim,
                                                                   int32_t ranks, int32_t nblocks,
                                                                   int32_t log2_ranks, int32_t log2_groups,
                                                                   float out_scale, float out_scale2) {
  constexpr int PPT = SPLIT ? 8 : 4;  // pairs per thread
  // ROW > 0 and HL > 0 fix the 16-byte vectors per head row (head_dim / 8)
  // and the heads per rank (a multiple of kRowsInFlight) at compile time, so
  // that the index arithmetic folds into shifts and constants.
  static_assert(HL % kRowsInFlight == 0, "whole groups of rows");
  const int row = ROW > 0 ? ROW : head_dim / 8;
  const int groups = SPLIT ? row / 2 : row;
  const int half = row * 4;
  // TWO: a second tensor of the same shape (K beside Q) in the same launch,
  // on workgroups of its own (the second half of each XCD's range).  Giving
  // one thread the rows of both tensors was 4 % slower than two launches.
  uint32_t lid = static_cast<uint32_t>(xcd_contiguous(blockIdx.x, TWO ? 2 * nblocks : nblocks));
  if constexpr (TWO) {
    if (lid >= static_cast<uint32_t>(nblocks)) {
      lid -= nblocks;
      src = src2;
      dst = dst2;
      out_scale = out_scale2;
    }
  }
  // Index arithmetic is a large part of a thread's work here: shifts when
  // the rank and group counts are powers of two (log2 >= 0), and no divide
  // by n_tokens for one batch entry.  (64-bit divides are software loops.)
  uint32_t p, blk;
  if (log2_ranks >= 0) {
    p = lid & ((1u << log2_ranks) - 1);
    blk = lid >> log2_ranks;
  } else {
    p = lid % static_cast<uint32_t>(ranks);
    blk = lid / static_cast<uint32_t>(ranks);
  }
  const int64_t t = static_cast<int64_t>(blk) * kThreads + threadIdx.x;
  int64_t r;  // token row b * n_tokens + n
  int g;
  if (log2_groups >= 0) {
    r = t >> log2_groups;
    g = static_cast<int>(t & (groups - 1));
  } else {
    r = t / groups;
    g = static_cast<int>(t - r * groups);
  }
  if (r >= batch * n_tokens) return;
  int64_t b = 0, n = r;
  if (batch > 1) {
    b = r / n_tokens;
    n = r - b * n_tokens;
  }

  // Pairs PPT g .. PPT g + PPT - 1 of token n, two per float4.  They are
  // scaled only after the first rows' loads are issued: scaling them first
  // made every thread wait for its table entries before requesting any row.
  const float4* e = tab + (n * half + PPT * g) / 2;
  float4 tv[PPT / 2];
#pragma unroll
  for (int k = 0; k < PPT / 2; ++k) tv[k] = e[k];
  float c[PPT], s[PPT];
  auto scale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < PPT / 2; ++k) {
      c[2 * k] = tv[k].x * out_scale;
      s[2 * k] = tv[k].y * out_scale;
      c[2 * k + 1] = tv[k].z * out_scale;
      s[2 * k + 1] = tv[k].w * out_scale;
    }
  };

  // Vector g (and, split, g + row / 2) of this rank's head rows: the rows
  // are consecutive in both layouts, `row` vectors apart.
  const int32_t hl = HL > 0 ? HL : heads / ranks;
  const u32x4* from = src + (r * heads + int64_t(p) * hl) * row + g;
  u32x4* to = dst + ((int64_t(p) * batch + b) * n_tokens + n) * hl * row + g;
  // Rows j0 .. j0 + count - 1: every load issued before the first rotation
  // (the compiler keeps that order: the pointers are restrict).
  auto rows = [&](int32_t j0, auto count_c, auto first_c) __attribute__((always_inline)) {
    constexpr int count = decltype(count_c)::value;
    if constexpr (SPLIT) {
      u32x4 lo[count], hi[count];
#pragma unroll
      for (int u = 0; u < count; ++u) {
        lo[u] = __builtin_nontemporal_load(from + (j0 + u) * row);
        hi[u] = __builtin_nontemporal_load(from + (j0 + u) * row + row / 2);
      }
      if constexpr (decltype(first_c)::value) scale();
#pragma unroll
      for (int u = 0; u < count; ++u) {
        rotate_split(lo[u], hi[u], c, s);
        __builtin_nontemporal_store(lo[u], to + (j0 + u) * row);
        __builtin_nontemporal_store(hi[u], to + (j0 + u) * row + row / 2);
      }
    } else {
      u32x4 w[count];
#pragma unroll
      for (int u = 0; u < count; ++u) w[u] = __builtin_nontemporal_load(from + (j0 + u) * row);
      if constexpr (decltype(first_c)::value) scale();
#pragma unroll
      for (int u = 0; u < count; ++u)
        __builtin_nontemporal_store(rotate_interleaved(w[u], c, s), to + (j0 + u) * row);
    }
  };
  using group = std::integral_constant<int, kRowsInFlight>;
  using one = std::integral_constant<int, 1>;
  int32_t j0 = 0;
  if (HL > 0 || hl >= kRowsInFlight) {
    rows(0, group{}, std::true_type{});
    j0 = kRowsInFlight;
  } else {
    scale();
  }
  for (; j0 + kRowsInFlight <= hl; j0 += kRowsInFlight) rows(j0, group{}, std::false_type{});
  if constexpr (HL == 0)
    for (; j0 < hl; ++j0) rows(j0, one{}, std::false_type{});
}

template <bool SPLIT, bool F64>
hipError_t launch_mode(const uint16_t* src, uint16_t* dst, const uint16_t* src2, uint16_t* dst2,
                       const int32_t* pos, int64_t n_tokens, int32_t axes, int64_t batch, int32_t heads,
                       int32_t head_dim, int32_t ranks, const RopeMode& mode, const RopeTable& table,
                       const RopeInner& inner, hipStream_t stream) {
  constexpr int PPT = SPLIT ? 8 : 4;
  const int groups = head_dim / (2 * PPT);
  if (!mode.inner) {
    const int64_t threads = n_tokens * groups;
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    // Few tokens: split each token's rows over grid y so that the launch
    // still fills the chip (each chunk recomputes its angles).
    const int64_t rows = batch * heads;
    int64_t chunks = (kFillThreads + threads - 1) / threads;
    const int64_t max_chunks = (rows + kRowsInFlight - 1) / kRowsInFlight;
    chunks = chunks < 1 ? 1 : chunks > max_chunks ? max_chunks : chunks;
    chunks = chunks > 65535 ? 65535 : chunks;  // grid y limit
    int64_t rows_per = (rows + chunks - 1) / chunks;
    rows_per = (rows_per + kRowsInFlight - 1) / kRowsInFlight * kRowsInFlight;
    chunks = (rows + rows_per - 1) / rows_per;
    if (rows_per > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rope_shared_kernel<SPLIT, F64>), dim3(static_cast<uint32_t>(blocks),
                       static_cast<uint32_t>(chunks)), dim3(kThreads), 0, stream, src, dst, src2, dst2, pos,
                       n_tokens, axes, batch, heads, head_dim, ranks, static_cast<int32_t>(rows_per), mode.mid,
                       mode.out_scale, mode.out_scale2, table);
  } else {
    const int64_t per_block = int64_t(kInnerTokensPerThread) * (kThreads / groups);
    const int64_t blocks = (n_tokens + per_block - 1) / per_block;
    if (blocks > 0x7fffffff || heads > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rope_inner_kernel<SPLIT, F64>), dim3(static_cast<uint32_t>(blocks), heads),
                       dim3(kThreads), 0, stream, src, dst, src2, dst2, pos, n_tokens, axes, batch, heads,
                       head_dim, ranks, mode.mid, mode.out_scale, mode.out_scale2, inner);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_any(const uint16_t* src, uint16_t* dst, const uint16_t* src2, uint16_t* dst2,
                           const int32_t* pos, int64_t n_tokens, int32_t axes, int64_t batch, int32_t heads,
                           int32_t head_dim, int32_t ranks, const RopeMode& mode, const RopeTable& table,
                           const RopeInner& inner, hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's error
  if (mode.split)
    return mode.f64 ? launch_mode<true, true>(src, dst, src2, dst2, pos, n_tokens, axes, batch, heads, head_dim,
                                              ranks, mode, table, inner, stream)
                    : launch_mode<true, false>(src, dst, src2, dst2, pos, n_tokens, axes, batch, heads, head_dim,
                                               ranks, mode, table, inner, stream);
  return mode.f64 ? launch_mode<false, true>(src, dst, src2, dst2, pos, n_tokens, axes, batch, heads, head_dim,
                                             ranks, mode, table, inner, stream)
                  : launch_mode<false, false>(src, dst, src2, dst2, pos, n_tokens, axes, batch, heads, head_dim,
                                              ranks, mode, table, inner, stream);
}


hipError_t launch_rope_angles(const int32_t* pos, float* table_out, int64_t n_tokens, int32_t axes,
                              int32_t head_dim, const RopeMode& mode, const RopeTable& table,
                              hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's error
  const int32_t half = head_dim / 2;
  const int64_t blocks = ((n_tokens + kAngleTokens - 1) / kAngleTokens * half + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  float2* out = reinterpret_cast<float2*>(table_out);
  const int32_t log2_half = (half & (half - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(half)) : -1;
  if (mode.f64)
    hipLaunchKernelGGL((rope_angles_kernel<true>), dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream,
                       pos, out, n_tokens, axes, half, log2_half, mode.mid, table);
  else
    hipLaunchKernelGGL((rope_angles_kernel<false>), dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream,
                       pos, out, n_tokens, axes, half, log2_half, mode.mid, table);
  return hipGetLastError();
}

hipError_t launch_rope_pack_table(const uint16_t* src, uint16_t* dst, const uint16_t* src2, uint16_t* dst2,
                                  const float* table, int64_t n_tokens, int64_t batch, int32_t heads,
                                  int32_t head_dim, int32_t ranks, bool split, float out_scale, float out_scale2,
                                  hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's error
  const int groups = head_dim / (split ? 16 : 8);
  const int64_t per_rank = (batch * n_tokens * groups + kThreads - 1) / kThreads;
  auto log2_or_minus1 = [](int32_t v) {
    int k = 0;
    while ((1 << k) < v) ++k;
    return (1 << k) == v ? k : -1;
  };
  const int32_t lr = log2_or_minus1(ranks), lg = log2_or_minus1(groups);
  const int64_t blocks = per_rank * ranks;
  if ((src2 ? 2 * blocks : blocks) > 0x7fffffff) return hipErrorInvalidConfiguration;
  const float4* tab = reinterpret_cast<const float4*>(table);
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  const u32x4* s2 = reinterpret_cast<const u32x4*>(src2);
  u32x4* d2 = reinterpret_cast<u32x4*>(dst2);
  // Two tensors: twice the workgroups.
  const dim3 grid(static_cast<uint32_t>(src2 ? 2 * blocks : blocks));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, s, d, s2, d2, tab, n_tokens, batch, heads,
                       head_dim, ranks, static_cast<int32_t>(blocks), lr, lg, out_scale, out_scale2);
  };
  // Specialised for the common shape, 4 heads per rank of head_dim 128 or
  // 64 (the index arithmetic of the general form costs ~1 % there); every
  // other shape takes the general form.
  const bool hl4 = heads / ranks == 4;
  auto pick = [&](auto split_c, auto two_c) {
    constexpr bool S = decltype(split_c)::value, T = decltype(two_c)::value;
    if (hl4 && head_dim == 128) go(rope_pack_table_kernel<S, 16, 4, T>);
    else if (hl4 && head_dim == 64) go(rope_pack_table_kernel<S, 8, 4, T>);
    else go(rope_pack_table_kernel<S, 0, 0, T>);
  };
  using yes = std::true_type;
  using no = std::false_type;
  if (split) src2 ? pick(yes{}, yes{}) : pick(yes{}, no{});
  else src2 ? pick(no{}, yes{}) : pick(no{}, no{});
  return hipGetLastError();
}

}  // namespace ltxa
