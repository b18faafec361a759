// Key-padding-masked scaled-dot-product attention, forward, for one
// sequence-parallel rank's heads (LTX-2 "Sequence Parallelism (SP)" page:
// after the head exchange each rank runs global attention over every token
// for its heads; padded keys are masked out).  bf16 inputs, bf16 matrix-core
// products with fp32 accumulation, fp32 online softmax.  Head dimensions 64
// and 128.
//
// Work split.  One workgroup = W waves = 32 W query rows of one (batch,
// head); each wave owns 32 query rows for the whole key loop.  At least two
// waves share each SIMD, so one wave's softmax (VALU) runs while another's
// matrix instructions execute.  D = 128 uses 8-wave workgroups (256
// registers per lane: one workgroup per CU, two waves per SIMD); D = 64 uses
// 4-wave workgroups held to 168 registers, three per CU, which overlap each
// other's start and end (the D = 64 workloads have short key loops).  Keys
// stream through LDS in tiles of 64 keys, double-buffered: while tile i is
// consumed, tile i+1 is copied global -> LDS directly (buffer_load ... lds,
// no register staging).
//
// Matrix instruction.  The products run on v_mfma_f32_16x16x32_bf16.
// Measured on MI355X with random bf16 operands, it sustains 15 % more
// TFLOP/s than v_mfma_f32_32x32x16_bf16 (2088 against 1818, two waves per
// SIMD).  The reason is power, not issue: the chip lowers its clock under
// matrix load, and this form draws less per flop.  A 32-head 32768-token
// launch at D = 128 held 1.97 GHz instead of ~1.7, at ~14 % more cycles:
// the instruction count doubles, and a wave issuing these products alone
// leaves gaps.  The cross-attention launch at D = 64 gained 2-5 %.
//
// Lane layout.  Lane l = 16 g + j (g = l / 16) supplies row j of A and
// column j of B, each as 8 k values of k-slice g, and receives column j of
// C, rows 4 g + r in accumulator register r.  The kernel computes the
// transposed score tile S^T = K * Q^T (A = keys, B = queries), so all of a
// lane's scores belong to its queries, and accumulates O^T = V^T * P^T, so
// the per-query rescale is a per-lane scalar.  Per wave: 32 queries as two
// 16-query blocks qb; per 64-key tile, four 16-key blocks kb.  The S^T block
// (kb, qb) leaves lane l with query 16 qb + j and keys 16 kb + 4 g + r.
// P^T for the 32-key chunk kc and block qb is the accumulators of key blocks
// 2 kc and 2 kc + 1, as k values 0..3 and 4..7 of slice g: keys
// {32 kc + 4 g + r, 32 kc + 16 + 4 g + r}, with no lane exchange.  The V^T
// operand is read in exactly that key order with two ds_read_b64_tr_b16,
// which transpose 4 rows x 16 columns of 16-bit values across each 16-lane
// group: lane j of a group receives element j of each of the 4 rows.  A
// query's 64 keys of a tile sit in the four lanes j, 16 + j, 32 + j,
// 48 + j, so its row statistics take two exchanges (needed only for the
// first tile, a rescale and the final sum).
//
// LDS layout.  K and V tiles are row-major [64 keys][D] with the 16-byte
// chunks of row r permuted by XOR with a function of r (swz_k, swz_v), so
// that the rows read by one K fragment or one V transpose read fall in
// different banks.
//
// Softmax.  Q is pre-multiplied by scale * log2(e) (rounded to bf16 once;
// or it arrives so multiplied, from the rotary pack, and is used as given),
// so the products are log2-domain scores, and every score product starts
// from a register block holding -m: exp2 consumes the accumulator as is.
// m is the first tile's row max and is not tracked per tile: the softmax is
// invariant to the offset, and fp32/bf16 hold probabilities up to 2^127, so
// m only has to rise when a probability could leave the safe range.  After
// each tile's exponentials the lane's row sums are checked: at or above
// 2^64, or not finite, the tile's exact max becomes m, O and the sums are
// rescaled and the tile's probabilities recomputed.  With the guard at 2^64,
// P <= 2^64, O <= 2^64 * |v| * keys and the sum stay far inside fp32.  The
// probabilities feed the P*V product rounded to bf16; the row sums add them
// unrounded in fp32.  The guard tests the sums' bit patterns as integers, so
// that a NaN or infinite sum (from non-finite valid inputs) takes the same
// path on any floating-point compile flags; such rows then come out
// non-finite.
//
// Output.  Staged per wave through LDS and stored as whole rows (see the
// end of the kernel); the row addressing also lets the output land directly
// in the token-major layout the head shards came from.
//
// Masking.  Only the one tile that straddles nk_valid is masked (scores of
// keys >= nk_valid set to -inf).  Its copy goes through a buffer resource
// whose extent ends at key nk_valid - 1, so rows past it arrive as zeros and
// no padded value (NaN included) is ever read; tiles wholly past nk_valid
// are not visited.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace ltxa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kQW = 32;                // query rows per wave
constexpr int kBK = 64;                // keys per tile
constexpr int kStages = 2;             // LDS ring depth
constexpr uint32_t kSumGuardBits = 0x5f800000u;  // bits of 2^64: a lane's tile row sum at or above it raises m
// Instruction-class masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kKAhead = 3;        // K fragments in flight ahead of the products
constexpr int kVAhead = 3;        // V fragments in flight ahead of the products
// Word 3 of a raw (unformatted, unswizzled) buffer resource on gfx9-family
// chips: 32-bit data format, everything else zero.
constexpr int kBufferFlags = 0x00020000;
// s_waitcnt immediate for vmcnt(0), with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8).
constexpr short kWaitVm0 = 0x0F70;
// s_waitcnt immediate for lgkmcnt(0), vmcnt and expcnt at their maxima.
constexpr short kWaitLgkm0 = static_cast<short>(0xC07F);

template <int N>
struct Int {
  static constexpr int value = N;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Value of x held by lane l ^ mask, through the LDS crossbar.
__device__ __forceinline__ float xlane(float x, int mask) {
  const int addr = ((__lane_id() ^ mask) << 2);
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
}

// Chunk permutations of the K and V tiles: chunk c of row r is stored at
// position c ^ swz(r).  A K fragment read gives lane 16 g + j row j (mod 16)
// and chunk 4 s + g.  A V transpose read is served one 32-lane half at a
// time over the 64 four-byte banks; the half reads 8 consecutive rows, 8
// bytes of each of two adjacent chunks {2a, 2a + 1} per row.  Each choice
// below was measured with SQ_LDS_BANK_CONFLICT on MI355X: zero conflict
// cycles for both reads.
// - D = 128 (16 chunks per 256-byte row, one row per bank window): K needs
//   r % 16.  V needs each 8-row half to spread its chunk pairs over all 64
//   banks: swz_v sends the pair {2a, 2a + 1} of row r to the position pair
//   a ^ (r % 8).  Neither works for the other read: one permutation shared
//   by both tiles costs 4 conflict cycles per K read or 2 per V read (128 per
//   wave and tile with the earlier shared choice, 4 % of the 32-head
//   32768-token launch).
// - D = 64 (8 chunks per 128-byte row, two rows per bank window): r % 8
//   serves both reads.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : (r & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : (r & 7);
}

// One 16-byte-per-lane copy global -> LDS through buffer resource r: lane l
// reads byte offset voff and writes LDS bytes [dst + 16 l, +16).  (Kept out
// of lambdas: inside one, this builtin stops the host-side launch stub from
// being emitted.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, LDS_AS void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}

__device__ __forceinline__ bf16x8 lds_tr_pair(const LDS_AS char* p0, const LDS_AS char* p1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p0);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Waves per workgroup for head dimension D, and the workgroups that must fit
// on one CU at once (which bounds the registers per lane: 2 waves per SIMD
// leave 256, 3 leave 168).
template <int D>
constexpr int waves_for() {
  return D == 128 ? 8 : 4;
}
template <int W>
constexpr int min_blocks_for() {
  return W == 8 ? 1 : 3;
}

template <int D, int W>
__global__ __launch_bounds__(W * 64, min_blocks_for<W>()) void attn_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int64_t nq, int64_t nk_pad, int64_t nk_valid,
    int32_t heads, int32_t qblocks, int32_t nblocks, float scale_log2, int32_t out_batch,
    int32_t out_heads) {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  constexpr int kThreads = W * 64;
  constexpr int kBQ = W * kQW;          // query rows per workgroup
  constexpr int KS = D / 32;            // 32-channel steps of K Q^T
  constexpr int CB = D / 16;            // 16-channel blocks of O^T
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int ROW = D * 2;            // bytes per K/V row
  constexpr int TILE = kBK * ROW;       // bytes per K or V tile
  constexpr int LOADS = TILE / (kThreads * 16);  // DMA instructions per thread per tensor per tile
  static_assert(LOADS * kThreads * 16 == TILE, "tile copy covers the tile");

  // The ring: one LDS object per stage and tensor, so that the compiler can
  // tell the stage being read from the stage being filled.
  __shared__ __attribute__((aligned(1024))) char sK0[TILE], sK1[TILE];
  __shared__ __attribute__((aligned(1024))) char sV0[TILE], sV1[TILE];

  const int lid = xcd_contiguous(blockIdx.x, nblocks);
  const int bh = lid / qblocks;
  const int qb0 = lid - bh * qblocks;
  const int64_t b = bh / heads;
  const int64_t h = bh - b * heads;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;
  const int64_t rs = int64_t(heads) * D;  // elements between consecutive tokens
  const __bf16* qbase = q + (b * nq * heads + h) * D;
  const __bf16* kbase = k + (b * nk_pad * heads + h) * D;
  const __bf16* vbase = v + (b * nk_pad * heads + h) * D;
  // Output slot of (b, h): head (b / out_batch) * heads + h of output batch
  // entry b % out_batch, out_heads heads per token (the operands' own layout
  // when out_batch is the batch and out_heads the head count).  b < 2^31 by
  // the grid limit.  Both output pointers are formed here and pinned, so
  // that their kernel-argument loads complete before the key loop instead
  // of staying in flight (and being waited on) inside it.
  const int32_t ob = static_cast<int32_t>(b) % out_batch, op = static_cast<int32_t>(b) / out_batch;
  __bf16* obase = o + ((int64_t(ob) * nq * out_heads) + int64_t(op) * heads + h) * D;
  float* lbase = lse ? lse + (b * heads + h) * nq : nullptr;
  asm volatile("" : "+s"(obase), "+s"(lbase));
  const int64_t ors = int64_t(out_heads) * D;  // elements between output tokens

  const int ntiles = static_cast<int>((nk_valid + kBK - 1) / kBK);
  const int full_tiles = static_cast<int>(nk_valid / kBK);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Tile copy: DMA instruction i of this wave fills LDS bytes
  // [(wave*LOADS + i) * 1024, +1024); lane l writes 16-byte slot
  // s = (wave*LOADS + i)*64 + l = (row s / CH, position s % CH), which holds
  // the row's global chunk (position ^ swz(row)); K and V take different
  // permutations, so each lane has a source offset per tensor.  The copy goes
  // through a buffer resource whose extent ends with the last valid key: rows
  // past it read as zeros, so the padded keys are never touched.
  uint32_t cpk_off[LOADS], cpv_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int s = (wave * LOADS + i) * 64 + lane;
    const int row = s / CH;
    cpk_off[i] = static_cast<uint32_t>((row * rs + ((s % CH) ^ swz_k<D>(row)) * 8) * 2);
    cpv_off[i] = static_cast<uint32_t>((row * rs + ((s % CH) ^ swz_v<D>(row)) * 8) * 2);
  }
  auto issue_tile = [&] __device__(int t, char* dK, char* dV) __attribute__((always_inline)) {
    const int64_t first = int64_t(t) * kBK;
    const int64_t rows = nk_valid - first < kBK ? nk_valid - first : kBK;
    const uint32_t extent = static_cast<uint32_t>((rows - 1) * rs * 2 + D * 2);
    const __amdgpu_buffer_rsrc_t rk = raw_buffer(kbase + first * rs, extent);
    const __amdgpu_buffer_rsrc_t rv = raw_buffer(vbase + first * rs, extent);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      LDS_AS void* kd = (LDS_AS void*)(dK + (wave_u * LOADS + i) * 1024);
      LDS_AS void* vd = (LDS_AS void*)(dV + (wave_u * LOADS + i) * 1024);
      dma16(rk, kd, cpk_off[i]);
      dma16(rv, vd, cpv_off[i]);
    }
  };
  // Bytes a copy leaves unwritten must not hold stale NaN patterns (a V row
  // past nk_valid meets a zero probability, and 0 * NaN is NaN): each lane
  // first zeroes the 16-byte slots its own copies fill, in every stage, and
  // waits for those stores before its first copy, so no ordering between
  // waves is needed.  Tile 0 is then requested before Q is read, so that
  // the two loads' latencies overlap.
  {
    char* const ring[4] = {sK0, sK1, sV0, sV1};
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        *reinterpret_cast<u32x4*>(ring[r] + (wave * LOADS + i) * 1024 + lane * 16) = u32x4{};
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }
  issue_tile(0, sK0, sV0);

  // Q^T operands: block qb holds query row q0 + 32 wave + 16 qb + j, channels 32 s + 8 g .. +7.
  // Q is multiplied by scale * log2(e) once here (rounded back to bf16), so
  // that the products are already log2-domain scores.  (For log2-domain q
  // the factor is 1.0f, and the value passes through unchanged.)
  const int64_t qrow0 = int64_t(qb0) * kBQ + wave * kQW + j;
  bf16x8 qf[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t qrow = qrow0 + 16 * qb;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 x = qrow < nq ? *reinterpret_cast<const bf16x8*>(qbase + qrow * rs + s * 32 + g * 8) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = static_cast<__bf16>(static_cast<float>(x[e]) * scale_log2);
      qf[qb][s] = x;
    }
  }

  // LDS offsets.  K fragment (A of S^T) for key block kb, step s: row 16 kb + j, chunk 4 s + g
  // at position (4 s + g) ^ swz_k(row), which depends on row % 16 = j.  V fragment (A of
  // O^T) for channel block cb, key chunk kc: transpose reads of rows 32 kc + 4 g + j / 4 (and
  // + 16), columns 16 cb + 4 (j % 4); row % 16 = 4 g + j / 4 for all of them.
  int k_off[KS], v_off[CB];
  {
#pragma unroll
    for (int s = 0; s < KS; ++s) k_off[s] = j * ROW + (((4 * s + g) ^ swz_k<D>(j)) << 4);
    const int vr = 4 * g + (j >> 2);
    const int vs = swz_v<D>(vr);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      v_off[cb] = vr * ROW + (j & 1) * 8 + (((2 * cb + ((j & 3) >> 1)) ^ vs) << 4);
  }

  f32x4 acc[CB][2];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb][0] = acc[cb][1] = f32x4{};
  // Softmax state of the two queries of each lane.  m is the offset
  // subtracted from every log2-domain score before exp2: the first tile's
  // max, raised only by the sum guard.  The score products start from a
  // register block holding -m, so they come out already offset.  l is the
  // running sum over this lane's keys.
  float m[2] = {0.0f, 0.0f};
  float l[2] = {0.0f, 0.0f};
  f32x4 neg_m[2] = {f32x4{}, f32x4{}};

  auto compute_tile = [&] __device__(int t, const char* cK, const char* cV, auto masked, auto first)
                          __attribute__((always_inline)) {
    const LDS_AS char* lK = (const LDS_AS char*)cK;
    const LDS_AS char* lV = (const LDS_AS char*)cV;
    // Keep the stage base out of the per-lane offsets (it is folded into
    // each read's immediate offset instead of costing a register per stage).
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(k_off[s]));
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) asm volatile("" : "+v"(v_off[cb]));
    f32x4 sc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[kb][0] = neg_m[0], sc[kb][1] = neg_m[1];
    // Matrix sections run at raised wave priority: when the other wave on
    // this SIMD is in its softmax, its vector instructions fill the cycles
    // between these products instead of delaying them.  S^T: fragment i
    // (key block i % 4, channel step i / 4) feeds both query blocks; reads
    // run kKAhead fragments ahead of the products.
    __builtin_amdgcn_s_setprio(1);
    {
      bf16x8 kf[4 * KS];
#pragma unroll
      for (int i = 0; i < 4 * KS; ++i)
        kf[i] = *(const LDS_AS bf16x8*)(lK + (i & 3) * 16 * ROW + k_off[i >> 2]);
#pragma unroll
      for (int i = 0; i < 4 * KS; ++i) {
        sc[i & 3][0] = mfma16(kf[i], qf[0][i >> 2], sc[i & 3][0]);
        sc[i & 3][1] = mfma16(kf[i], qf[1][i >> 2], sc[i & 3][1]);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kKAhead, 0);
#pragma unroll
      for (int i = 0; i < 4 * KS - kKAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * kKAhead, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    if constexpr (decltype(masked)::value != 0) {
      // Key of register r in block kb is 16 kb + 4 g + r.
      const int lim = static_cast<int>(nk_valid - int64_t(t) * kBK) - 4 * g;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kb + r >= lim) sc[kb][0][r] = sc[kb][1][r] = -INFINITY;
    }
    auto tile_max = [&] __device__(int qb) __attribute__((always_inline)) {
      float a = fmaxf(sc[0][qb][0], sc[1][qb][0]);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) a = fmaxf(a, sc[kb][qb][r]);
      a = fmaxf(a, xlane(a, 16));
      return fmaxf(a, xlane(a, 32));  // tile max of the query, relative to m
    };
    auto shift = [&] __device__(float d0, float d1) __attribute__((always_inline)) {
      m[0] += d0;
      m[1] += d1;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[kb][0][r] -= d0;
          sc[kb][1][r] -= d1;
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        neg_m[0][r] = -m[0];
        neg_m[1][r] = -m[1];
      }
    };
    if constexpr (decltype(first)::value != 0) shift(tile_max(0), tile_max(1));
    // Probabilities: exp2 of the offset scores, rounded to bf16 for the P*V
    // product.  The row sums add the unrounded fp32 values with plain adds.
    // (Measured on MI355X: v_dot2c_f32_bf16, which would sum the bf16
    // values, does not overlap the matrix instructions, while fp32 adds do.)
    float sum0 = 0.0f, sum1 = 0.0f;
    bf16x8 pf[2][2];
    auto probs = [&] __device__() __attribute__((always_inline)) {
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a0 = __builtin_amdgcn_exp2f(sc[2 * kc][0][r]);
          const float a1 = __builtin_amdgcn_exp2f(sc[2 * kc + 1][0][r]);
          const float b0 = __builtin_amdgcn_exp2f(sc[2 * kc][1][r]);
          const float b1 = __builtin_amdgcn_exp2f(sc[2 * kc + 1][1][r]);
          pf[kc][0][r] = static_cast<__bf16>(a0);
          pf[kc][0][r + 4] = static_cast<__bf16>(a1);
          pf[kc][1][r] = static_cast<__bf16>(b0);
          pf[kc][1][r + 4] = static_cast<__bf16>(b1);
          s0 += a0;
          s0 += a1;
          s1 += b0;
          s1 += b1;
        }
      sum0 = s0;
      sum1 = s1;
    };
    probs();
    // m is only raised when a probability could leave the safe range (a
    // lane's sum at or above 2^64, +inf or NaN: with the sign bit cleared,
    // exactly the patterns that compare at or above kSumGuardBits as
    // unsigned integers).  Then the tile's exact max becomes the new m, the
    // accumulated state is rescaled and the probabilities are recomputed;
    // P*V has not consumed them yet.
    const uint32_t worst = (__builtin_bit_cast(uint32_t, sum0) & 0x7fffffffu) >
                                   (__builtin_bit_cast(uint32_t, sum1) & 0x7fffffffu)
                               ? (__builtin_bit_cast(uint32_t, sum0) & 0x7fffffffu)
                               : (__builtin_bit_cast(uint32_t, sum1) & 0x7fffffffu);
    if (__builtin_amdgcn_ballot_w64(worst >= kSumGuardBits)) {
      const float d0 = fmaxf(tile_max(0), 0.0f), d1 = fmaxf(tile_max(1), 0.0f);
      const float a0 = __builtin_amdgcn_exp2f(-d0), a1 = __builtin_amdgcn_exp2f(-d1);
      l[0] *= a0;
      l[1] *= a1;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        acc[cb][0] *= a0;
        acc[cb][1] *= a1;
      }
      shift(d0, d1);
      probs();
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    bf16x8 vf[2 * CB];
#pragma unroll
    for (int i = 0; i < 2 * CB; ++i) {
      const int kc = i / CB, cb = i % CB;
      vf[i] = lds_tr_pair(lV + kc * 32 * ROW + v_off[cb], lV + kc * 32 * ROW + 16 * ROW + v_off[cb]);
    }
#pragma unroll
    for (int i = 0; i < 2 * CB; ++i) {
      const int kc = i / CB, cb = i % CB;
      acc[cb][0] = mfma16(vf[i], pf[kc][0], acc[cb][0]);
      acc[cb][1] = mfma16(vf[i], pf[kc][1], acc[cb][1]);
    }
    l[0] += sum0;
    l[1] += sum1;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kVAhead, 1);
#pragma unroll
    for (int i = 0; i < 2 * CB; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 1);
      if (i + kVAhead < 2 * CB) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };

  char* const ringK[kStages] = {sK0, sK1};
  char* const ringV[kStages] = {sV0, sV1};
  // One iteration with the ring slot known at compile time: wait for tile t
  // (stage ST), then copy tile t+1 into the other stage (which held tile
  // t-1: every wave is done with it once past the barrier) and consume tile t.
  auto iteration = [&] __device__(int t, auto st, auto masked, auto first) __attribute__((always_inline)) {
    constexpr int ST = decltype(st)::value;
    constexpr int S1 = (ST + 1) % kStages;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this thread's copies of tile t landed
    __syncthreads();                         // everyone's
    if (t + 1 < ntiles) issue_tile(t + 1, ringK[S1], ringV[S1]);
    compute_tile(t, ringK[ST], ringV[ST], masked, first);
  };
  // Tile 0, which sets the offset m, runs outside the loop (with the
  // first-tile branch in the loop, the register allocator copied the -m
  // block on every tile).  Then pairs of wholly valid tiles, no masking; then
  // at most one more full tile and the one tile that straddles nk_valid.
  if (full_tiles >= 1)
    iteration(0, Int<0>{}, Int<0>{}, Int<1>{});
  else
    iteration(0, Int<0>{}, Int<1>{}, Int<1>{});
  int t = 1;
  for (; t + 2 <= full_tiles; t += 2) {
    iteration(t, Int<1>{}, Int<0>{}, Int<0>{});
    iteration(t + 1, Int<0>{}, Int<0>{}, Int<0>{});
  }
  if (t < full_tiles) {
    iteration(t, Int<1>{}, Int<0>{}, Int<0>{});
    if (t + 1 < ntiles) iteration(t + 1, Int<0>{}, Int<1>{}, Int<0>{});
  } else if (t < ntiles) {
    iteration(t, Int<1>{}, Int<1>{}, Int<0>{});
  }

  float lt[2], inv[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float x = l[qb] + xlane(l[qb], 16);
    lt[qb] = x + xlane(x, 32);
    inv[qb] = 1.0f / lt[qb];
  }
  if (lbase && g == 0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      if (qrow0 + 16 * qb < nq) lbase[qrow0 + 16 * qb] = (m[qb] + __builtin_log2f(lt[qb])) * 0.69314718055994531f;
  }

  // Output.  A lane holds 4-channel pieces of its query rows, so storing them
  // directly would scatter 8-byte writes over 16 rows per instruction; with
  // a wide token stride (the unpacked layout) the L2 then writes lines back
  // half-filled.  Instead each wave stages its 32 x D tile in LDS (the ring
  // is free once every wave has left the key loop), row-major with the
  // 16-byte chunks of row r permuted by XOR with r % CH, and writes whole
  // rows: 16 bytes per lane, 64 / CH rows per instruction.
  static_assert(2 * kQW == kBK && W <= 8, "two waves' output tiles fill one ring stage");
  __syncthreads();
  char* const stage = (wave < 2 ? sK0 : wave < 4 ? sK1 : wave < 6 ? sV0 : sV1) + (wave & 1) * (kQW * ROW);
  // Lane l holds, for local row 16 qb + j, channels 16 cb + 4 g .. + 3: 8 bytes of chunk
  // 2 cb + g / 2, half g % 2.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = 16 * qb + j;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const u32x2 w = {pack_bf16x2(acc[cb][qb][0] * inv[qb], acc[cb][qb][1] * inv[qb]),
                       pack_bf16x2(acc[cb][qb][2] * inv[qb], acc[cb][qb][3] * inv[qb])};
      const int c = 2 * cb + (g >> 1);
      *reinterpret_cast<u32x2*>(stage + r * ROW + ((c ^ (r % CH)) << 4) + (g & 1) * 8) = w;
    }
  }
  __syncthreads();
  constexpr int RPI = 64 / CH;  // rows per store instruction
  const int64_t q0 = int64_t(qb0) * kBQ + wave * kQW;
#pragma unroll
  for (int i = 0; i < kQW / RPI; ++i) {
    const int r = i * RPI + lane / CH, c = lane % CH;
    const u32x4 w = *reinterpret_cast<const u32x4*>(stage + r * ROW + ((c ^ (r % CH)) << 4));
    if (q0 + r < nq) *reinterpret_cast<u32x4*>(obase + (q0 + r) * ors + c * 8) = w;
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, float* lse, int64_t batch,
                    int32_t heads, int64_t nq, int64_t nk_pad, int64_t nk_valid, float scale,
                    int64_t out_batch, int32_t out_heads, hipStream_t stream, bool q_log2) {
  if (out_batch < 1 || out_batch > batch || batch % out_batch != 0 ||
      int64_t(out_heads) != (batch / out_batch) * heads)
    return hipErrorInvalidValue;
  (void)hipGetLastError();  // report only this launch's error
  constexpr int W = waves_for<D>();
  constexpr int kBQ = W * kQW;
  const int64_t qblocks = (nq + kBQ - 1) / kBQ;
  const int64_t nblocks = qblocks * batch * heads;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  // Log2-domain q is taken as given: x * 1.0f rounded to bf16 is x.
  const float scale_log2 = q_log2 ? 1.0f : static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipLaunchKernelGGL((attn_fwd_kernel<D, W>), dim3(static_cast<uint32_t>(nblocks)), dim3(W * 64), 0, stream,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, nq, nk_pad, nk_valid,
                     heads, static_cast<int32_t>(qblocks), static_cast<int32_t>(nblocks), scale_log2,
                     static_cast<int32_t>(out_batch), out_heads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t batch, int32_t heads, int32_t head_dim, int64_t nq, int64_t nk_pad,
                       int64_t nk_valid, float scale, int64_t out_batch, int32_t out_heads,
                       hipStream_t stream, bool q_log2) {
  if (head_dim == 128)
    return launch_d<128>(q, k, v, o, lse, batch, heads, nq, nk_pad, nk_valid, scale, out_batch, out_heads,
                         stream, q_log2);
  return launch_d<64>(q, k, v, o, lse, batch, heads, nq, nk_pad, nk_valid, scale, out_batch, out_heads,
                      stream, q_log2);
}

}  // namespace ltxa
