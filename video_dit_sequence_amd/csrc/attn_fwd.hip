// Key-padding-masked scaled-dot-product attention, forward, for one
// sequence-parallel rank's heads (LTX-2 "Sequence Parallelism (SP)" page:
// after the head exchange each rank runs global attention over every token
// for its heads; padded keys are masked out).  bf16 inputs, bf16 matrix-core
// products with fp32 accumulation, fp32 online softmax.
//
// Work split.  One workgroup = 4 waves = 128 query rows of one (batch, head);
// each wave owns 32 query rows for the whole key loop.  Keys stream through
// LDS in tiles of 64.  The whole query block is live in registers.
//
// Matrix-core orientation.  v_mfma_f32_32x32x16_bf16 computes a 32x32 fp32
// tile C += A(32x16) * B(16x32).  Lane l supplies row (l % 32) of A and
// column (l % 32) of B, each as 8 consecutive k values starting at
// 8 * (l / 32); it receives column (l % 32) of C, rows
// 8 * (r / 4) + 4 * (l / 32) + (r % 4) in accumulator register r.
// The kernel computes the transposed score tile S^T = K * Q^T (A = 32 keys,
// B = 32 queries), so every lane holds 16 scores of ONE query: the softmax
// row statistics are mostly in-register, plus one exchange between the two
// half-waves (ds_bpermute).  The output is likewise accumulated
// transposed, O^T = V^T * P^T (A = 32 channels of V^T, B = P^T), so the
// per-query rescale is a per-lane scalar.
//
// Key order inside the P^T operand.  P^T comes straight from the S^T
// accumulator: for 16 keys of a tile (registers 8j..8j+7 of one 32-key
// block), lane half hf holds keys {4hf..4hf+3, 8+4hf..8+4hf+3} as its k
// values 0..7.  The contraction index is only summed over, so V^T is stored
// in LDS with its keys permuted the same way inside every 16-key group
// (slot 8hf + e holds key 8(e/4) + 4hf + e%4); the A operand then is one
// 16-byte LDS read.
//
// Masking.  Tiles wholly below nk_valid take no mask; the one tile that
// straddles nk_valid sets the scores of keys >= nk_valid to -inf, and the
// K/V loads of those keys are replaced by zeros, so no padded value
// (NaN included) is read.  Tiles wholly at or past nk_valid are not visited.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace ltxa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;              // query rows per wave
constexpr int kBQ = kWaves * kQW;    // query rows per workgroup
constexpr int kBK = 64;              // keys per tile

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value of x held by lane l ^ 32 (the other half-wave, which holds the other
// keys of the same query), through the LDS crossbar (ds_bpermute).
__device__ __forceinline__ float partner(float x) {
  const int addr = ((__lane_id() ^ 32) << 2);
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
}
__device__ __forceinline__ float halfwave_max(float x) { return fmaxf(x, partner(x)); }
__device__ __forceinline__ float halfwave_sum(float x) { return x + partner(x); }

// LDS slot of key kk (0..63) inside a V^T row: the 16-key groups keep their
// place, inside a group the 4-key runs go in the order 0, 2, 1, 3.
__device__ __forceinline__ int vt_slot(int kk) {
  const int g = kk & ~15, w = kk & 15;
  return g + 8 * ((w >> 2) & 1) + 4 * (w >> 3) + (w & 3);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int64_t nq, int64_t nk_pad, int64_t nk_valid,
    int32_t heads, int32_t qblocks, int32_t nblocks, float scale_log2) {
  constexpr int KS = D / 16;     // 16-channel steps of Q K^T
  constexpr int DB = D / 32;     // 32-channel blocks of O^T
  constexpr int KROW = D + 8;    // padded K row in LDS (elements)
  constexpr int VROW = kBK + 8;  // padded V^T row in LDS (elements)
  constexpr int CH = D / 8;      // 16-byte chunks per head row
  constexpr int VK = D / 32;     // keys per thread in the tile load
  static_assert(VK * (kThreads / CH) == kBK, "tile load covers the tile");

  __shared__ __attribute__((aligned(16))) __bf16 sK[kBK * KROW];
  __shared__ __attribute__((aligned(16))) __bf16 sV[D * VROW];

  const int lid = xcd_contiguous(blockIdx.x, nblocks);
  const int bh = lid / qblocks;
  const int qb = lid - bh * qblocks;
  const int64_t b = bh / heads;
  const int64_t h = bh - b * heads;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 31, hf = lane >> 5;
  const int64_t rs = int64_t(heads) * D;  // elements between consecutive tokens
  const __bf16* qbase = q + (b * nq * heads + h) * D;
  const __bf16* kbase = k + (b * nk_pad * heads + h) * D;
  const __bf16* vbase = v + (b * nk_pad * heads + h) * D;

  // Q^T operand: this lane's query row, 8 channels per 16-channel step.
  const int64_t qrow = int64_t(qb) * kBQ + wave * kQW + ln;
  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (qrow < nq)
      qf[s] = *reinterpret_cast<const bf16x8*>(qbase + qrow * rs + s * 16 + hf * 8);
    else
      qf[s] = bf16x8{};
  }

  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x16{};
  float m = -INFINITY;  // running max of scale*log2(e)*s
  float l = 0.0f;       // running sum of exp2(.) over this lane's keys

  // Tile load mapping: thread -> 16-byte chunk `ch` of VK consecutive keys.
  const int ch = tid % CH;
  const int kg = tid / CH;
  const int ntiles = static_cast<int>((nk_valid + kBK - 1) / kBK);

  u32x4 kreg[VK], vreg[VK];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < VK; ++i) {
      const int64_t key = int64_t(t) * kBK + kg * VK + i;
      if (key < nk_valid) {
        kreg[i] = *reinterpret_cast<const u32x4*>(kbase + key * rs + ch * 8);
        vreg[i] = *reinterpret_cast<const u32x4*>(vbase + key * rs + ch * 8);
      } else {
        kreg[i] = u32x4{};
        vreg[i] = u32x4{};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < VK; ++i)
      *reinterpret_cast<u32x4*>(&sK[(kg * VK + i) * KROW + ch * 8]) = kreg[i];
    // Transpose VK keys x 8 channels into 8 channel rows of VK keys.
    const int slot = vt_slot(kg * VK);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      const bool hi = e & 1;
      uint32_t words[VK / 2];
#pragma unroll
      for (int i = 0; i < VK / 2; ++i) {
        const uint32_t a = vreg[2 * i][w], c = vreg[2 * i + 1][w];
        words[i] = hi ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      }
      __bf16* dstp = &sV[(ch * 8 + e) * VROW + slot];
      if constexpr (VK == 4)
        *reinterpret_cast<u32x2*>(dstp) = u32x2{words[0], words[1]};
      else
        *reinterpret_cast<uint32_t*>(dstp) = words[0];
    }
  };

  load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);  // in flight during this tile's math

    // S^T = K * Q^T for two 32-key blocks.
    f32x16 sc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sc[mb] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sK[(mb * 32 + ln) * KROW + s * 16 + hf * 8]);
        sc[mb] = mfma32(kf, qf[s], sc[mb]);
      }
    }

    const int64_t tile0 = int64_t(t) * kBK;
    if (tile0 + kBK > nk_valid) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t key = tile0 + mb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= nk_valid) sc[mb][r] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[mb][r]);
    mx = halfwave_max(mx);
    const float m_new = fmaxf(m, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;

    float psum = 0.0f;
    bf16x8 pf[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mb][8 * j + e], scale_log2, -m_new));
          psum += p;
          pf[2 * mb + j][e] = static_cast<__bf16>(p);
        }
    l = __builtin_fmaf(l, alpha, psum);
#pragma unroll
    for (int d = 0; d < DB; ++d) acc[d] *= alpha;

    // O^T += V^T * P^T, one 16-key group at a time.
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&sV[(d * 32 + ln) * VROW + g * 16 + hf * 8]);
        acc[d] = mfma32(vf, pf[g], acc[d]);
      }
  }

  const float lt = halfwave_sum(l);
  if (qrow < nq) {
    const float inv = 1.0f / lt;
    __bf16* orow = o + (b * nq * heads + h) * D + qrow * rs;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const u32x2 w = {pack_bf16x2(acc[d][4 * rg] * inv, acc[d][4 * rg + 1] * inv),
                         pack_bf16x2(acc[d][4 * rg + 2] * inv, acc[d][4 * rg + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d * 32 + 8 * rg + 4 * hf) = w;
      }
    if (lse && hf == 0) lse[(b * heads + h) * nq + qrow] = (m + __builtin_log2f(lt)) * 0.69314718055994531f;
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, float* lse, int64_t batch,
                    int32_t heads, int64_t nq, int64_t nk_pad, int64_t nk_valid, float scale,
                    hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's error
  const int64_t qblocks = (nq + kBQ - 1) / kBQ;
  const int64_t nblocks = qblocks * batch * heads;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const float scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipLaunchKernelGGL((attn_fwd_kernel<D>), dim3(static_cast<uint32_t>(nblocks)), dim3(kThreads), 0, stream,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<__bf16*>(o), lse, nq, nk_pad, nk_valid,
                     heads, static_cast<int32_t>(qblocks), static_cast<int32_t>(nblocks), scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t batch, int32_t heads, int32_t head_dim, int64_t nq, int64_t nk_pad,
                       int64_t nk_valid, float scale, hipStream_t stream) {
  if (head_dim == 128)
    return launch_d<128>(q, k, v, o, lse, batch, heads, nq, nk_pad, nk_valid, scale, stream);
  return launch_d<64>(q, k, v, o, lse, batch, heads, nq, nk_pad, nk_valid, scale, stream);
}

}  // namespace ltxa
