// Token-major <-> per-rank head-shard permutation: the one-GPU share of the
// sequence-parallel all2all (LTX-2 "Sequence Parallelism (SP)" page, "What
// it is": each rank ends up with every token for a subset of heads, and the
// exchange moves bytes only).
//
// View both tensors as rows of head blocks.  With R = batch * n_tokens token
// rows, P ranks and a head block of C vectors (heads/P * head_dim * elem
// bytes, in units of the vector width):
//   token-major : [R][P][C]      packed : [P][R][C]
// Workgroup row y of the grid is rank p; x walks rank p's packed slab
// [R][C], which is contiguous on the packed side and a run of C vectors
// every P*C on the token-major side.  Each thread moves kUnroll vectors,
// loads first, then stores, with non-temporal hints: both tensors stream
// through once.
#include "common.h"
#include "kernels.h"

namespace ltxa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <typename V, bool kPow2>
__global__ __launch_bounds__(kThreads) void perm_kernel(const V* __restrict__ src, V* __restrict__ dst,
                                                        uint64_t slab, uint64_t chunk, uint32_t log2_chunk,
                                                        uint64_t ranks, bool to_packed) {
  const uint64_t p = blockIdx.y;
  const uint64_t j0 = static_cast<uint64_t>(blockIdx.x) * (kThreads * kUnroll) + threadIdx.x;
  V val[kUnroll];
  uint64_t out[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint64_t j = j0 + static_cast<uint64_t>(u) * kThreads;
    out[u] = ~uint64_t(0);
    if (j < slab) {
      const uint64_t r = kPow2 ? (j >> log2_chunk) : (j / chunk);
      const uint64_t c = j - r * chunk;
      const uint64_t packed = p * slab + j;
      const uint64_t token = (r * ranks + p) * chunk + c;
      const uint64_t in = to_packed ? token : packed;
      out[u] = to_packed ? packed : token;
      val[u] = __builtin_nontemporal_load(src + in);
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (out[u] != ~uint64_t(0)) __builtin_nontemporal_store(val[u], dst + out[u]);
}

template <typename V>
hipError_t launch_width(const void* src, void* dst, const PermPlan& plan, int world_size,
                        bool to_packed, hipStream_t stream) {
  const uint64_t chunk = static_cast<uint64_t>(plan.chunk) / sizeof(V);
  const uint64_t slab = static_cast<uint64_t>(plan.rows) * chunk;
  const uint64_t per_block = kThreads * kUnroll;
  const uint64_t gx = (slab + per_block - 1) / per_block;
  if (gx > 0x7fffffffull) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<uint32_t>(gx), static_cast<uint32_t>(world_size));
  const bool pow2 = (chunk & (chunk - 1)) == 0;
  uint32_t lg = 0;
  while ((uint64_t(1) << lg) < chunk) ++lg;
  if (pow2)
    hipLaunchKernelGGL((perm_kernel<V, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const V*>(src), static_cast<V*>(dst), slab, chunk, lg,
                       static_cast<uint64_t>(world_size), to_packed);
  else
    hipLaunchKernelGGL((perm_kernel<V, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const V*>(src), static_cast<V*>(dst), slab, chunk, lg,
                       static_cast<uint64_t>(world_size), to_packed);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_perm(const void* src, void* dst, const PermPlan& plan, int world_size,
                       bool to_packed, hipStream_t stream) {
  (void)hipGetLastError();  // report only this launch's error
  // Widest vector that divides the head block and both base addresses.
  const uint64_t bits = static_cast<uint64_t>(plan.chunk) | reinterpret_cast<uintptr_t>(src) |
                        reinterpret_cast<uintptr_t>(dst);
  if ((bits & 15) == 0) return launch_width<u32x4>(src, dst, plan, world_size, to_packed, stream);
  if ((bits & 7) == 0) return launch_width<u32x2>(src, dst, plan, world_size, to_packed, stream);
  if ((bits & 3) == 0) return launch_width<uint32_t>(src, dst, plan, world_size, to_packed, stream);
  if ((bits & 1) == 0) return launch_width<uint16_t>(src, dst, plan, world_size, to_packed, stream);
  return launch_width<uint8_t>(src, dst, plan, world_size, to_packed, stream);
}

}  // namespace ltxa
