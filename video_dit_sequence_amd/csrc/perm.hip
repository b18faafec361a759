// Token-major <-> per-rank head-shard permutation: the one-GPU share of the
// sequence-parallel all2all (LTX-2 "Sequence Parallelism (SP)" page, "What
// it is": each rank ends up with every token for a subset of heads, and the
// exchange moves bytes only).
//
// View both tensors as rows of head blocks.  With R = batch * n_tokens token
// rows, P ranks and a head block of C vectors (heads/P * head_dim * elem
// bytes, in units of the vector width):
//   token-major : [R][P][C]      packed : [P][R][C]
// Workgroup b moves 256 consecutive vectors of rank p = b % P's packed slab
// [R][C] (contiguous on the packed side, a run of C vectors every P*C on the
// token-major side), block b / P of that slab.  Consecutive workgroups
// therefore cover every rank of the same tokens, so the workgroups in
// flight read whole token rows of the token-major tensor (one DRAM page
// after another) and write P streams.  One vector per thread, non-temporal
// load and store: both tensors stream through once.  (Walking one rank's
// slab at a time instead reads 1/P of every token row per pass, about 10 %
// slower.)
#include "common.h"
#include "kernels.h"

namespace ltxa {
namespace {

constexpr int kThreads = 256;

template <typename V, bool kPow2>
__global__ __launch_bounds__(kThreads) void perm_kernel(const V* __restrict__ src, V* __restrict__ dst,
                                                        uint64_t slab, uint64_t chunk, uint32_t log2_chunk,
                                                        uint32_t ranks, bool to_packed) {
  const uint32_t p = blockIdx.x % ranks;
  const uint64_t j = static_cast<uint64_t>(blockIdx.x / ranks) * kThreads + threadIdx.x;
  if (j >= slab) return;
  const uint64_t r = kPow2 ? (j >> log2_chunk) : (j / chunk);
  const uint64_t c = j - r * chunk;
  const uint64_t packed = p * slab + j;
  const uint64_t token = (r * ranks + p) * chunk + c;
  const V val = __builtin_nontemporal_load(src + (to_packed ? token : packed));
  __builtin_nontemporal_store(val, dst + (to_packed ? packed : token));
}

template <typename V>
hipError_t launch_width(const void* src, void* dst, const PermPlan& plan, int world_size,
                        bool to_packed, hipStream_t stream) {
  const uint64_t chunk = static_cast<uint64_t>(plan.chunk) / sizeof(V);
  const uint64_t slab = static_cast<uint64_t>(plan.rows) * chunk;
  const uint64_t gx = (slab + kThreads - 1) / kThreads * static_cast<uint64_t>(world_size);
  if (gx > 0x7fffffffull) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<uint32_t>(gx));
  const bool pow2 = (chunk & (chunk - 1)) == 0;
  uint32_t lg = 0;
  while ((uint64_t(1) << lg) < chunk) ++lg;
  if (pow2)
    hipLaunchKernelGGL((perm_kernel<V, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const V*>(src), static_cast<V*>(dst), slab, chunk, lg,
                       static_cast<uint32_t>(world_size), to_packed);
  else
    hipLaunchKernelGGL((perm_kernel<V, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const V*>(src), static_cast<V*>(dst), slab, chunk, lg,
                       static_cast<uint32_t>(world_size), to_packed);
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
