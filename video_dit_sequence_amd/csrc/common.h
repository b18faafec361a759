// Shared device-side helpers of the ltxa HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace ltxa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Workgroups are dealt to the 8 XCDs of an MI355X round-robin by launch
// index.  This maps the launch index to a logical index so that each XCD
// receives one contiguous range of logical workgroups (which then share that
// XCD's L2).  A bijection on [0, n).
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
  constexpr int kXcds = 8;
  const int per = n / kXcds, rem = n % kXcds;
  const int x = bid % kXcds, local = bid / kXcds;
  return x * per + (x < rem ? x : rem) + local;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

}  // namespace ltxa
