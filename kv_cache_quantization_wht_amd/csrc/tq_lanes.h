// Cross-lane helpers of the attention kernels (64-wide wavefronts, 16-lane MFMA rows): reductions over the
// lanes that hold one MFMA column, butterflies for the Walsh-Hadamard transform, the fast exponential.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// 2^x on the hardware exponential unit (results below 2^-126 flush to zero; 2^-inf = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max over the lanes l, l ^ 16 (permlane16 swap: rows 0<->1 and 2<->3 of 16 lanes) and over l, l ^ 32.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16_32(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Value of lane (lane ^ H) within a wavefront, for H a power of two below 64: quad permutes for 1 and 2,
// swizzles (32-lane groups) for 4, 8, the permlane swaps for 16 and 32. No LDS memory is touched.
template <int H>
__device__ __forceinline__ float xor_partner(float v, int lane) {
  const int x = __float_as_int(v);
  if constexpr (H == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  else if constexpr (H == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  else if constexpr (H == 4 || H == 8) return __int_as_float(__builtin_amdgcn_ds_swizzle(x, (H << 10) | 0x1F));
  else if constexpr (H == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    static_assert(H == 32, "xor distance");
    const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

// One Walsh-Hadamard butterfly stage across lanes at distance H: (a, b) -> (a + b, a - b).
template <int H>
__device__ __forceinline__ float wht_stage(float x, int lane) {
  const float p = xor_partner<H>(x, lane);
  return (lane & H) ? (p - x) : (x + p);
}

// Maximum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_max(float v, int lane) {
  v = fmaxf(v, xor_partner<1>(v, lane));
  v = fmaxf(v, xor_partner<2>(v, lane));
  v = fmaxf(v, xor_partner<4>(v, lane));
  v = fmaxf(v, xor_partner<8>(v, lane));
  return max_xor32(max_xor16(v));
}

// Sum over the 64 lanes of a wavefront (the xor-butterfly tree: every lane ends with the same total).
__device__ __forceinline__ float wave_sum(float v, int lane) {
  v += xor_partner<1>(v, lane);
  v += xor_partner<2>(v, lane);
  v += xor_partner<4>(v, lane);
  v += xor_partner<8>(v, lane);
  v += xor_partner<16>(v, lane);
  return v + xor_partner<32>(v, lane);
}

}  // namespace tq
