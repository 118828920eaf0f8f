// Device helpers of the quantize-on-write path, shared by the quantize kernel and the decode-step kernel
// (which quantizes the appended token itself): input widening, DPP lane exchanges inside 16-lane rows,
// the Walsh-Hadamard lane stages, and the register search over the positive Lloyd-Max thresholds.
#pragma once

#include <hip/hip_runtime.h>

#include "tq_common.h"
#include "tq_internal.h"

namespace tq {

typedef const __attribute__((address_space(4))) int32_t *const_i32;  // read through the scalar cache

// Eight consecutive elements of an input row (16-byte aligned) widened to fp32.
__device__ __forceinline__ void load8(const void *p, int64_t i, int dtype, float *x) {
  if (dtype == TQ_F32) {
    const float4 u = *(const float4 *)((const float *)p + i);
    const float4 w = *(const float4 *)((const float *)p + i + 4);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
  } else {
    const uint4 u = *(const uint4 *)((const uint16_t *)p + i);
    const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (dtype == TQ_BF16) {
        x[2 * k] = __uint_as_float(d[k] << 16);
        x[2 * k + 1] = __uint_as_float(d[k] & 0xFFFF0000u);
      } else {
        x[2 * k] = half_bits_to_float((uint16_t)(d[k] & 0xFFFF));
        x[2 * k + 1] = half_bits_to_float((uint16_t)(d[k] >> 16));
      }
    }
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Value of lane (lane ^ M) inside the lane's 16-lane row, M in {1, 2, 4, 8}: quad permutes for 1 and 2,
// a half-row mirror (lane ^ 7) then a quad permute (lane ^ 3) for 4, a row rotation by 8 for 8.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (M == 1) return dpp<0xB1>(v);
  else if constexpr (M == 2) return dpp<0x4E>(v);
  else if constexpr (M == 4) return dpp<0x1B>(dpp<0x141>(v));
  else {
    static_assert(M == 8, "xor distance inside a 16-lane row");
    return dpp<0x128>(v);
  }
}

// Sum over the LANES lanes of a vector's group.
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  v += xor_lane<1>(v);
  v += xor_lane<2>(v);
  v += xor_lane<4>(v);
  if constexpr (LANES == 16) v += xor_lane<8>(v);
  return v;
}

// Walsh-Hadamard butterfly across lanes at distance M: (a, b) -> (a + b, a - b).
template <int M>
__device__ __forceinline__ void wht_lanes(float *x, int lane) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float p = xor_lane<M>(x[k]);
    x[k] = (lane & M) ? (p - x[k]) : (x[k] + p);
  }
}

// The positive Lloyd-Max thresholds P1 < ... < P7 of a code of up to 4 bits (unused ones +inf), as the
// integer bit patterns of non-negative floats (which order like the floats). Named fields, not an array:
// the search below selects between values, and an array would invite a dynamically indexed (scratch) copy.
struct PosThresholds {
  int p1, p2, p3, p4, p5, p6, p7;
};

// Positive thresholds t[half-1+m], m = 1 .. half-1, of a threshold table t (t[half-1] = 0 by symmetry).
template <typename Ptr>
__device__ __forceinline__ PosThresholds pos_thresholds(Ptr t, int half) {
  auto at = [&](int m) { return m < half ? (int)t[half - 1 + m] : 0x7F800000; };
  return PosThresholds{at(1), at(2), at(3), at(4), at(5), at(6), at(7)};
}

// Magnitude part of the sign-magnitude code for B <= 4 bits: the number of positive thresholds at or below z,
// by a binary search over the 2^(B-1) - 1 ascending positive thresholds, held as per-lane (vector register)
// copies: every selection is one v_cndmask between two registers, and the thresholds are plain values, never
// a table (a selection between the fields of a scalar struct can be turned into an indexed memory copy).
struct PosThresholdsV {
  int p1, p2, p3, p4, p5, p6, p7;
};
__device__ __forceinline__ int to_vgpr(int s) {
  int v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(s));
  return v;
}
__device__ __forceinline__ PosThresholdsV thresholds_in_vgprs(const PosThresholds &P) {
  return PosThresholdsV{to_vgpr(P.p1), to_vgpr(P.p2), to_vgpr(P.p3), to_vgpr(P.p4),
                        to_vgpr(P.p5), to_vgpr(P.p6), to_vgpr(P.p7)};
}
template <int B>
__device__ __forceinline__ int magnitude_v(int z, const PosThresholdsV &P) {
  if constexpr (B == 1) {
    return 0;
  } else if constexpr (B == 2) {
    return z >= P.p1 ? 1 : 0;
  } else if constexpr (B == 3) {
    const bool h2 = z >= P.p2;
    const int t = h2 ? P.p3 : P.p1;
    return (h2 ? 2 : 0) + (z >= t ? 1 : 0);
  } else {
    static_assert(B == 4, "register search covers up to 4 bits");
    const bool h4 = z >= P.p4;
    const int t2 = h4 ? P.p6 : P.p2;
    const bool h2 = z >= t2;
    const int ta = h2 ? P.p3 : P.p1;
    const int tb = h2 ? P.p7 : P.p5;
    const int t1 = h4 ? tb : ta;
    return (h4 ? 4 : 0) + (h2 ? 2 : 0) + (z >= t1 ? 1 : 0);
  }
}

// The same count by one compare per threshold (no selection between thresholds): for callers whose
// thresholds live in vector registers, where selecting between them could be turned into an indexed
// memory copy.
template <int B>
__device__ __forceinline__ int magnitude_count(int z, const PosThresholds &P) {
  int m = 0;
  if constexpr (B >= 2) m += z >= P.p1 ? 1 : 0;
  if constexpr (B >= 3) {
    m += z >= P.p2 ? 1 : 0;
    m += z >= P.p3 ? 1 : 0;
  }
  if constexpr (B >= 4) {
    m += z >= P.p4 ? 1 : 0;
    m += z >= P.p5 ? 1 : 0;
    m += z >= P.p6 ? 1 : 0;
    m += z >= P.p7 ? 1 : 0;
  }
  return m;
}

}  // namespace tq
