// fp16 MFMA operands of the attention kernels: the query's hi + lo split with its power-of-two range factor,
// and the byte tables that turn packed codes into fp16 levels with v_perm lookups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_common.h"

namespace tq {

// Largest power of two sigma with max|x| * sigma < 256 (1 if x is all zero).
__device__ __forceinline__ float range_factor(float maxabs) {
  if (!(maxabs > 0.f)) return 1.0f;
  int e;
  frexpf(maxabs, &e);  // maxabs in [2^(e-1), 2^e)
  return ldexpf(1.0f, 8 - e);
}

// Range control of the value weights P' = p * ||v||, which enter the value MFMAs as fp16 hi + lo parts. The softmax
// reference keeps every p <= 1, but a value norm far from 1 (a cache of tiny or huge values, or a winning key whose
// value is zero, so that the weights that matter are far below 1) would put P' outside the fp16 range. Each column
// therefore carries a power-of-two shift 2^ev applied to its weights, its softmax sum and its value sums alike (the
// ratio, the output, does not see it): the effective reference is m_run - ev. A column whose largest weight so far
// passes 2^14 (fp16 ends below 2^16) or stays under 2^-2 is shifted so that it lies in [2^6, 2^7); hi + lo then
// carry ~22 bits of every weight within 2^-16 of the column's largest. The upward shift is capped so that
// 2^ev times the softmax sum stays finite in fp32.
constexpr float kWeightHigh = 16384.0f;
constexpr float kWeightLow = 0.25f;
constexpr int kWeightTopExp = 7;
constexpr float kWeightShiftCap = 80.0f;

// wcol: the column's largest value weight so far (> 0, the same in every lane of the column). Returns the factor
// that the column's weights and sums are multiplied by (1 when it is in range), adds its exponent to ev, and sets
// wmax to the column's largest weight after the shift (at least kWeightLow, so that a column held down by the cap
// does not ask again on every step).
__device__ __forceinline__ float weight_shift(float wcol, float &ev, float &wmax) {
  float f = 1.0f;
  if (wcol > kWeightHigh || wcol < kWeightLow) {
    int e;
    frexpf(wcol, &e);  // wcol in [2^(e-1), 2^e)
    const float sh = fminf((float)(kWeightTopExp - e), kWeightShiftCap - ev);
    f = ldexpf(1.0f, (int)sh);
    ev += sh;
  }
  wmax = fmaxf(wcol * f, kWeightLow);
  return f;
}

__device__ __forceinline__ void split_hi_lo(float x, _Float16 &hi, _Float16 &lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// p | (~s & 0x80808080): the sign bit of every byte set where bit 7 of s is clear (one v_bitop3).
__device__ __forceinline__ uint32_t or_signs(uint32_t p, uint32_t s) {
  return __builtin_amdgcn_bitop3_b32(p, s, 0x80808080u, 0xF2);
}

__device__ __forceinline__ half8_t from_dwords(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3) {
  union {
    uint32_t u[4];
    half8_t h;
  } x;
  x.u[0] = r0; x.u[1] = r1; x.u[2] = r2; x.u[3] = r3;
  return x.h;
}

// MFMA position p (0..7) of the K operand -> coordinate offset inside its 8-coordinate group.
template <int KB>
__device__ __forceinline__ constexpr int k_order(int p) {
  return (KB == 4 || KB == 3) ? ((p < 4) ? 2 * p : 2 * (p - 4) + 1) : p;
}

// Byte tables of the fp16 levels for v_perm lookups.
struct Tab {
  uint32_t lo0, lo1, hi0, hi1;
};

// 4-bit codes: the 8 magnitudes (codes 8..15 of the code-indexed table); a clear top bit negates.
__device__ __forceinline__ Tab make_tab_k4(const uint16_t *lut) {
  Tab t{0, 0, 0, 0};
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t h = lut[8 + m];
    if (m < 4) {
      t.lo0 |= (h & 0xFFu) << (8 * m);
      t.hi0 |= (h >> 8) << (8 * m);
    } else {
      t.lo1 |= (h & 0xFFu) << (8 * (m - 4));
      t.hi1 |= (h >> 8) << (8 * (m - 4));
    }
  }
  return t;
}

// 2-bit codes: the four levels by code; low bytes in lo0, high bytes in hi0.
__device__ __forceinline__ Tab make_tab_v2(const uint16_t *lut) {
  Tab t{0, 0, 0, 0};
#pragma unroll
  for (int c2 = 0; c2 < 4; ++c2) {
    t.lo0 |= ((uint32_t)lut[c2] & 0xFFu) << (8 * c2);
    t.hi0 |= ((uint32_t)lut[c2] >> 8) << (8 * c2);
  }
  return t;
}

// Eight 4-bit sign-magnitude codes (coordinate e in nibble e) -> fp16 levels in MFMA order
// e = 0,2,4,6,1,3,5,7: byte-table lookups of the magnitude, sign bit set when the code's top bit is clear.
__device__ __forceinline__ half8_t lut_k4(uint32_t w, const Tab &T) {
  const uint32_t me = w & 0x07070707u, mo = (w >> 4) & 0x07070707u;
  const uint32_t le = perm(T.lo1, T.lo0, me);
  const uint32_t he = or_signs(perm(T.hi1, T.hi0, me), w << 4);
  const uint32_t lo = perm(T.lo1, T.lo0, mo);
  const uint32_t ho = or_signs(perm(T.hi1, T.hi0, mo), w);
  return from_dwords(perm(he, le, 0x05010400u), perm(he, le, 0x07030602u), perm(ho, lo, 0x05010400u),
                     perm(ho, lo, 0x07030602u));
}

// Two 2-bit codes at bits 0-1 and 16-17 of x -> two fp16 levels.
__device__ __forceinline__ uint32_t lut_v2_pair(uint32_t x, const Tab &T) {
  return perm(T.hi0, T.lo0, (x & 0x00030003u) * 0x0101u + 0x04000400u);
}

}  // namespace tq
