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

// Walsh-Hadamard butterfly across lanes at distance M, on values that each lane holds times its own sign
// factor: x <- x + f * x[lane ^ M], with f = -1 on the lanes whose bit M is set and +1 on the others. On the
// lanes with bit M clear this is a + b; on the others it is b - a = -(a - b), so the lane's factor changes
// sign; partners at distance M always hold the same factor (it depends on the lane bits below M only), and a
// lane's values end as its factor times the butterfly's exact results (rounding is symmetric in sign). One
// v_fmac with a DPP operand per value.
// The compiler does not fold a DPP move into an fma, so the v_fmac_f32_dpp is written out, eight values per
// statement; the leading s_nop gives the two wait states that a DPP read of a VGPR written by the previous VALU
// instruction requires (every value of the statement is read before any of them is written).
#define TQ_FMAC_DPP(i, QP) "v_fmac_f32_dpp %" #i ", %" #i ", %8 quad_perm:" QP " row_mask:0xf bank_mask:0xf\n\t"
template <int M>
__device__ __forceinline__ void wht_lane_signed8(float *x, float f) {
  static_assert(M == 1 || M == 2, "quad permutes");
#define TQ_STAGE(QP)                                                                                       \
  asm("s_nop 1\n\t" TQ_FMAC_DPP(0, QP) TQ_FMAC_DPP(1, QP) TQ_FMAC_DPP(2, QP) TQ_FMAC_DPP(3, QP)            \
          TQ_FMAC_DPP(4, QP) TQ_FMAC_DPP(5, QP) TQ_FMAC_DPP(6, QP) TQ_FMAC_DPP(7, QP)                    \
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])    \
      : "v"(f))
  if constexpr (M == 1) TQ_STAGE("[1,0,3,2]");
  else TQ_STAGE("[2,3,0,1]");
#undef TQ_STAGE
}
#undef TQ_FMAC_DPP

// Norm of a vector from its sum of squares, and the reciprocal that scales its rotated coordinates: the
// hardware square root and reciprocal (each within about one ulp). Every quantizing layout takes them this
// way, so all of them write the same bytes.
__device__ __forceinline__ void norm_and_inverse(float ss, float &n, float &inv) {
  n = __builtin_amdgcn_sqrtf(ss);
  inv = n > 0.f ? __builtin_amdgcn_rcpf(n) : 0.f;
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

// Stored codes ("sign-magnitude": top bit set unless the coordinate is negative, low bits the rank away from
// zero) for B <= 4 bits, shifted into a bit stream as they are found. For one coordinate x held by the lane
// (possibly negated, see nn_class): a = |x| * inv (inv = 1 / norm) is compared, as an integer bit pattern
// (non-negative floats order like their patterns), with the positive thresholds P1 < P2 < ... in vector
// registers; the rank is the number of thresholds at or below a (a binary search: P4, then P2 or P6, then one
// of P1 P3 P5 P7), so a value exactly on a threshold takes the larger magnitude on either side of zero. Each
// bit of the code enters the stream as w <- 2 w + bit, one v_addc_co_u32 whose carry-in is the compare's lane
// mask, top bit first, so codes pushed from the highest coordinate down land at ascending b-bit fields.
// The compiler turns this pattern into selects and ors, so it is written out. The s_nops give the two wait
// states that a VALU read of an SGPR (lane mask) written by the previous VALU instruction requires; `junk`
// takes the carry-outs.
//
// nn_class: the v_cmp_class mask of the values that are not negative coordinates: 0x3E3 (NaNs, zeros,
// positive values) where the lane holds the coordinates themselves, 0x07F (NaNs, zeros, negative values) where it
// holds them negated.
template <int B>
__device__ __forceinline__ void push_code(uint32_t &w, float x, float inv, int nn_class, const PosThresholdsV &P) {
  uint64_t nn, h4, h2, h1, junk;
  int a, t, ta, tb;
  if constexpr (B == 1) {
    asm("v_cmp_class_f32_e64 %[nn], %[x], %[cm]\n\t"
        "s_nop 1\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[nn]"
        : [w] "+v"(w), [nn] "=&s"(nn), [junk] "=&s"(junk)
        : [x] "v"(x), [cm] "v"(nn_class));
  } else if constexpr (B == 2) {
    asm("v_mul_f32_e64 %[a], |%[x]|, %[inv]\n\t"
        "v_cmp_class_f32_e64 %[nn], %[x], %[cm]\n\t"
        "v_cmp_ge_i32_e64 %[h1], %[a], %[p1]\n\t"
        "s_nop 0\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[nn]\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[h1]"
        : [w] "+v"(w), [a] "=&v"(a), [nn] "=&s"(nn), [h1] "=&s"(h1), [junk] "=&s"(junk)
        : [x] "v"(x), [inv] "v"(inv), [cm] "v"(nn_class), [p1] "v"(P.p1));
  } else if constexpr (B == 3) {
    asm("v_mul_f32_e64 %[a], |%[x]|, %[inv]\n\t"
        "v_cmp_class_f32_e64 %[nn], %[x], %[cm]\n\t"
        "v_cmp_ge_i32_e64 %[h2], %[a], %[p2]\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_e64 %[t], %[p1], %[p3], %[h2]\n\t"
        "v_cmp_ge_i32_e64 %[h1], %[a], %[t]\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[nn]\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[h2]\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[h1]"
        : [w] "+v"(w), [a] "=&v"(a), [t] "=&v"(t), [nn] "=&s"(nn), [h2] "=&s"(h2), [h1] "=&s"(h1),
          [junk] "=&s"(junk)
        : [x] "v"(x), [inv] "v"(inv), [cm] "v"(nn_class), [p1] "v"(P.p1), [p2] "v"(P.p2), [p3] "v"(P.p3));
  } else {
    static_assert(B == 4, "register search covers up to 4 bits");
    asm("v_mul_f32_e64 %[a], |%[x]|, %[inv]\n\t"
        "v_cmp_class_f32_e64 %[nn], %[x], %[cm]\n\t"
        "v_cmp_ge_i32_e64 %[h4], %[a], %[p4]\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_e64 %[t], %[p2], %[p6], %[h4]\n\t"
        "v_cmp_ge_i32_e64 %[h2], %[a], %[t]\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_e64 %[ta], %[p1], %[p3], %[h2]\n\t"
        "v_cndmask_b32_e64 %[tb], %[p5], %[p7], %[h2]\n\t"
        "v_cndmask_b32_e64 %[t], %[ta], %[tb], %[h4]\n\t"
        "v_cmp_ge_i32_e64 %[h1], %[a], %[t]\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[nn]\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[h4]\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[h2]\n\t"
        "v_addc_co_u32_e64 %[w], %[junk], %[w], %[w], %[h1]"
        : [w] "+v"(w), [a] "=&v"(a), [t] "=&v"(t), [ta] "=&v"(ta), [tb] "=&v"(tb), [nn] "=&s"(nn),
          [h4] "=&s"(h4), [h2] "=&s"(h2), [h1] "=&s"(h1), [junk] "=&s"(junk)
        : [x] "v"(x), [inv] "v"(inv), [cm] "v"(nn_class), [p1] "v"(P.p1), [p2] "v"(P.p2), [p3] "v"(P.p3),
          [p4] "v"(P.p4), [p5] "v"(P.p5), [p6] "v"(P.p6), [p7] "v"(P.p7));
  }
}

// Bits 0..15 of the result are the even bits of x (bit 2j -> bit j), bits 16..31 the odd bits (bit 2j+1 ->
// bit 16 + j): the inverse perfect shuffle of Hacker's Delight (section 7-2), four swap stages.
__host__ __device__ __forceinline__ uint32_t unshuffle_bits(uint32_t x) {
  uint32_t t;
  t = (x ^ (x >> 1)) & 0x22222222u;
  x ^= t ^ (t << 1);
  t = (x ^ (x >> 2)) & 0x0C0C0C0Cu;
  x ^= t ^ (t << 2);
  t = (x ^ (x >> 4)) & 0x00F000F0u;
  x ^= t ^ (t << 4);
  t = (x ^ (x >> 8)) & 0x0000FF00u;
  x ^= t ^ (t << 8);
  return x;
}

// x ^ (s & m) in one v_bitop3 (truth table 0x78 over the operands in the order x, s, m).
__device__ __forceinline__ uint32_t xor_masked(uint32_t x, uint32_t s, uint32_t m) {
  return __builtin_amdgcn_bitop3_b32(x, s, m, 0x78);
}

// The codebook's signs on 32 fp32 coordinates: bit k of sword set negates x[k].
__device__ __forceinline__ void apply_signs32(float *x, uint32_t sword) {
#pragma unroll
  for (int k = 0; k < 32; ++k) x[k] = __uint_as_float(xor_masked(__float_as_uint(x[k]), sword << (31 - k), 0x80000000u));
}

// 32 bf16 coordinates (16 packed dwords, coordinate 2j in the low half of d[j]) with the codebook's signs,
// widened to fp32: W is the lane's sign word deinterleaved by unshuffle_bits, so (W << (15 - j)) carries the
// signs of coordinates 2j and 2j + 1 at bits 15 and 31; one v_bitop3 negates both bf16 values of a dword.
__device__ __forceinline__ void signed_bf16_to_f32(const uint32_t *d, uint32_t W, float *x) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t u = xor_masked(d[j], W << (15 - j), 0x80008000u);
    x[2 * j] = __uint_as_float(u << 16);
    x[2 * j + 1] = __uint_as_float(u & 0xFFFF0000u);
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
