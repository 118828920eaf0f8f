// Quantize-on-write ("Closing - The Three-Step Summary", Steps 1-3): for every K and V vector,
//   n = ||x||, y' = H (s * x) / n   (the rotated unit vector in N(0,1) units),
//   idx_i = #{j : y'_i >= t_j}      (Gaussian Lloyd-Max thresholds, midpoints of the fp16 levels),
//   code_i = sign-magnitude form of idx_i, pack the b-bit codes, store n as fp16, and in prod mode also
//   r = (y' - level[code]) / sqrt(d), gamma = ||r||, z_j = [(S r)_j >= 0].
// The kernels decide in fp32: the code's top bit is set unless the rotated coordinate is negative, and its
// magnitude is the number of positive thresholds at or below |y| (the thresholds are symmetric about 0, so this
// is idx_i except where |y| falls exactly on a threshold, which it then takes to the larger magnitude).
// MSE mode: one vector is handled by d/32 lanes that each own 32 consecutive coordinates: the five lowest
// Walsh-Hadamard stages run in registers, the others combine values across lanes with one DPP fmac per value.
// A lane's 32 codes are 4b whole bytes of the vector's bit stream (four whole V pieces), so each lane writes
// its own bytes. The vectors of a work-group are consecutive tokens of one head, so the records they write are
// neighbours in a page. The code width is a compile-time parameter (one uniform switch per work-group).
// The kernel is bound by its vector ALU work, so each step is shaped for instruction count: the signs are
// applied to the packed bf16 input (one xor per two coordinates), the code bits are shifted into the packed
// stream by add-with-carry, and a lane group quantizes several vectors with the next one's input in flight.
// Prod mode runs in its own kernel: the MSE steps with d/8 lanes of 8 coordinates per vector, then the
// residual sketch S r, a dense d x d product per vector, on MFMA for 16 vectors at a time (Z^T = R S^T) with
// S held in registers for a long run of tokens. Both layouts (and the decode step's append) take the norm's
// partial sums, the butterflies and the code rule in the same order, so they write the same bytes.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_common.h"
#include "tq_internal.h"
#include "tq_lanes.h"
#include "tq_quant_common.h"

namespace tq {
namespace {

struct QuantArgs {
  unsigned char *pages;
  int64_t num_slots;
  int64_t page_bytes;
  const void *in[2];
  int64_t stride[2];
  const int64_t *slots;
  int64_t n_tok;
  const unsigned char *cb[2];
  BlobOffsets cbo[2];  // section offsets inside the K and V codebook blobs
  int64_t codes_off[2], norms_off[2], qjl_off[2], gamma_off[2];
  int bits[2], mode[2];
  int H;
  int dtype;
  int which_of_y[2];  // tensor (0 = K, 1 = V) of each grid row
  const float *rot[2];  // dense-rotation launches: the K and V matrices M applied ahead of the WHT
};

constexpr int kProdChunk = 1024;  // tokens per work-group of the prod kernel (S is loaded once per work-group)
// vectors per lane group of one MSE work-group: two for codes of 1 to 4 bits; eight for 8-bit codes, whose
// work-group first builds its bucket table (below), so that the build is spread over more tokens
constexpr int kQuantPasses = 2;
constexpr int kQuantPassesWide = 8;
constexpr int quant_passes(int bits) { return bits == 8 ? kQuantPassesWide : kQuantPasses; }

// 8-bit codes: a bucket table over the bit patterns of |y| (non-negative floats order like their patterns). Bucket
// b covers the patterns [(z0 + b) << kBucketShift, (z0 + b + 1) << kBucketShift); its entry holds the pattern of the
// threshold inside it (INT_MAX if none) and the number of thresholds below it, so that the magnitude
// #{m : P_m <= |y|} is base + [pattern(|y|) >= T] as long as no bucket holds two thresholds. That is checked while
// the table is built (a bucket spans 1/64 of an octave; the Gaussian Lloyd-Max thresholds of 8-bit codes lie at
// least 1.6% apart); otherwise the binary search over the thresholds is used.
constexpr int kBucketShift = 17;
constexpr int kMaxBuckets = 1024;
struct CodeBuckets {
  const uint2 *e;
  int z0, nb;  // nb == 0: no table
};

// Every thread of the work-group calls this after s_th (the full threshold table) is in LDS.
__device__ __forceinline__ CodeBuckets build_code_buckets(const float *s_th, int half, uint2 *s_bkt) {
  const int npos = half - 1;  // positive thresholds P_m = s_th[half - 1 + m], m = 1 .. npos, ascending
  auto P = [&](int m) { return __float_as_int(s_th[half - 1 + m]); };
  const int z0 = P(1) >> kBucketShift;
  const int nb = (P(npos) >> kBucketShift) - z0 + 2;
  bool bad = nb > kMaxBuckets;
  if (!bad) {
    for (int b = threadIdx.x; b < nb; b += blockDim.x) {
      const int lo = (z0 + b) << kBucketShift, hi = lo + (1 << kBucketShift);
      int base = 0;  // #{m : P_m < lo}
      for (int st = half >> 1; st > 0; st >>= 1)
        if (base + st <= npos && P(base + st) < lo) base += st;
      int t = 0x7FFFFFFF;
      if (base < npos && P(base + 1) < hi) {
        t = P(base + 1);
        if (base + 1 < npos && P(base + 2) < hi) bad = true;
      }
      s_bkt[b] = uint2{(uint32_t)t, (uint32_t)base};
    }
  }
  bad = __syncthreads_or(bad);
  return CodeBuckets{s_bkt, z0, bad ? 0 : nb};
}

// One vector: norm, signs, rotation, codes, record write. Leaves the rotated unit vector y (N(0,1)/sqrt(d)
// units), the stored codes, whether the slot is valid and the byte offset of the record's page for the
// prod kernel's residual. BT: the code width when it is 1..4 (then every shift, search and store is fixed
// at compile time), 0 for wide codes (the width read from the arguments).
template <int D, int BT>
__device__ __forceinline__ void quantize_vector(const QuantArgs &a, int which, float *x, int64_t slot, bool active,
                                                int h, int lane, uint32_t sword, const PosThresholds &P,
                                                const float *s_th, float *y, int *code, bool &valid_out,
                                                int64_t &page_base, int &slot_off, float &norm) {
  constexpr int LANES = D / 8;
  const unsigned char *cb = a.cb[which];
  const BlobOffsets bo = a.cbo[which];
  const int b = BT ? BT : a.bits[which];
  const int half = (1 << b) >> 1;
  const bool valid = active && slot >= 0 && slot < a.num_slots;

  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss = fmaf(x[k], x[k], ss);
  ss = group_sum<LANES>(ss);
  float n, inv;
  norm_and_inverse(ss, n, inv);

  const uint32_t sbits = (sword >> ((8 * lane) & 31)) & 0xFFu;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if ((sbits >> k) & 1u) x[k] = -x[k];
  // Walsh-Hadamard butterflies (a, b) -> (a + b, a - b), lowest stride first.
#pragma unroll
  for (int hs = 1; hs < 8; hs <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (!(k & hs)) {
        float u = x[k], w = x[k + hs];
        x[k] = u + w;
        x[k + hs] = u - w;
      }
    }
  }
  wht_lanes<1>(x, lane);
  wht_lanes<2>(x, lane);
  wht_lanes<4>(x, lane);
  if constexpr (LANES == 16) wht_lanes<8>(x, lane);

  // the stored sign-magnitude code: the top bit set unless the coordinate is negative, the low bits the number
  // of positive thresholds at or below |y| (the rule of the 32-coordinate layout's push_code)
  const PosThresholdsV PV = thresholds_in_vgprs(P);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    y[k] = x[k] * inv;
    const bool neg = x[k] < 0.f;
    const int z = __float_as_int(fabsf(x[k]) * inv);
    int mag;
    if constexpr (BT >= 1) {
      mag = magnitude_v<BT>(z, PV);
    } else {  // wide codes: binary search over the positive thresholds in LDS
      mag = 0;
      for (int st = half >> 1; st > 0; st >>= 1)
        if (z >= __float_as_int(s_th[half - 1 + mag + st])) mag += st;
    }
    code[k] = neg ? mag : (half | mag);
  }

  const int64_t page = valid ? slot / TQ_PAGE_TOKENS : 0;
  const int off = valid ? (int)(slot % TQ_PAGE_TOKENS) : 0;
  unsigned char *pg = a.pages + page * a.page_bytes;
  if (valid) {
    uint64_t packed = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) packed |= (uint64_t)code[k] << (b * k);
    unsigned char *dst;
    if (which == 0)
      dst = pg + a.codes_off[0] + (int64_t)(h * TQ_PAGE_TOKENS + off) * (D * b / 8) + lane * b;
    else
      dst = pg + a.codes_off[1] + ((int64_t)(h * (D / 8) + lane) * TQ_PAGE_TOKENS + off) * b;
    if (b == 1) *dst = (unsigned char)packed;
    else if (b == 2) *(uint16_t *)dst = (uint16_t)packed;
    else if (b == 4) *(uint32_t *)dst = (uint32_t)packed;
    else if (b == 8) *(uint64_t *)dst = packed;
    else
      for (int i = 0; i < b; ++i) dst[i] = (unsigned char)(packed >> (8 * i));
    if (lane == 0)
      *(uint16_t *)(pg + a.norms_off[which] + (int64_t)(h * TQ_PAGE_TOKENS + off) * 2) = float_to_half_bits(n);
  }

  valid_out = valid;
  page_base = page * a.page_bytes;
  slot_off = off;
  norm = n;
}

// The MSE kernel's layout: a vector is handled by D / 32 lanes that each own 32 consecutive coordinates (the
// Walsh-Hadamard stages of stride 1 .. 16 in registers, 32 and 64 across lanes), so the per-vector work
// (norm, reciprocal, record addresses) is shared by fewer lanes and a lane writes 4b bytes of a K record or
// four b-byte V pieces. The norm's partial sums (8 coordinates, then pairs, then lanes) and the butterflies
// (ascending strides) are taken in the same order as the 8-coordinate layout of the prod kernel and of the
// decode step's append, so every layout writes the same bytes. x: the lane's 32 coordinates with the
// codebook's signs applied.
template <int D, int BT>
__device__ __forceinline__ void quantize_vector32(const QuantArgs &a, int which, float *x, int64_t slot, bool active,
                                                  int h, int lane, const PosThresholdsV &PV, const float *s_th,
                                                  const CodeBuckets &cbk) {
  constexpr int LANES = D / 32;
  static_assert(BT >= 1 && BT <= 8 && BT != 5 && BT != 6 && BT != 7, "MSE code widths 1, 2, 3, 4, 8");
  constexpr int half = (1 << BT) >> 1;
  const bool valid = active && slot >= 0 && slot < a.num_slots;

  float s8[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) t = fmaf(x[8 * g + k], x[8 * g + k], t);
    s8[g] = t;
  }
  float ss = (s8[0] + s8[1]) + (s8[2] + s8[3]);
  ss += xor_lane<1>(ss);
  if constexpr (LANES == 4) ss += xor_lane<2>(ss);
  float n, inv;
  norm_and_inverse(ss, n, inv);

#pragma unroll
  for (int hs = 1; hs < 32; hs <<= 1) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (!(k & hs)) {
        const float u = x[k], w = x[k + hs];
        x[k] = u + w;
        x[k + hs] = u - w;
      }
    }
  }
  // the lane stages leave every value times the lane's factor (-1)^(number of set lane bits)
  const float f1 = (lane & 1) ? -1.f : 1.f;
#pragma unroll
  for (int k = 0; k < 32; k += 8) wht_lane_signed8<1>(x + k, f1);
  bool flip = (lane & 1) != 0;
  if constexpr (LANES == 4) {
    const float f2 = (lane & 2) ? -1.f : 1.f;
#pragma unroll
    for (int k = 0; k < 32; k += 8) wht_lane_signed8<2>(x + k, f2);
    flip = flip != ((lane & 2) != 0);
  }
  // v_cmp_class mask of the values that are not negative coordinates (the lane may hold them negated)
  const int nn_class = flip ? 0x07F : 0x3E3;

  // codes (sign-magnitude), packed into the lane's 32 * b bits: for 1, 2 and 4 bits each dword's codes are
  // shifted in from its highest coordinate down; 3-bit codes straddle dwords and are placed by shifts
  constexpr int BW = BT;  // dwords of the lane's 32 * BT bit stream
  uint32_t w[BW];
  if constexpr (BT == 1 || BT == 2 || BT == 4) {
    constexpr int PER = 32 / BT;
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      uint32_t wi = 0u;
#pragma unroll
      for (int j = PER - 1; j >= 0; --j) push_code<BT>(wi, x[PER * i + j], inv, nn_class, PV);
      w[i] = wi;
    }
  } else {
#pragma unroll
    for (int i = 0; i < BW; ++i) w[i] = 0u;
    auto put = [&](int k, uint32_t code) {
      const int bit = BT * k;
      w[bit >> 5] |= code << (bit & 31);
      if ((bit & 31) + BT > 32) w[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
    };
    if constexpr (BT == 3) {
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        uint32_t code = 0u;
        push_code<3>(code, x[k], inv, nn_class, PV);
        put(k, code);
      }
    } else if (cbk.nb) {  // 8-bit codes by the bucket table: eight lookups in flight at a time
#pragma unroll
      for (int k0 = 0; k0 < 32; k0 += 8) {
        int z[8];
        uint2 e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          z[j] = __float_as_int(fabsf(x[k0 + j]) * inv);
          e[j] = cbk.e[min(max((z[j] >> kBucketShift) - cbk.z0, 0), cbk.nb - 1)];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = (int)e[j].y + (z[j] >= (int)e[j].x ? 1 : 0);
          put(k0 + j, (uint32_t)(__builtin_amdgcn_classf(x[k0 + j], nn_class) ? (half | c) : c));
        }
      }
    } else {  // 8-bit codes: binary search over the positive thresholds in LDS
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int z = __float_as_int(fabsf(x[k]) * inv);
        int c = 0;
#pragma unroll
        for (int st = half >> 1; st > 0; st >>= 1)
          if (z >= __float_as_int(s_th[half - 1 + c + st])) c += st;
        put(k, (uint32_t)(__builtin_amdgcn_classf(x[k], nn_class) ? (half | c) : c));
      }
    }
  }
  if (valid) {
    const int64_t page = slot / TQ_PAGE_TOKENS;
    const int off = (int)(slot % TQ_PAGE_TOKENS);
    unsigned char *pg = a.pages + page * a.page_bytes;
    if (which == 0) {
      uint32_t *dst = (uint32_t *)(pg + a.codes_off[0] + (int64_t)(h * TQ_PAGE_TOKENS + off) * (D * BT / 8) + lane * 4 * BT);
      if constexpr (BT == 8) {
        ((uint4 *)dst)[0] = uint4{w[0], w[1], w[2], w[3]};
        ((uint4 *)dst)[1] = uint4{w[4], w[5], w[6], w[7]};
      } else if constexpr (BT == 4) {
        *(uint4 *)dst = uint4{w[0], w[1], w[2], w[3]};
      } else if constexpr (BT == 2) {
        *(uint2 *)dst = uint2{w[0], w[1]};
      } else {
#pragma unroll
        for (int i = 0; i < BT; ++i) dst[i] = w[i];
      }
    } else {
      // piece i (codes 8i .. 8i + 7 of the lane) = bits 8 * BT * i .. of the lane's stream
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        unsigned char *dst = pg + a.codes_off[1] + ((int64_t)(h * (D / 8) + 4 * lane + i) * TQ_PAGE_TOKENS + off) * BT;
        const int bit = 8 * BT * i;
        const uint64_t two = (uint64_t)w[bit >> 5] | ((bit >> 5) + 1 < BW ? (uint64_t)w[(bit >> 5) + 1] << 32 : 0ull);
        const uint64_t piece = two >> (bit & 31);
        if constexpr (BT == 1) *dst = (unsigned char)piece;
        else if constexpr (BT == 2) *(uint16_t *)dst = (uint16_t)piece;
        else if constexpr (BT == 4) *(uint32_t *)dst = (uint32_t)piece;
        else if constexpr (BT == 8) *(uint64_t *)dst = piece;
        else {
#pragma unroll
          for (int q = 0; q < BT; ++q) dst[q] = (unsigned char)(piece >> (8 * q));
        }
      }
    }
    if (lane == 0)
      *(uint16_t *)(pg + a.norms_off[which] + (int64_t)(h * TQ_PAGE_TOKENS + off) * 2) = float_to_half_bits(n);
  }
}

// The sign word of coordinates 32 * lane .. 32 * lane + 31, and its deinterleaved form (unshuffle_bits), from the
// D / 32 words read through the scalar cache (the deinterleave runs once per wavefront on the scalar unit).
template <int D>
__device__ __forceinline__ void lane_sign_words(const unsigned char *signs, int lane, uint32_t &sword, uint32_t &W) {
  const const_i32 sw = (const_i32)signs;
  const uint32_t s0 = (uint32_t)sw[0], s1 = (uint32_t)sw[1];
  if constexpr (D == 128) {
    const uint32_t s2 = (uint32_t)sw[2], s3 = (uint32_t)sw[3];
    const uint32_t u0 = unshuffle_bits(s0), u1 = unshuffle_bits(s1), u2 = unshuffle_bits(s2), u3 = unshuffle_bits(s3);
    sword = (lane & 2) ? ((lane & 1) ? s3 : s2) : ((lane & 1) ? s1 : s0);
    W = (lane & 2) ? ((lane & 1) ? u3 : u2) : ((lane & 1) ? u1 : u0);
  } else {
    static_assert(D == 64, "head_dim 64 or 128");
    sword = (lane & 1) ? s1 : s0;
    W = (lane & 1) ? unshuffle_bits(s1) : unshuffle_bits(s0);
  }
}

// A work-group holds quant_passes(BT) * VPB consecutive tokens of one head (K or V, MSE mode): in each pass one
// vector per D / 32 lanes, the next pass's input rows already in flight (bf16 inputs).
template <int D, int BT>
__device__ __forceinline__ void quantize_tokens(const QuantArgs &a, int which, float *s_th) {
  constexpr int LANES = D / 32;
  constexpr int VPB = 256 / LANES;
  const unsigned char *cb = a.cb[which];
  const BlobOffsets bo = a.cbo[which];
  constexpr int nl = 1 << BT;
  constexpr int half = nl >> 1;

  const int lane = threadIdx.x % LANES;
  const int vl = threadIdx.x / LANES;
  const int h = blockIdx.x % a.H;
  constexpr int NP = quant_passes(BT);
  const int64_t t0 = (int64_t)(blockIdx.x / a.H) * (VPB * NP);  // first token of the work-group

  uint32_t sword, W;
  lane_sign_words<D>(cb + bo.signs, lane, sword, W);
  // positive thresholds (t[half-1] is 0 by symmetry), as integer bit patterns
  PosThresholdsV PV{};
  CodeBuckets cbk{nullptr, 0, 0};
  if constexpr (BT <= 4) {
    PV = thresholds_in_vgprs(pos_thresholds((const_i32)(cb + bo.thresholds), half));
  } else {
    __shared__ uint2 s_bkt[kMaxBuckets];
    for (int i = threadIdx.x; i < nl - 1; i += 256) s_th[i] = ((const float *)(cb + bo.thresholds))[i];
    __syncthreads();
    cbk = build_code_buckets(s_th, half, s_bkt);
  }
  const void *in = a.in[which];
  const int64_t stride = a.stride[which];
  const int64_t col = (int64_t)h * D + 32 * lane;
  if (a.dtype == TQ_BF16) {
    // the signs of coordinate pairs 2j, 2j + 1 at bits 15 and 31: one xor negates both bf16 values of a dword
    uint32_t sm[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) sm[j] = (W << (15 - j)) & 0x80008000u;
    auto fetch = [&](int64_t t, uint32_t *d, int64_t &slot) {
      const int64_t tc = t < a.n_tok ? t : 0;
      const uint4 *src = (const uint4 *)((const uint16_t *)in + tc * stride + col);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint4 u = src[g];
        d[4 * g] = u.x; d[4 * g + 1] = u.y; d[4 * g + 2] = u.z; d[4 * g + 3] = u.w;
      }
      slot = a.slots[tc];
    };
    uint32_t d[2][16];
    int64_t slot[2];
    fetch(t0 + vl, d[0], slot[0]);
#pragma unroll
    for (int v = 0; v < NP; ++v) {
      const int64_t tp = t0 + (int64_t)v * VPB;  // first token of the pass
      if (tp >= a.n_tok) break;
      if (v + 1 < NP && tp + VPB < a.n_tok) fetch(tp + VPB + vl, d[(v + 1) & 1], slot[(v + 1) & 1]);
      float x[32];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t u = d[v & 1][j] ^ sm[j];
        x[2 * j] = __uint_as_float(u << 16);
        x[2 * j + 1] = __uint_as_float(u & 0xFFFF0000u);
      }
      quantize_vector32<D, BT>(a, which, x, slot[v & 1], tp + vl < a.n_tok, h, lane, PV, s_th, cbk);
    }
  } else {
#pragma unroll 1
    for (int v = 0; v < NP; ++v) {
      const int64_t tp = t0 + (int64_t)v * VPB;
      if (tp >= a.n_tok) break;
      const int64_t t = tp + vl;
      const int64_t tc = t < a.n_tok ? t : 0;
      float x[32];
#pragma unroll
      for (int g = 0; g < 4; ++g) load8(in, tc * stride + col + 8 * g, a.dtype, x + 8 * g);
      apply_signs32(x, sword);
      quantize_vector32<D, BT>(a, which, x, a.slots[tc], t < a.n_tok, h, lane, PV, s_th, cbk);
    }
  }
}

// MSE codes of 1 to 4 bits. The 8-bit codes have a kernel of their own: their longer work-groups need more
// registers, and in one kernel that allocation would cost the narrow widths a wavefront per SIMD.
template <int D>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  __shared__ float s_th[256];
  const int which = a.which_of_y[blockIdx.y];  // 0 = K, 1 = V
  switch (a.bits[which]) {  // uniform over the work-group
    case 1: quantize_tokens<D, 1>(a, which, s_th); break;
    case 2: quantize_tokens<D, 2>(a, which, s_th); break;
    case 3: quantize_tokens<D, 3>(a, which, s_th); break;
    default: quantize_tokens<D, 4>(a, which, s_th); break;  // the launch holds widths 1..4 only
  }
}

// MSE codes of 8 bits.
template <int D>
__global__ __launch_bounds__(256) void quantize_wide_kernel(QuantArgs a) {
  __shared__ float s_th[256];
  quantize_tokens<D, 8>(a, a.which_of_y[blockIdx.y], s_th);
}

// Dense random (QR) rotation ahead of the MSE steps ("What the Paper Doesn't Tell You", Finding 4), fused:
// a work-group takes VPB consecutive tokens of one head at a time (a persistent loop over the tiles of its
// tensor). The tile's rows go to LDS as fp32; the four wavefronts rotate them by the tensor's matrix M on
// MFMA - M held in registers as fp16 high + low parts (16 M, exact to ~2^-22) for the whole launch, wavefront w
// computing the 16-coordinate output blocks w, w + 4; each row scaled by the power of two that puts its
// largest magnitude in [2^13, 2^14), split into high + low parts, three products hi.hi + hi.lo + lo.hi - into a
// second LDS tile; then the MSE steps above run on the rotated rows (the WHT with the codebook's signs follows,
// and W M is the dense rotation). The arithmetic is that of tq_rotate_rows followed by quantize_kernel on its
// fp32 output, so both routes write the same bytes; the fused one saves the fp32 round trip through HBM.
__device__ __forceinline__ void qr_split(float x, _Float16 &hi, _Float16 &lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

template <int D, int BT>
__device__ __forceinline__ void quantize_qr_tiles(const QuantArgs &a, int which, float *s_x, float *s_y,
                                                  float *s_th) {
  constexpr int LANES = D / 32;           // lanes per vector in the MSE steps
  constexpr int VPB = 256 / LANES;        // vectors of a tile
  constexpr int XS = D + 4;               // LDS row stride (floats)
  constexpr int JB = D / 32;              // 32-wide blocks of the rotation's contraction
  constexpr int IB = D / 16 / 4;          // 16-coordinate output blocks of one wavefront
  constexpr float kMat = 16.f;
  const unsigned char *cb = a.cb[which];
  const BlobOffsets bo = a.cbo[which];
  constexpr int half = (1 << BT) >> 1;
  const int tid = threadIdx.x;
  const int l64 = tid & 63, wave = tid >> 6;
  const int c = l64 & 15, g4 = l64 >> 4;
  const int ln = tid % LANES, vl = tid / LANES;

  half8_t ahi[IB][JB], alo[IB][JB];
  {
    const float *mat = a.rot[which];
#pragma unroll
    for (int ib = 0; ib < IB; ++ib)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const float *src = mat + (16 * (wave + 4 * ib) + c) * D + 32 * jb + 8 * g4;
        const float4 u0 = *(const float4 *)src;
        const float4 u1 = *(const float4 *)(src + 4);
        const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          _Float16 hh, ll;
          qr_split(v[p] * kMat, hh, ll);
          ahi[ib][jb][p] = hh;
          alo[ib][jb][p] = ll;
        }
      }
  }
  const uint32_t sword = ((const uint32_t *)(cb + bo.signs))[ln];
  PosThresholdsV PV{};
  if constexpr (BT <= 4) {
    PV = thresholds_in_vgprs(pos_thresholds((const_i32)(cb + bo.thresholds), half));
  } else {
    for (int i = tid; i < (1 << BT) - 1; i += 256) s_th[i] = ((const float *)(cb + bo.thresholds))[i];
    __syncthreads();
  }

  const int64_t tiles = (a.n_tok + VPB - 1) / VPB * a.H;
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int h = (int)(tile % a.H);
    const int64_t t0 = tile / a.H * VPB;
    // the tile's rows into LDS (rows past the last token are zero): every load in flight before the stores
    {
      constexpr int PER = VPB * (D / 8) / 256;
      float xv[PER][8];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int idx = tid + 256 * u;
        const int64_t t = t0 + idx / (D / 8);
        if (t < a.n_tok) {
          load8(a.in[which], t * a.stride[which] + (int64_t)h * D + 8 * (idx % (D / 8)), a.dtype, xv[u]);
        } else {
#pragma unroll
          for (int p = 0; p < 8; ++p) xv[u][p] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int idx = tid + 256 * u;
        float *dst = &s_x[(idx / (D / 8)) * XS + 8 * (idx % (D / 8))];
        *(float4 *)dst = float4{xv[u][0], xv[u][1], xv[u][2], xv[u][3]};
        *(float4 *)(dst + 4) = float4{xv[u][4], xv[u][5], xv[u][6], xv[u][7]};
      }
    }
    __syncthreads();
    // rotation, 16 rows at a time
#pragma unroll 1
    for (int rt = 0; rt < VPB / 16; ++rt) {
      const int v = 16 * rt + c;
      float xv[JB][8];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const float4 u0 = *(const float4 *)&s_x[v * XS + 32 * jb + 8 * g4];
        const float4 u1 = *(const float4 *)&s_x[v * XS + 32 * jb + 8 * g4 + 4];
        xv[jb][0] = u0.x; xv[jb][1] = u0.y; xv[jb][2] = u0.z; xv[jb][3] = u0.w;
        xv[jb][4] = u1.x; xv[jb][5] = u1.y; xv[jb][6] = u1.z; xv[jb][7] = u1.w;
      }
      float mx = 0.f;
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int p = 0; p < 8; ++p) mx = fmaxf(mx, fabsf(xv[jb][p]));
      mx = max_xor32(max_xor16(mx));
      int e = 0;
      (void)frexpf(mx, &e);
      const float sc = mx > 0.f ? ldexpf(1.f, 14 - e) : 1.f;
      const float back = 1.f / (kMat * sc);
      half8_t xhi[JB], xlo[JB];
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          _Float16 hh, ll;
          qr_split(xv[jb][p] * sc, hh, ll);
          xhi[jb][p] = hh;
          xlo[jb][p] = ll;
        }
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[ib][jb], xhi[jb], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[ib][jb], xlo[jb], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[ib][jb], xhi[jb], acc, 0, 0, 0);
        }
        *(float4 *)&s_y[v * XS + 16 * (wave + 4 * ib) + 4 * g4] =
            float4{acc[0] * back, acc[1] * back, acc[2] * back, acc[3] * back};
      }
    }
    __syncthreads();
    // the MSE steps on the rotated rows
    {
      const int64_t t = t0 + vl;
      const int64_t tc = t < a.n_tok ? t : 0;
      const int64_t slot = a.slots[tc];
      float x[32];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 u = *(const float4 *)&s_y[vl * XS + 32 * ln + 4 * k];
        x[4 * k] = u.x;
        x[4 * k + 1] = u.y;
        x[4 * k + 2] = u.z;
        x[4 * k + 3] = u.w;
      }
      apply_signs32(x, sword);
      quantize_vector32<D, BT>(a, which, x, slot, t < a.n_tok, h, ln, PV, s_th, CodeBuckets{nullptr, 0, 0});
    }
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(256) void quantize_qr_kernel(QuantArgs a) {
  constexpr int VPB = 256 / (D / 32);
  __shared__ __align__(16) float s_x[VPB * (D + 4)];
  __shared__ __align__(16) float s_y[VPB * (D + 4)];
  __shared__ float s_th[256];
  const int which = blockIdx.y;  // 0 = K, 1 = V
  switch (a.bits[which]) {       // uniform over the work-group
    case 1: quantize_qr_tiles<D, 1>(a, which, s_x, s_y, s_th); break;
    case 2: quantize_qr_tiles<D, 2>(a, which, s_x, s_y, s_th); break;
    case 3: quantize_qr_tiles<D, 3>(a, which, s_x, s_y, s_th); break;
    case 4: quantize_qr_tiles<D, 4>(a, which, s_x, s_y, s_th); break;
    default: quantize_qr_tiles<D, 8>(a, which, s_x, s_y, s_th); break;
  }
}

// Largest power of two sigma with max|x| * sigma < 256 (1 if x is all zero).
__device__ __forceinline__ float pow2_range(float maxabs) {
  if (!(maxabs > 0.f)) return 1.0f;
  int e;
  frexpf(maxabs, &e);
  return ldexpf(1.0f, 8 - e);
}

__device__ __forceinline__ void split16(float x, _Float16 &hi, _Float16 &lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

// Prod mode ("Closing - The Three-Step Summary", Step 3): the MSE steps at bits - 1, then the residual
// r = y - level[code] (the rotated unit-vector domain), gamma = ||r|| and the 1-bit sketch z_j = [(S r)_j >= 0].
// A work-group takes kProdChunk consecutive tokens of one head, VPB at a time: the lane groups run the MSE
// steps and leave r (scaled per vector by a power of two, which keeps every sign of S r) in LDS; then the
// four wavefronts compute Z^T[vectors][rows] = R[vectors][d] S^T[d][rows] on MFMA, each for its d / 4 rows of
// S, which it holds in registers as fp16 high + low parts for the whole run (16 S, exact); r enters as high
// + low parts too, and the three products hi*hi, hi*lo, lo*hi carry ~22 bits. The signs of the 16 x 16
// output blocks come out of wave ballots as 16-bit runs of the sketch bytes.
template <int D, int BT>
__global__ __launch_bounds__(256) void quantize_prod_kernel(QuantArgs a) {
  constexpr int LANES = D / 8;
  constexpr int VPB = 256 / LANES;  // vectors per round: 16 (d = 128) or 32 (d = 64)
  constexpr int MB = VPB / 16;      // 16-vector MFMA row blocks per round
  constexpr int NBW = D / 64;       // 16-row blocks of S per wavefront: 2 (d = 128) or 1 (d = 64)
  constexpr int KBLK = D / 32;
  constexpr int RS = D + 4;         // padded LDS row of residuals
  const int which = a.which_of_y[blockIdx.y];
  const unsigned char *cb = a.cb[which];
  const BlobOffsets bo = a.cbo[which];
  const int b = BT ? BT : a.bits[which];
  const int nl = 1 << b;
  const int half = nl >> 1;

  __shared__ float s_th[256];
  __shared__ float s_lv[256];
  __shared__ __align__(16) float s_r[VPB][RS];
  __shared__ long long s_zoff[VPB];  // byte offset of each vector's sketch in the pool, or -1

  const int tid = threadIdx.x;
  const int lane = tid % LANES, vl = tid / LANES;
  const int l64 = tid & 63, wave = tid >> 6, c = l64 & 15, g4 = l64 >> 4;
  const int h = blockIdx.x % a.H;
  const int64_t t0 = (int64_t)(blockIdx.x / a.H) * kProdChunk;
  const int64_t t_end = t0 + kProdChunk < a.n_tok ? t0 + kProdChunk : a.n_tok;

  const uint32_t sword = ((const uint32_t *)(cb + bo.signs))[(8 * lane) >> 5];
  PosThresholds P{};
  if constexpr (BT >= 1) P = pos_thresholds((const_i32)(cb + bo.thresholds), half);
  for (int i = tid; i < nl - 1; i += 256) s_th[i] = ((const float *)(cb + bo.thresholds))[i];
  for (int i = tid; i < nl; i += 256) s_lv[i] = half_bits_to_float(((const uint16_t *)(cb + bo.levels))[i]);

  // this wavefront's rows of 16 S: row 16 * (NBW * wave + nb) + c, contraction rows 8 * g4 .. of block kb =
  // coordinates 32 * kb + 8 * g4 + p
  half8_t shi[NBW][KBLK], slo[NBW][KBLK];
  {
    const float *S = (const float *)(cb + bo.proj);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int row = 16 * (NBW * wave + nb) + c;
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) {
        const float4 u0 = *(const float4 *)(S + (int64_t)row * D + 32 * kb + 8 * g4);
        const float4 u1 = *(const float4 *)(S + (int64_t)row * D + 32 * kb + 8 * g4 + 4);
        const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          _Float16 hi, lo;
          split16(16.0f * v[p], hi, lo);
          shi[nb][kb][p] = hi;
          slo[nb][kb][p] = lo;
        }
      }
    }
  }
  __syncthreads();

  const float inv_sqrt_d = D == 128 ? 0.088388347648318440f : 0.125f;
  for (int64_t tb = t0; tb < t_end; tb += VPB) {
    // ---- the MSE steps, the residual, gamma
    const int64_t t = tb + vl;
    const bool act = t < t_end;
    const int64_t tc = act ? t : 0;
    float x[8], y[8], n;
    int code[8], off;
    bool valid;
    int64_t base;
    load8(a.in[which], tc * a.stride[which] + (int64_t)h * D + 8 * lane, a.dtype, x);
    quantize_vector<D, BT>(a, which, x, a.slots[tc], act, h, lane, sword, P, s_th, y, code, valid, base, off, n);
    float r[8], g2 = 0.f, mx = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = (code[k] & half) ? code[k] : half - 1 - code[k];  // ascending index of the stored code
      r[k] = (y[k] - s_lv[idx]) * inv_sqrt_d;
      g2 = fmaf(r[k], r[k], g2);
      mx = fmaxf(mx, fabsf(r[k]));
    }
    g2 = group_sum<LANES>(g2);
#pragma unroll
    for (int m = 1; m < LANES; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, LANES));
    const float sc = pow2_range(mx);
#pragma unroll
    for (int k = 0; k < 8; ++k) s_r[vl][8 * lane + k] = r[k] * sc;
    unsigned char *pg = a.pages + base;
    if (valid && lane == 0)
      *(uint16_t *)(pg + a.gamma_off[which] + (int64_t)(h * TQ_PAGE_TOKENS + off) * 2) = float_to_half_bits(sqrtf(g2));
    if (lane == 0) s_zoff[vl] = valid ? base + a.qjl_off[which] + (int64_t)(h * TQ_PAGE_TOKENS + off) * (D / 8) : -1;
    __syncthreads();

    // ---- sketch signs: Z^T = R S^T on MFMA, 16 vectors x 16 rows per block
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      half8_t ahi[KBLK], alo[KBLK];
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) {
        const float4 w0 = *(const float4 *)&s_r[16 * mb + c][32 * kb + 8 * g4];
        const float4 w1 = *(const float4 *)&s_r[16 * mb + c][32 * kb + 8 * g4 + 4];
        const float v[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          _Float16 hi, lo;
          split16(v[p], hi, lo);
          ahi[kb][p] = hi;
          alo[kb][p] = lo;
        }
      }
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kb], shi[nb][kb], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[kb], slo[nb][kb], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[kb], shi[nb][kb], acc, 0, 0, 0);
        }
        // lane (c, g4) holds rows 4 * g4 + j (vectors) of column c (row of S): one ballot per j gives, for
        // vector 4 * g4 + j, its 16 sign bits of this block in bits 16 * g4 ..
        const unsigned long long m0 = __ballot(acc[0] >= 0.f), m1 = __ballot(acc[1] >= 0.f);
        const unsigned long long m2 = __ballot(acc[2] >= 0.f), m3 = __ballot(acc[3] >= 0.f);
        if (l64 < 16) {
          const int vv = l64;  // vector of the block this lane writes
          const unsigned long long m = (vv & 3) == 0 ? m0 : (vv & 3) == 1 ? m1 : (vv & 3) == 2 ? m2 : m3;
          const long long zo = s_zoff[16 * mb + vv];
          if (zo >= 0)
            *(uint16_t *)(a.pages + zo + 2 * (NBW * wave + nb)) = (uint16_t)(m >> (16 * (vv >> 2)));
        }
      }
    }
    __syncthreads();  // the residuals of this round are read before the next round writes them
  }
}

template <int D, int BT>
void launch_prod(dim3 grid, const QuantArgs &p, hipStream_t stream) {
  hipLaunchKernelGGL((quantize_prod_kernel<D, BT>), grid, dim3(256), 0, stream, p);
}

}  // namespace

namespace {

QuantArgs quant_args(const PageGeom &g, void *pages, int64_t num_pages, const void *k, const void *v, int dtype,
                     int64_t n_tok, int64_t k_stride, int64_t v_stride, const int64_t *slots, const void *k_cb,
                     const void *v_cb) {
  QuantArgs a;
  a.pages = (unsigned char *)pages;
  a.num_slots = num_pages * TQ_PAGE_TOKENS;
  a.page_bytes = g.page_bytes;
  a.in[0] = k;
  a.in[1] = v;
  a.stride[0] = k_stride;
  a.stride[1] = v_stride;
  a.slots = slots;
  a.n_tok = n_tok;
  a.cb[0] = (const unsigned char *)k_cb;
  a.cb[1] = (const unsigned char *)v_cb;
  a.cbo[0] = g.kcb;
  a.cbo[1] = g.vcb;
  a.codes_off[0] = g.k_codes;
  a.norms_off[0] = g.k_norms;
  a.qjl_off[0] = g.k_qjl;
  a.gamma_off[0] = g.k_gamma;
  a.codes_off[1] = g.v_codes;
  a.norms_off[1] = g.v_norms;
  a.qjl_off[1] = g.v_qjl;
  a.gamma_off[1] = g.v_gamma;
  a.bits[0] = g.k_mse_bits;
  a.bits[1] = g.v_mse_bits;
  a.mode[0] = g.k_mode;
  a.mode[1] = g.v_mode;
  a.H = g.num_kv_heads;
  a.dtype = dtype;
  a.rot[0] = a.rot[1] = nullptr;
  a.which_of_y[0] = 0;
  a.which_of_y[1] = 1;
  return a;
}

}  // namespace

int launch_quantize_qr(const PageGeom &g, void *pages, int64_t num_pages, const void *k, const void *v, int dtype,
                       int64_t n_tok, const int64_t *slots, const void *k_cb, const void *v_cb, const float *k_rot,
                       const float *v_rot, hipStream_t stream) {
  if (g.k_mode == TQ_PROD || g.v_mode == TQ_PROD) return TQ_ENOTSUP;
  const int64_t stride = (int64_t)g.num_kv_heads * g.head_dim;
  QuantArgs a = quant_args(g, pages, num_pages, k, v, dtype, n_tok, stride, stride, slots, k_cb, v_cb);
  a.rot[0] = k_rot;
  a.rot[1] = v_rot;
  const int vpb = 256 / (g.head_dim / 32);
  const int64_t tiles = (n_tok + vpb - 1) / vpb * g.num_kv_heads;
  if (tiles == 0) return TQ_OK;
  // a persistent loop over the tiles: the matrix is loaded once per work-group
  const dim3 grid((unsigned)std::min<int64_t>(tiles, 512), 2);
  if (g.head_dim == 128) hipLaunchKernelGGL(quantize_qr_kernel<128>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(quantize_qr_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

int launch_quantize(const PageGeom &g, void *pages, int64_t num_pages, const void *k, const void *v,
                    int dtype, int64_t n_tok, int64_t k_stride, int64_t v_stride,
                    const int64_t *slots, const void *k_cb, const void *v_cb, hipStream_t stream) {
  QuantArgs a = quant_args(g, pages, num_pages, k, v, dtype, n_tok, k_stride, v_stride, slots, k_cb, v_cb);
  // MSE tensors: work-groups of consecutive tokens of one head; prod tensors: long runs of one head
  int n_mse = 0, n_prod = 0, mse_of[2] = {0, 0}, prod_of[2] = {0, 0};
  for (int w = 0; w < 2; ++w) {
    if (a.mode[w] == TQ_PROD) prod_of[n_prod++] = w;
    else mse_of[n_mse++] = w;
  }
  // one launch for both MSE tensors when both codes are 8-bit or both narrower, else one launch each
  const bool both = n_mse == 2 && (a.bits[mse_of[0]] == 8) == (a.bits[mse_of[1]] == 8);
  for (int i = 0; i < n_mse; i += both ? 2 : 1) {
    QuantArgs m = a;
    m.which_of_y[0] = mse_of[i];
    m.which_of_y[1] = both ? mse_of[1] : mse_of[i];
    const int bits = a.bits[mse_of[i]];
    const int vpb = 256 / (g.head_dim / 32) * quant_passes(bits);  // vectors per work-group
    const int64_t blocks = (n_tok + vpb - 1) / vpb * g.num_kv_heads;
    if (blocks > 0x7FFFFFFF) return TQ_EINVAL;
    const dim3 grid((unsigned)blocks, both ? 2 : 1);
    const bool d128 = g.head_dim == 128;
    if (bits == 8) {
      if (d128) hipLaunchKernelGGL(quantize_wide_kernel<128>, grid, dim3(256), 0, stream, m);
      else hipLaunchKernelGGL(quantize_wide_kernel<64>, grid, dim3(256), 0, stream, m);
    } else {
      if (d128) hipLaunchKernelGGL(quantize_kernel<128>, grid, dim3(256), 0, stream, m);
      else hipLaunchKernelGGL(quantize_kernel<64>, grid, dim3(256), 0, stream, m);
    }
    if (hipGetLastError() != hipSuccess) return TQ_EHIP;
  }
  for (int i = 0; i < n_prod; ++i) {  // one launch per prod tensor, its code width fixed at compile time
    QuantArgs p = a;
    p.which_of_y[0] = prod_of[i];
    const int64_t blocks = (n_tok + kProdChunk - 1) / kProdChunk * g.num_kv_heads;
    if (blocks > 0x7FFFFFFF) return TQ_EINVAL;
    const dim3 grid((unsigned)blocks, 1);
    const bool d128 = g.head_dim == 128;
    switch (a.bits[prod_of[i]]) {
      case 1: d128 ? launch_prod<128, 1>(grid, p, stream) : launch_prod<64, 1>(grid, p, stream); break;
      case 2: d128 ? launch_prod<128, 2>(grid, p, stream) : launch_prod<64, 2>(grid, p, stream); break;
      case 3: d128 ? launch_prod<128, 3>(grid, p, stream) : launch_prod<64, 3>(grid, p, stream); break;
      default: d128 ? launch_prod<128, 0>(grid, p, stream) : launch_prod<64, 0>(grid, p, stream); break;
    }
    if (hipGetLastError() != hipSuccess) return TQ_EHIP;
  }
  return TQ_OK;
}

}  // namespace tq
