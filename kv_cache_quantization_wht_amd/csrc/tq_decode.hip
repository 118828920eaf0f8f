// Decode attention over the packed cache, one kernel launch ("Where This Fits in the Inference Stack",
// "TensorRT-LLM: Why Integration Is a Kernel Problem": dequantize in registers while the K/V tiles stream
// in; "Why the KV Cache Exists", "The KV Cache Solution": the new query attends over every cached token).
//
// Grid (splits, KV heads, batch); a work-group of WAVES wavefronts owns one run of pages of one
// (sequence, KV head) and all G = Hq/Hkv query heads that share it, so every K/V byte is read once.
//   1. Query rotation: q_rot = R q = H (s * q) / sqrt(d) for the G heads, in LDS (Walsh-Hadamard
//      butterflies); stored divided once more by sqrt(d) because the stored levels are in N(0,1) units.
//      For a sketched K also q_s = S q_rot * sqrt(pi/2) / m. A power-of-two factor per head brings each
//      into [128, 256) so that an fp16 hi + lo split carries ~22 bits.
//   2. Each wavefront walks page pairs (32 tokens), loading the next pair while it computes this one:
//        scores  S^T[16 tok, 16 col] = Khat[16, d] Q[d, 16] on MFMA 16x16x32 f16: the K operand holds fp16
//                levels looked up from the codes (v_perm byte tables for 4-bit codes), the Q operand the
//                hi and lo parts of the G rotated queries (two MFMAs per 32 coordinates);
//        softmax running max per head (base-2), sums kept per lane;
//        values  O[rows, d] += P'[rows, 32 tok] Vhat[32 tok, d] with P' = p * ||v|| as fp16 hi + lo (each
//                column's weights shifted by a power of two that keeps them in the fp16 range) and
//                Vhat the fp16 V levels (v_perm table for 2-bit codes).
//   3. The wavefronts merge in LDS (fixed-order tree). With one run per (sequence, KV head) the work-group
//      applies R_V^T once per output (butterflies in LDS) and writes fp32 out; with several runs it writes
//      its (max, sum, O) partial and a second, small kernel merges the runs and finishes the rows.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "tq_common.h"
#include "tq_internal.h"
#include "tq_lanes.h"
#include "tq_operands.h"
#include "tq_quant_common.h"

namespace tq {

// Arguments of one decode launch (split-K kernel and merge kernel).
struct DecodeArgs {
  const unsigned char *pages;
  int64_t num_pages;
  int num_pages32;  // min(num_pages, INT32_MAX): page ids are int32, so the check stays in scalar registers
  int64_t page_bytes;
  int64_t k_codes, k_norms, k_qjl, k_gamma, v_codes, v_norms;
  const void *q;
  int q_dtype;
  int B, Hq, Hkv, G;
  const int32_t *page_table;
  int max_pages;
  const int32_t *seq_lens;
  float scale_log2;
  const unsigned char *kcb, *vcb;
  BlobOffsets ko, vo;  // section offsets inside the K and V codebook blobs
  float *part_o, *part_ml;
  int n_splits, pps;
  float *out;
  int passes;  // kPassScan and/or kPassCombine
  // decode step (append): the new token of each sequence, quantized by the work-group that owns its page
  const void *k_new, *v_new;
  int kv_dtype;
};

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kHeadroom = 4.0f;  // log2 units between the running maximum and the weight reference
constexpr int kWaves = 8;
constexpr int kMlCap = 2048;   // split partials merged by one combine work-group
constexpr int kPidCap = 4096;  // page ids of one run held in LDS


// NBYTES bytes from p (aligned to ALIGN bytes) into dwords (little-endian).
template <int NBYTES, int ALIGN>
__device__ __forceinline__ void load_bytes(const unsigned char *p, uint32_t *w) {
  if constexpr (NBYTES % 16 == 0 && ALIGN >= 16) {
#pragma unroll
    for (int i = 0; i < NBYTES / 16; ++i) {
      uint4 t = ((const uint4 *)p)[i];
      w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
    }
  } else if constexpr (NBYTES % 8 == 0 && ALIGN >= 8) {
#pragma unroll
    for (int i = 0; i < NBYTES / 8; ++i) {
      uint2 t = ((const uint2 *)p)[i];
      w[2 * i] = t.x; w[2 * i + 1] = t.y;
    }
  } else if constexpr (NBYTES % 4 == 0 && ALIGN >= 4) {
#pragma unroll
    for (int i = 0; i < NBYTES / 4; ++i) w[i] = ((const uint32_t *)p)[i];
  } else {
    static_assert(NBYTES % 2 == 0, "even byte counts only");
#pragma unroll
    for (int i = 0; i < (NBYTES + 3) / 4; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < NBYTES / 2; ++i) w[i >> 1] |= (uint32_t)((const uint16_t *)p)[i] << (16 * (i & 1));
  }
}

// Bits [off, off + NB) of a little-endian dword stream.
template <int NB>
__device__ __forceinline__ uint32_t bits_at(const uint32_t *w, int off) {
  const int wi = off >> 5, sh = off & 31;
  uint64_t two = (uint64_t)w[wi] | ((sh + NB > 32) ? ((uint64_t)w[wi + 1] << 32) : 0ull);
  return (uint32_t)(two >> sh) & ((1u << NB) - 1u);
}

__device__ __forceinline__ half8_t from_halves(const uint16_t *hv) {
  return from_dwords(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16),
                     hv[4] | ((uint32_t)hv[5] << 16), hv[6] | ((uint32_t)hv[7] << 16));
}

// 3-bit sign-magnitude codes: the four magnitudes (levels of codes 4..7), low bytes in lo0, high bytes in hi0.
__device__ __forceinline__ Tab make_tab_k3(const uint16_t *lut) {
  Tab t{0, 0, 0, 0};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    t.lo0 |= ((uint32_t)lut[4 + m] & 0xFFu) << (8 * m);
    t.hi0 |= ((uint32_t)lut[4 + m] >> 8) << (8 * m);
  }
  return t;
}

// Eight sign bits at bits off..off+7 of w (bit p set: +level, clear: -level) -> fp16 operand of the eight
// values in order p. hitab: the high byte of -level in byte 0 and of +level in byte 1; lo4: the low byte of the
// level in all four bytes. Each nibble's bits are spread to bit 0 of bytes 0..3 by one 24-bit multiply (the copies
// of bit j land 7 apart; only its own lands on 8j), which then select the high bytes from hitab; a last permute
// pairs them with the low byte.
__device__ __forceinline__ half8_t signs_to_half8(uint32_t w, int off, uint32_t hitab, uint32_t lo4) {
  const uint32_t n0 = __builtin_amdgcn_ubfe(w, off, 4), n1 = __builtin_amdgcn_ubfe(w, off + 4, 4);
  const uint32_t h0 = perm(hitab, hitab, (n0 * 0x00204081u) & 0x01010101u);
  const uint32_t h1 = perm(hitab, hitab, (n1 * 0x00204081u) & 0x01010101u);
  return from_dwords(perm(h0, lo4, 0x05000400u), perm(h0, lo4, 0x07000600u), perm(h1, lo4, 0x05000400u),
                     perm(h1, lo4, 0x07000600u));
}

// The 24 bits of 3-bit codes of 32-coordinate block kb (8 coordinates) from the lane's run of codes.
template <int KW>
__device__ __forceinline__ uint32_t k3_field(const uint32_t (&w)[KW], int kb) {
  if (kb == 0) return w[0];
  if (kb == 1) return __builtin_amdgcn_alignbit(w[1], w[0], 24);
  if constexpr (KW > 2) {
    if (kb == 2) return __builtin_amdgcn_alignbit(w[2], w[1], 16);
    return w[2] >> 8;
  }
  return 0u;
}

// Eight 3-bit codes at bits 3e..3e+2 of g -> the pair (2k, 2k + 1) in bits 0-5 of byte k.
__device__ __forceinline__ uint32_t spread3(uint32_t g) {
  return (g & 0x3Fu) | ((g << 2) & 0x3F00u) | ((g << 4) & 0x3F0000u) | ((g << 6) & 0x3F000000u);
}

// 3-bit codes in bits 0-2 of each byte of x -> the four fp16 levels as two dwords (bytes 0, 1 and 2, 3).
__device__ __forceinline__ void lut3_bytes(uint32_t x, const Tab &T, uint32_t &d01, uint32_t &d23) {
  const uint32_t m = x & 0x03030303u;
  const uint32_t lb = perm(T.lo0, T.lo0, m);
  const uint32_t hb = or_signs(perm(T.hi0, T.hi0, m), x << 5);
  d01 = perm(hb, lb, 0x05010400u);
  d23 = perm(hb, lb, 0x07030602u);
}

// Eight 3-bit sign-magnitude codes (coordinate e at bits 3e..3e+2 of g) -> fp16 levels in MFMA order
// e = 0,2,4,6,1,3,5,7: the code pairs spread one per byte, then byte-table lookups of the magnitudes, sign bit set
// when the code's top bit is clear.
__device__ __forceinline__ half8_t lut_k3(uint32_t g, const Tab &T) {
  const uint32_t P = spread3(g);
  const uint32_t me = P & 0x03030303u, mo = (P >> 3) & 0x03030303u;
  const uint32_t le = perm(T.lo0, T.lo0, me);
  const uint32_t he = or_signs(perm(T.hi0, T.hi0, me), P << 5);
  const uint32_t lo = perm(T.lo0, T.lo0, mo);
  const uint32_t ho = or_signs(perm(T.hi0, T.hi0, mo), P << 2);
  return from_dwords(perm(he, le, 0x05010400u), perm(he, le, 0x07030602u), perm(ho, lo, 0x05010400u),
                     perm(ho, lo, 0x07030602u));
}

// --------------------------------------------------------------------------------------------------
// per page-pair register fragment
// --------------------------------------------------------------------------------------------------
template <int D, int KB, bool KPROD, int VB>
struct Frag {
  static constexpr int KCH = D / 4 * KB / 8;  // K code bytes per lane per token
  static constexpr int VCH = 4 * VB;          // V code bytes per lane per page
  static constexpr int KW = (KCH + 3) / 4;
  static constexpr int VW = VCH / 4;
  uint32_t kw[2][KW];
  uint32_t vw[2][VW];
  uint2 nk[2], nv[2];
  uint32_t zb[2];
  uint2 gm[2];
  bool ok[2];
};

// Byte offsets, inside one page, of everything one lane reads (fixed for the whole launch).
struct LaneOffsets {
  uint32_t k, nk, nv, v, z, gm;
};

template <int D, int KB, int VB>
__device__ __forceinline__ LaneOffsets lane_offsets(const DecodeArgs &a, int kvh, int c, int g4) {
  constexpr int KREC = D * KB / 8;
  constexpr int KCH = D / 4 * KB / 8;
  LaneOffsets o;
  o.k = (uint32_t)(a.k_codes + (int64_t)(kvh * TQ_PAGE_TOKENS + c) * KREC + g4 * KCH);
  o.nk = (uint32_t)(a.k_norms + (int64_t)(kvh * TQ_PAGE_TOKENS + 4 * g4) * 2);
  o.nv = (uint32_t)(a.v_norms + (int64_t)(kvh * TQ_PAGE_TOKENS + 4 * g4) * 2);
  const int piece = (D / 16) * c / 8;
  o.v = (uint32_t)(a.v_codes + ((int64_t)(kvh * (D / 8) + piece) * TQ_PAGE_TOKENS + 4 * g4) * VB);
  o.z = (uint32_t)(a.k_qjl + (int64_t)(kvh * TQ_PAGE_TOKENS + c) * (D / 8) + g4 * (D / 32));
  o.gm = (uint32_t)(a.k_gamma + (int64_t)(kvh * TQ_PAGE_TOKENS + 4 * g4) * 2);
  return o;
}

// NBYTES bytes at byte offset off of a buffer resource, into dwords (little-endian).
template <int NBYTES>
__device__ __forceinline__ void buf_bytes(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *w) {
  if constexpr (NBYTES % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NBYTES / 16; ++i) {
      const uint4 t = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0));
      w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
    }
  } else if constexpr (NBYTES % 8 == 0) {
#pragma unroll
    for (int i = 0; i < NBYTES / 8; ++i) {
      const uint2 t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off + 8 * i, 0, 0));
      w[2 * i] = t.x; w[2 * i + 1] = t.y;
    }
  } else if constexpr (NBYTES % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NBYTES / 4; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, 0);
  } else {
    static_assert(NBYTES % 2 == 0, "even byte counts only");
#pragma unroll
    for (int i = 0; i < (NBYTES + 3) / 4; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < NBYTES / 2; ++i)
      w[i >> 1] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * i, 0, 0) << (16 * (i & 1));
  }
}

// Both pages of one pair (page ids pg0, pg1; an id outside [0, num_pages) - a pair past the end of the run
// included - is marked invalid and gets a zero-size buffer, so its loads return zeros without a memory
// request). The page id is the same for the whole wavefront: each page is a buffer resource in scalar
// registers and every lane adds its fixed 32-bit offset.
template <int D, int KB, bool KPROD, int VB>
__device__ __forceinline__ void load_pages(const DecodeArgs &a, const LaneOffsets &lo, int pg0, int pg1,
                                           Frag<D, KB, KPROD, VB> &f) {
  using F = Frag<D, KB, KPROD, VB>;
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int pg = __builtin_amdgcn_readfirstlane(q2 ? pg1 : pg0);
    const bool ok = pg >= 0 && pg < a.num_pages32;
    f.ok[q2] = ok;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.pages + (int64_t)(ok ? pg : 0) * a.page_bytes), (short)0, ok ? (int)a.page_bytes : 0, 0x00020000);
    buf_bytes<F::KCH>(r, lo.k, f.kw[q2]);
    uint32_t t[2];
    buf_bytes<8>(r, lo.nk, t);
    f.nk[q2] = uint2{t[0], t[1]};
    buf_bytes<8>(r, lo.nv, t);
    f.nv[q2] = uint2{t[0], t[1]};
    buf_bytes<F::VCH>(r, lo.v, f.vw[q2]);
    if constexpr (KPROD) {
      uint32_t z[1];
      buf_bytes<D / 32>(r, lo.z, z);
      f.zb[q2] = z[0];
      buf_bytes<8>(r, lo.gm, t);
      f.gm[q2] = uint2{t[0], t[1]};
    }
  }
}

// Both pages of one pair given as checked page ids (pg.x, pg.y; -1 for an invalid page, whose loads get a zero-size
// buffer as in load_pages). A page is smaller than 2^31 bytes (its buffer size is 32-bit), so the byte offset is one
// 32 x 32 -> 64-bit unsigned product.
template <int D, int KB, bool KPROD, int VB>
__device__ __forceinline__ void load_pages_id(const DecodeArgs &a, const LaneOffsets &lo, int2 pg,
                                              Frag<D, KB, KPROD, VB> &f) {
  using F = Frag<D, KB, KPROD, VB>;
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int id = __builtin_amdgcn_readfirstlane(q2 ? pg.y : pg.x);
    const bool ok = id >= 0;
    f.ok[q2] = ok;
    const uint64_t off = (uint64_t)(uint32_t)id * (uint32_t)a.page_bytes;  // unused (size 0) for an invalid page
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)(a.pages + off), (short)0,
                                                                       ok ? (int)a.page_bytes : 0, 0x00020000);
    buf_bytes<F::KCH>(r, lo.k, f.kw[q2]);
    uint32_t t[2];
    buf_bytes<8>(r, lo.nk, t);
    f.nk[q2] = uint2{t[0], t[1]};
    buf_bytes<8>(r, lo.nv, t);
    f.nv[q2] = uint2{t[0], t[1]};
    buf_bytes<F::VCH>(r, lo.v, f.vw[q2]);
    if constexpr (KPROD) {
      uint32_t z[1];
      buf_bytes<D / 32>(r, lo.z, z);
      f.zb[q2] = z[0];
      buf_bytes<8>(r, lo.gm, t);
      f.gm[q2] = uint2{t[0], t[1]};
    }
  }
}

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ half4_t as_half4(uint2 w) { return __builtin_bit_cast(half4_t, w); }

__device__ __forceinline__ void unpack4(uint2 w, float *x) {
  x[0] = half_bits_to_float(w.x & 0xFFFF);
  x[1] = half_bits_to_float(w.x >> 16);
  x[2] = half_bits_to_float(w.y & 0xFFFF);
  x[3] = half_bits_to_float(w.y >> 16);
}

// In-place Walsh-Hadamard transform of `rows` rows of D floats in LDS (row stride D), all threads.
template <int D, int NT>
__device__ __forceinline__ void lds_wht(float (*buf)[D], int rows, int tid) {
  for (int hs = 1; hs < D; hs <<= 1) {
    for (int p = tid; p < rows * (D / 2); p += NT) {
      const int r = p / (D / 2), j = p % (D / 2);
      const int i1 = (j / hs) * 2 * hs + (j % hs), i2 = i1 + hs;
      const float u = buf[r][i1], w = buf[r][i2];
      buf[r][i1] = u + w;
      buf[r][i2] = u - w;
    }
    __syncthreads();
  }
}

// One appended vector (K or V of the new token of one head), in two steps so that its reads join the
// prologue's first round of reads: load (input row, sign word, positive thresholds), then quantize: the
// d/8 lanes of its lane group quantize it exactly as the quantize kernel does, write its codes and fp16
// norm into the page slot, and leave the fp16 levels of its codes (as fp32, one per coordinate) and the
// rounded norm in LDS for the scoring of the new token.
struct AppendIn {
  float x[8];
  uint32_t sword;
  PosThresholds P;
};

// K lanes and V lanes run the same instruction stream: the code width is a per-lane value, the search
// counts over thresholds padded with +inf, and only the final byte stores differ.
template <int D>
__device__ __forceinline__ void append_load(const DecodeArgs &a, bool is_v, int nbits, int kvh, int lq,
                                            AppendIn &in) {
  const void *src = is_v ? a.v_new : a.k_new;
  const unsigned char *cb = is_v ? a.vcb : a.kcb;
  const BlobOffsets bo = is_v ? a.vo : a.ko;
  load8(src, ((int64_t)blockIdx.z * a.Hkv + kvh) * D + 8 * lq, a.kv_dtype, in.x);
  in.sword = ((const uint32_t *)(cb + bo.signs))[(8 * lq) >> 5];
  in.P = pos_thresholds((const int *)(cb + bo.thresholds), (1 << nbits) >> 1);
}

template <int D, int KB, int VB>
__device__ __forceinline__ void append_quantize(const DecodeArgs &a, bool is_v, int kvh, int lq, AppendIn &in,
                                                int64_t page_off, int slot, const uint16_t *lut, float *s_lev,
                                                float *s_norm) {
  const int nbits = is_v ? VB : KB;
  const int half = (1 << nbits) >> 1;
  float *x = in.x;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss = fmaf(x[k], x[k], ss);
  ss = group_sum<D / 8>(ss);
  float n, inv;
  norm_and_inverse(ss, n, inv);
  const uint32_t sbits = (in.sword >> ((8 * lq) & 31)) & 0xFFu;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if ((sbits >> k) & 1u) x[k] = -x[k];
#pragma unroll
  for (int hs = 1; hs < 8; hs <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (!(k & hs)) {
        const float u = x[k], w = x[k + hs];
        x[k] = u + w;
        x[k + hs] = u - w;
      }
    }
  }
  wht_lanes<1>(x, lq);
  wht_lanes<2>(x, lq);
  wht_lanes<4>(x, lq);
  if constexpr (D == 128) wht_lanes<8>(x, lq);
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool neg = x[k] < 0.f;
    const int z = __float_as_int(fabsf(x[k]) * inv);
    const int mag = magnitude_count<4>(z, in.P);  // thresholds past the code's own are +inf
    const int code = neg ? mag : (half | mag);
    packed |= (uint32_t)code << (nbits * k);
    s_lev[8 * lq + k] = half_bits_to_float(lut[code]);  // the stored fp16 level of the code
  }
  const uint16_t n16 = float_to_half_bits(n);
  if (lq == 0) *s_norm = half_bits_to_float(n16);
  unsigned char *pg = (unsigned char *)a.pages + page_off;
  unsigned char *dst = is_v ? pg + a.v_codes + ((int64_t)(kvh * (D / 8) + lq) * TQ_PAGE_TOKENS + slot) * VB
                            : pg + a.k_codes + (int64_t)(kvh * TQ_PAGE_TOKENS + slot) * (D * KB / 8) + lq * KB;
  switch (nbits) {  // a lane's 8 codes are nbits whole bytes
    case 1: *dst = (unsigned char)packed; break;
    case 2: *(uint16_t *)dst = (uint16_t)packed; break;
    case 4: *(uint32_t *)dst = packed; break;
    default:
      for (int i = 0; i < nbits; ++i) dst[i] = (unsigned char)(packed >> (8 * i));
  }
  if (lq == 0) *(uint16_t *)(pg + (is_v ? a.v_norms : a.k_norms) + (int64_t)(kvh * TQ_PAGE_TOKENS + slot) * 2) = n16;
}

// PK (at most 8 query heads per KV head): MFMA column c carries query head c & 7, the high fp16 part of its
// operand when c < 8 and the low part when c >= 8, so one MFMA does the work of the hi and lo pair. The
// two partial scores meet by one row rotation; the two partial value sums are added once, before the merge.
// Otherwise column c is query head c and every product is an hi + lo pair of MFMAs.
template <int D, int KB, bool KPROD, int VB, bool APPEND, bool PK>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(DecodeArgs a) {
  constexpr int NT = 64 * kWaves;
  constexpr int KBLK = D / 32;  // 32-coordinate blocks of the score contraction
  constexpr int NB = D / 16;    // 16-coordinate blocks of the value contraction
  constexpr int QF = 16 * D;    // floats in one [16][D] block
  constexpr bool LUT = KB == 4 && VB == 2 && D == 128 && !KPROD;
  constexpr bool LUT1 = KB == 1 && KPROD && D == 128;  // 1-bit K with its sketch: one table for both operands
  constexpr bool LUT3 = KB == 3 && VB == 3 && D == 128 && !KPROD;  // 3-bit K and V: a table of code pairs
  using F = Frag<D, KB, KPROD, VB>;

  // Every argument the prologue needs, fetched from the argument segment in one round trip (left to
  // itself the compiler fetches them in several dependent rounds, each a full memory latency).
  asm volatile("" ::"s"(a.pages), "s"(a.num_pages32), "s"(a.page_bytes), "s"(a.k_codes), "s"(a.k_norms),
               "s"(a.v_codes), "s"(a.v_norms), "s"(a.q), "s"(a.q_dtype), "s"(a.Hq), "s"(a.G), "s"(a.page_table),
               "s"(a.max_pages), "s"(a.seq_lens), "s"(a.kcb), "s"(a.vcb), "s"(a.ko.signs), "s"(a.ko.levels),
               "s"(a.vo.levels), "s"(a.pps), "s"(a.scale_log2), "s"(a.n_splits));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15;   // MFMA row/column inside a 16-block
  const int g4 = lane >> 4;  // 8-deep slice of the contraction held by this lane
  const int hc = PK ? (c & 7) : c;                // query head (inside the KV head's group) of column c
  const bool lo_part = PK && c >= 8;              // PK: column c carries the low fp16 parts
  float neg_one = -1.0f;  // opaque to the compiler, so that x - (float)h stays one mixed-precision FMA
  asm volatile("" : "+s"(neg_one));
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.G;
  const int head0 = kvh * G;

  // LDS arena reused by phase: queries (prologue), then the wave-merge tree. Query rows are padded to
  // QS floats so that the operand reads of different heads fall in different banks.
  constexpr int QS = D + 4;
  static_assert(2 * 16 * QS <= 4 * QF, "query rows fit in the arena");
  __shared__ __align__(16) float arena[4 * QF];
  __shared__ float s_sig[16][2];
  __shared__ uint16_t s_lutk[1 << KB];
  __shared__ uint16_t s_lutv[1 << VB];
  __shared__ float s_m[kWaves][16], s_l[kWaves][16];
  __shared__ float s_rowm[16], s_rowl[16];
  __shared__ __align__(16) float s_newlev[APPEND ? 2 : 1][APPEND ? D : 4];  // appended token: K and V levels
  // LUT (4-bit K, 2-bit V, head_dim 128): codes become fp16 levels through LDS lookups. Row x (256 bytes) of the
  // table holds, for the code byte x, the K entry (levels of its two 4-bit codes, one dword) 32 times in bytes
  // 0..127 and the V entry (levels of its four 2-bit codes, two dwords) 16 times in bytes 128..255: lane l reads
  // copy l % 32 (K) or l % 16 (V), so the 32 lanes of a 4-byte read or the 16 lanes of an 8-byte read fall in
  // distinct banks. The row address is the code byte itself shifted up by 8 bits, so one v_perm of the code word
  // and the lane's copy offset forms each address.
  // LUT1 (1-bit K with the QJL sketch, head_dim 128): row x holds the eight fp16 values +1 / -1 of the bits of x
  // (bit i: value i; a set bit: +1), 16 bytes, 16 times: lane l reads copy l % 16, so the 16 lanes of a 16-byte read
  // fall in distinct banks. A byte of sketch bits looks up its eight sketch values, and a byte of 1-bit K codes the
  // signs of its eight levels: the Lloyd-Max levels of one bit are -L and +L, and L multiplies the query operand.
  // LUT3 (3-bit K and V, head_dim 128): row x (256 bytes, 64 rows) holds, for the code pair x (first code in bits
  // 0..2, second in 3..5), the K entry (their two fp16 levels, one dword) 32 times in bytes 0..127 and the V entry
  // 32 times in bytes 128..255; lane l reads copy l % 32.
  __shared__ __align__(16) uint32_t s_lut[(LUT || LUT1) ? 256 * 64 : (LUT3 ? 64 * 64 : 4)];
  auto lut_read = [&](uint32_t byte_addr) { return *(const uint32_t *)((const unsigned char *)s_lut + byte_addr); };
  auto lut_read4 = [&](uint32_t byte_addr) { return *(const uint4 *)((const unsigned char *)s_lut + byte_addr); };
  auto lut_read2 = [&](uint32_t byte_addr) { return *(const uint2 *)((const unsigned char *)s_lut + byte_addr); };
  __shared__ float s_newnorm[2];
  float(*s_q)[QS] = (float(*)[QS])arena;              // rotated queries / d
  float(*s_qs)[QS] = (float(*)[QS])(arena + 16 * QS);  // sketch-domain queries

  // the run's pages in the table (p_begin .. p_cap) do not depend on the sequence length, so the page-id
  // reads are issued alongside the length read instead of after it
  // runs of pps pages; the last run of a sequence also takes the remainder (fewer than pps pages)
  const bool last_run = split == a.n_splits - 1;
  const int p_begin = split * a.pps;
  const int p_cap = last_run ? a.max_pages : min(p_begin + a.pps, a.max_pages);
  typedef const __attribute__((address_space(4))) int32_t *const_i32;  // read through the scalar cache
  int seq_len = ((const_i32)a.seq_lens)[b];
  seq_len = seq_len < 0 ? 0 : (seq_len > a.max_pages * TQ_PAGE_TOKENS ? a.max_pages * TQ_PAGE_TOKENS : seq_len);
  const int npages = (seq_len + TQ_PAGE_TOKENS - 1) / TQ_PAGE_TOKENS;
  const int p_end = last_run ? npages : min(p_begin + a.pps, npages);
  const int npairs = p_end > p_begin ? (p_end - p_begin + 1) / 2 : 0;
  // decode step: position seq_len - 1 is the appended token; the page loop reads positions before it
  // and the work-group owning its page scores it from the codes it quantizes itself
  const int seq_mem = APPEND ? max(seq_len - 1, 0) : seq_len;
  const bool own_new = APPEND && seq_len >= 1 && (seq_len - 1) / TQ_PAGE_TOKENS >= p_begin &&
                       (seq_len - 1) / TQ_PAGE_TOKENS < p_end;

  // ---- 0. the small global reads of the prologue, into registers first (memory returns in issue order,
  //         so these must not queue behind the page data): page ids of the run, this wavefront's query
  //         rows, the rotation signs of the query's coordinates, the level tables
  // page ids of this wavefront's first pairs through the scalar cache: the head of the longest chain
  // (page id -> page data)
  constexpr int R = (KB >= 8 || VB >= 8) ? 2 : 3;  // fragments in the ring (wide codes leave room for fewer)
  // The run's page ids (an invalid id replaced by -1), followed by -1 entries for the ring's loads past the run,
  // so a load takes its two ids with one LDS read and no bounds test.
  constexpr int PID_PAD = 4 * (R - 1) * kWaves + 4;
  __shared__ __align__(8) int s_pid[kPidCap + PID_PAD];
  int first_ids[R - 1][2];
  {
    const const_i32 ptab = (const_i32)(a.page_table) + (int64_t)b * a.max_pages;
#pragma unroll
    for (int r = 0; r + 1 < R; ++r) {
      const int pp = p_begin + 2 * (wave + r * kWaves);
      first_ids[r][0] = pp < p_cap ? ptab[pp] : -1;
      first_ids[r][1] = pp + 1 < p_cap ? ptab[pp + 1] : -1;
    }
  }
  // decode step: the appending wavefront's reads of the new K (lanes 0..) and V (lanes 32..)
  AppendIn app;
  const bool app_lane = APPEND && wave == kWaves - 1 && (lane & 31) < D / 8;
  if constexpr (APPEND) {
    if (app_lane) append_load<D>(a, lane >= 32, lane >= 32 ? VB : KB, kvh, lane & 31, app);
  }
  // No loaded value is used (converted, compared, selected) before the page loads of step 1 are issued:
  // addresses are clamped in bounds instead, so no wait lands here.
  constexpr int PID_PER_THREAD = kPidCap / NT;
  int pgv[PID_PER_THREAD];
  {
    const int32_t *row = a.page_table + (int64_t)b * a.max_pages;
#pragma unroll
    for (int u = 0; u < PID_PER_THREAD; ++u)
      if (tid + u * NT < p_cap - p_begin) pgv[u] = row[p_begin + tid + u * NT];  // read below under the same bound
  }
  uint32_t qraw[2][2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int r = wave + rr * kWaves;
    const int64_t base = ((int64_t)b * a.Hq + head0 + (r < G ? r : 0)) * D + lane;
#pragma unroll
    for (int h = 0; h < (D == 128 ? 2 : 1); ++h) {
      if (a.q_dtype == TQ_F32) qraw[rr][h] = ((const uint32_t *)a.q)[base + 64 * h];
      else qraw[rr][h] = ((const uint16_t *)a.q)[base + 64 * h];
    }
    if (D != 128) qraw[rr][1] = 0;
  }
  const uint32_t *ksw = (const uint32_t *)(a.kcb + a.ko.signs);
  const uint32_t sgn0 = ksw[lane >> 5];
  const uint32_t sgn1 = D == 128 ? ksw[(lane + 64) >> 5] : 0u;
  // code-indexed level tables: code c -> ascending level c (upper half) or half - 1 - c (lower half)
  uint16_t lk, lv;
  {
    const int nk = 1 << KB, nv = 1 << VB;
    const int ck = tid < nk ? tid : 0, cv = tid < nv ? tid : 0;
    lk = ((const uint16_t *)(a.kcb + a.ko.levels))[ck >= nk / 2 ? ck : nk / 2 - 1 - ck];
    lv = ((const uint16_t *)(a.vcb + a.vo.levels))[cv >= nv / 2 ? cv : nv / 2 - 1 - cv];
  }

  // ---- 1. this wavefront's first page pairs in flight: their page ids come through the scalar cache
  //         (no LDS, no barrier). Every fragment load is issued unconditionally (a pair past the run
  //         reads page 0 and is never used): with the same loads on every path the compiler's wait
  //         counts keep R - 1 pairs in flight.
  const LaneOffsets lo = lane_offsets<D, KB, VB>(a, kvh, c, g4);
  F f[R];
#pragma unroll
  for (int r = 0; r + 1 < R; ++r) {
    const int pp = p_begin + 2 * (wave + r * kWaves);
    load_pages<D, KB, KPROD, VB>(a, lo, pp < p_end ? first_ids[r][0] : -1, pp + 1 < p_end ? first_ids[r][1] : -1, f[r]);
  }

  // the page ids and level tables into LDS (waits only for the small reads above)
  int pids_ok = 1;
#pragma unroll
  for (int u = 0; u < PID_PER_THREAD; ++u) {
    const int j = tid + u * NT;
    if (j < p_end - p_begin) {
      const bool ok = pgv[u] >= 0 && pgv[u] < a.num_pages32;
      s_pid[j] = ok ? pgv[u] : -1;
      pids_ok &= ok ? 1 : 0;
    }
  }
  if (tid < PID_PAD) s_pid[max(p_end - p_begin, 0) + tid] = -1;
  if (tid < (1 << KB)) s_lutk[tid] = lk;
  if (tid < (1 << VB)) s_lutv[tid] = lv;

  // ---- 1b. decode step: is the new token's page this run's, and a valid page?
  bool new_ok = false;
  int new_pg = 0;
  if constexpr (APPEND) {
    if (own_new) {
      new_pg = ((const_i32)a.page_table)[(int64_t)b * a.max_pages + (seq_len - 1) / TQ_PAGE_TOKENS];
      new_ok = new_pg >= 0 && new_pg < a.num_pages32;
    }
  }

  // ---- 2. query rotation, one row per wavefront: H (s * q) with cross-lane butterflies (no barrier
  //         needed before: the row and the signs are this wavefront's own loads)
  {
    const bool neg0 = (sgn0 >> (lane & 31)) & 1u;
    const bool neg1 = (sgn1 >> (lane & 31)) & 1u;
    auto widen = [&](uint32_t u) {
      return a.q_dtype == TQ_F32 ? __uint_as_float(u)
                                 : (a.q_dtype == TQ_BF16 ? bf16_bits_to_float((uint16_t)u) : half_bits_to_float((uint16_t)u));
    };
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = wave + rr * kWaves;
      if (r >= G) continue;
      const float q0 = widen(qraw[rr][0]), q1 = D == 128 ? widen(qraw[rr][1]) : 0.f;
      float x0 = neg0 ? -q0 : q0;
      float x1 = neg1 ? -q1 : q1;
      x0 = wht_stage<1>(x0, lane);
      x1 = wht_stage<1>(x1, lane);
      x0 = wht_stage<2>(x0, lane);
      x1 = wht_stage<2>(x1, lane);
      x0 = wht_stage<4>(x0, lane);
      x1 = wht_stage<4>(x1, lane);
      x0 = wht_stage<8>(x0, lane);
      x1 = wht_stage<8>(x1, lane);
      x0 = wht_stage<16>(x0, lane);
      x1 = wht_stage<16>(x1, lane);
      x0 = wht_stage<32>(x0, lane);
      x1 = wht_stage<32>(x1, lane);
      if (D == 128) {
        const float u = x0;
        x0 = u + x1;
        x1 = u - x1;
      }
      x0 *= (1.0f / D);
      x1 *= (1.0f / D);
      const float mx = wave_max(fmaxf(fabsf(x0), D == 128 ? fabsf(x1) : 0.f), lane);
      s_q[r][lane] = x0;
      if (D == 128) s_q[r][lane + 64] = x1;
      if (lane == 0) s_sig[r][0] = range_factor(mx);
    }
  }
  // a run of whole, valid page pairs needs no per-token masking; one barrier publishes the page ids,
  // level tables and rotated queries
  // pairs [0, n_full) of the run hold only cached tokens of valid pages: they need no masking
  const bool all_ok = __syncthreads_and(pids_ok);
  if constexpr (LUT) {
    // thread pair (2x, 2x + 1) writes row x: the even thread the K copies, the odd one the V copies, 16 bytes at a
    // time starting at a chunk that rotates with the lane, so the 8 lanes of a 16-byte store cycle hit all banks
    const int x = tid >> 1;
    uint4 val;
    if ((tid & 1) == 0) {
      const uint32_t e = (uint32_t)s_lutk[x & 15] | ((uint32_t)s_lutk[x >> 4] << 16);
      val = uint4{e, e, e, e};
    } else {
      const uint32_t e0 = (uint32_t)s_lutv[x & 3] | ((uint32_t)s_lutv[(x >> 2) & 3] << 16);
      const uint32_t e1 = (uint32_t)s_lutv[(x >> 4) & 3] | ((uint32_t)s_lutv[x >> 6] << 16);
      val = uint4{e0, e1, e0, e1};
    }
    uint4 *row = (uint4 *)&s_lut[x * 64 + (tid & 1) * 32];
#pragma unroll
    for (int i = 0; i < 8; ++i) row[(i + lane) & 7] = val;
  }
  if constexpr (LUT3) {
    // eight threads per row x: threads 0..3 the K copies, 4..7 the V copies, two 16-byte chunks each
    const int x = tid >> 3, q = tid & 7;
    const uint16_t *lv = q < 4 ? s_lutk : s_lutv;
    const uint32_t e = (uint32_t)lv[x & 7] | ((uint32_t)lv[x >> 3] << 16);
    uint4 *row = (uint4 *)&s_lut[x * 64];
    row[2 * q] = uint4{e, e, e, e};
    row[2 * q + 1] = uint4{e, e, e, e};
  }
  if constexpr (LUT1) {
    // thread pair (2x, 2x + 1) writes row x, eight 16-byte copies each, starting at a copy that rotates with the lane
    const int x = tid >> 1;
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      d[i] = (((x >> (2 * i)) & 1) ? 0x3C00u : 0xBC00u) | ((((x >> (2 * i + 1)) & 1) ? 0x3C00u : 0xBC00u) << 16);
    const uint4 val = {d[0], d[1], d[2], d[3]};
    uint4 *row = (uint4 *)&s_lut[x * 64 + (tid & 1) * 32];
#pragma unroll
    for (int i = 0; i < 8; ++i) row[(i + lane) & 7] = val;
  }
  const int full_end = min(p_end, seq_mem / TQ_PAGE_TOKENS);
  const int n_full = (all_ok && full_end > p_begin) ? (full_end - p_begin) / 2 : 0;
  if constexpr (KPROD) {
    // q_s = S (R q) sqrt(pi/2) / m with R q = (d * s_q) / sqrt(d)
    const float *S = (const float *)(a.kcb + a.ko.proj);
    const float cq = 1.2533141373155003f / (float)a.ko.qjl_rows * (float)D * (D == 128 ? 0.088388347648318440f : 0.125f);
    for (int idx = tid; idx < G * D; idx += NT) {
      const int r = idx / D, j = idx % D;
      float acc = 0.f;
      for (int k = 0; k < D; ++k) acc = fmaf(S[(int64_t)j * D + k], s_q[r][k], acc);
      s_qs[r][j] = acc * cq;
    }
    __syncthreads();
    for (int r = wave; r < G; r += kWaves) {
      float mx = 0.f;
      for (int k = lane; k < D; k += 64) mx = fmaxf(mx, fabsf(s_qs[r][k]));
      mx = wave_max(mx, lane);
      if (lane == 0) s_sig[r][1] = range_factor(mx);
    }
    __syncthreads();
  }

  // query operands: column c = query head head0 + c, contraction rows 8*g4.. of each 32-block,
  // i.e. coordinates cbase + 8*kb + k_order(p)
  const int cbase = (D / 4) * g4;
  half8_t qhi[KBLK], qlo[PK ? 1 : KBLK];  // PK: qhi holds this column's part (high or low)
  half8_t shi[KPROD ? KBLK : 1], slo[(KPROD && !PK) ? KBLK : 1];
  float colscale, skratio;
  {
    const bool real = hc < G;
    const int r = real ? hc : 0;
    const float sig = s_sig[r][0], sig2 = KPROD ? s_sig[r][1] : 1.f;
    colscale = real ? a.scale_log2 / sig : 0.f;
    skratio = sig / sig2;
    // LUT1: the K operand holds the signs of the levels (+1 / -1), the query operand the level L = level of code 1
    const float kq = LUT1 ? half_bits_to_float(s_lutk[1]) * sig : sig;
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb) {
      // the lane's 8 consecutive coordinates as two 16-byte LDS reads
      const float4 u0 = *(const float4 *)&s_q[r][cbase + 8 * kb];
      const float4 u1 = *(const float4 *)&s_q[r][cbase + 8 * kb + 4];
      const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float x = real ? v[(LUT || LUT3) ? p : k_order<KB>(p)] * kq : 0.f;
        _Float16 h, l;
        split_hi_lo(x, h, l);
        if constexpr (PK) {
          qhi[kb][p] = lo_part ? l : h;
        } else {
          qhi[kb][p] = h;
          qlo[kb][p] = l;
        }
      }
      if constexpr (KPROD) {
        const float4 w0 = *(const float4 *)&s_qs[r][cbase + 8 * kb];
        const float4 w1 = *(const float4 *)&s_qs[r][cbase + 8 * kb + 4];
        const float z[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const float y = real ? z[p] * sig2 : 0.f;
          _Float16 h, l;
          split_hi_lo(y, h, l);
          if constexpr (PK) {
            shi[kb][p] = lo_part ? l : h;
          } else {
            shi[kb][p] = h;
            slo[kb][p] = l;
          }
        }
      }
    }
  }
  Tab tk{0, 0, 0, 0}, tv{0, 0, 0, 0};
  // LUT: byte 0 of these words is the lane's copy offset inside a table row (K: bytes 0..127, V: 128..255)
  const uint32_t lut_kb = (uint32_t)(lane & 31) * 4u, lut_vb = 128u + (uint32_t)(lane & 15) * 8u;
  const uint32_t lut1_off = (uint32_t)(lane & 15) * 16u;  // LUT1: the lane's copy inside a row
  const uint32_t lut3_vb = 128u + (uint32_t)(lane & 31) * 4u;  // LUT3: the lane's V copy (K: lut_kb)
  // LUT3: the table address of code pair k (bits 6k..6k+5) of a 24-bit group of eight codes
  auto lut3_addr = [&](uint32_t g, int k, uint32_t off) { return (__builtin_amdgcn_ubfe(g, 6 * k, 6) << 8) | off; };
  if constexpr (LUT || LUT1 || LUT3) __syncthreads();  // the table is complete
  if constexpr (KB == 4 && !LUT) tk = make_tab_k4(s_lutk);
  if constexpr (KB == 3 && !LUT3) tk = make_tab_k3(s_lutk);
  if constexpr (VB == 2 && !LUT) tv = make_tab_v2(s_lutv);
  if constexpr (VB == 3 && D == 128 && !LUT3) tv = make_tab_k3(s_lutv);
  // 1-bit levels: the high byte of the negative and the positive level, and the low byte in all four bytes
  uint32_t lev1_hitab = 0, lev1_lo4 = 0;
  if constexpr (KB == 1) {
    lev1_hitab = ((uint32_t)s_lutk[0] >> 8) | ((uint32_t)s_lutk[1] & 0xFF00u);
    lev1_lo4 = ((uint32_t)s_lutk[0] & 0xFFu) * 0x01010101u;
  }

  // ---- 3. stream the page pairs
  float m_run = -INFINITY;
  float l_part = 0.f;
  float ev = 0.f;    // the column's weight shift (power of two), see weight_shift
  float wmax = 0.f;  // the largest value weight the lane has seen, in the current units
  floatx4_t O[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) O[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (APPEND) {
    // The last wavefront quantizes the appended K (lanes 0..) and V (lanes 32..) of this KV head into the
    // new token's slot (after the barrier: no other wavefront waits for it), then starts its softmax state
    // with the new token: score from the fp16 levels of its codes and its fp16 norm (as the page would give
    // them), weight and value sum at the reference.
    if (own_new && new_ok && wave == kWaves - 1) {
      if (app_lane) {
        const bool is_v = lane >= 32;
        append_quantize<D, KB, VB>(a, is_v, kvh, lane & 31, app, (int64_t)new_pg * a.page_bytes,
                                   (seq_len - 1) % TQ_PAGE_TOKENS, is_v ? s_lutv : s_lutk,
                                   s_newlev[is_v ? (APPEND ? 1 : 0) : 0], &s_newnorm[is_v ? 1 : 0]);
      }
      const int r = hc < G ? hc : 0;
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < D / 4; i += 4) {
        const int coord = (D / 4) * g4 + i;
        const float4 qv = *(const float4 *)&s_q[r][coord];
        const float4 kv = *(const float4 *)&s_newlev[0][coord];
        part = fmaf(qv.x, kv.x, fmaf(qv.y, kv.y, fmaf(qv.z, kv.z, fmaf(qv.w, kv.w, part))));
      }
      const float raw = sum_xor16_32(part);
      if (hc < G) {
        const float x = s_newnorm[0] * raw * a.scale_log2;
        m_run = x + kHeadroom;
        const float p = fast_exp2(-kHeadroom);
        l_part = (g4 == 0 && !lo_part) ? p : 0.f;  // PK: the low lanes' sums are added at the merge
        const float pv = lo_part ? 0.f : p * s_newnorm[1];  // PK: the value enters once, in the high column
        wmax = p * s_newnorm[1];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int nb = 0; nb < NB; nb += 4) {
            const float4 vv = *(const float4 *)&s_newlev[APPEND ? 1 : 0][(D / 16) * (4 * g4 + j) + nb];
            O[nb][j] = pv * vv.x;
            O[nb + 1][j] = pv * vv.y;
            O[nb + 2][j] = pv * vv.z;
            O[nb + 3][j] = pv * vv.w;
          }
      }
    }
  }

  // fp16 V levels of one page pair as MFMA operands: Bop[nb] holds, for lane (c, g4), the level of
  // coordinate (D / 16) * c + nb for the 8 tokens of contraction rows 8 * g4 .. 8 * g4 + 7.
  auto v_operands = [&](const F &cur, half8_t *Bop) {
    if constexpr (LUT) {
      // each code byte (four coordinates of one token) looked up once; the levels of a coordinate for a token pair
      // are then paired into one dword (two fp16 halves)
      uint32_t pairs[8][4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t vw = cur.vw[w >> 1][w & 1];  // tokens 2(w&1), 2(w&1) + 1 of the page: bytes a0, a1, b0, b1
        const uint2 a0 = lut_read2(perm(vw, lut_vb, 0x0C0C0400u)), a1 = lut_read2(perm(vw, lut_vb, 0x0C0C0500u));
        const uint2 b0 = lut_read2(perm(vw, lut_vb, 0x0C0C0600u)), b1 = lut_read2(perm(vw, lut_vb, 0x0C0C0700u));
        pairs[0][w] = perm(b0.x, a0.x, 0x05040100u);
        pairs[1][w] = perm(b0.x, a0.x, 0x07060302u);
        pairs[2][w] = perm(b0.y, a0.y, 0x05040100u);
        pairs[3][w] = perm(b0.y, a0.y, 0x07060302u);
        pairs[4][w] = perm(b1.x, a1.x, 0x05040100u);
        pairs[5][w] = perm(b1.x, a1.x, 0x07060302u);
        pairs[6][w] = perm(b1.y, a1.y, 0x05040100u);
        pairs[7][w] = perm(b1.y, a1.y, 0x07060302u);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) Bop[nb] = from_dwords(pairs[nb][0], pairs[nb][1], pairs[nb][2], pairs[nb][3]);
    } else if constexpr (LUT3) {
      // per code pair k: the four tokens' entries of each page (levels of coordinates 2k and 2k + 1), then paired
      // into the two coordinates' operands (low halves: coordinate 2k, high halves: 2k + 1)
      uint32_t g[2][4];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int j = 0; j < 4; ++j) g[q2][j] = k3_field(cur.vw[q2], j);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) d[j] = lut_read(lut3_addr(g[q2][j], k, lut3_vb));
          lo[2 * q2] = perm(d[1], d[0], 0x05040100u);
          hi[2 * q2] = perm(d[1], d[0], 0x07060302u);
          lo[2 * q2 + 1] = perm(d[3], d[2], 0x05040100u);
          hi[2 * q2 + 1] = perm(d[3], d[2], 0x07060302u);
        }
        Bop[2 * k] = from_dwords(lo[0], lo[1], lo[2], lo[3]);
        Bop[2 * k + 1] = from_dwords(hi[0], hi[1], hi[2], hi[3]);
      }
    } else if constexpr (VB == 3 && D == 128) {
      // each token's 24-bit group (code nb = coordinate nb of the lane's group) spread one code pair per byte;
      // then per byte k and page, the four tokens' pair k gathered into one dword
      uint32_t X[2][4];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        uint32_t Pt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) Pt[j] = spread3(k3_field(cur.vw[q2], j));
#pragma unroll
        for (int k = 0; k < 4; k += 2) {
          const uint32_t sel = k == 0 ? 0x05010400u : 0x07030602u;  // bytes k, k + 1 of two tokens
          const uint32_t a01 = perm(Pt[1], Pt[0], sel), a23 = perm(Pt[3], Pt[2], sel);
          X[q2][k] = perm(a23, a01, 0x05040100u);
          X[q2][k + 1] = perm(a23, a01, 0x07060302u);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint32_t d[4];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) lut3_bytes(X[q2][nb >> 1] >> (3 * (nb & 1)), tv, d[2 * q2], d[2 * q2 + 1]);
        Bop[nb] = from_dwords(d[0], d[1], d[2], d[3]);
      }
    } else if constexpr (VB == 2 && D == 128) {
      // code blocks nb and nb + 4 of a token sit one byte apart: one mask yields four codes, whose low and
      // high level bytes are looked up at once and then paired into fp16 values
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t lo_[4], hi_[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t y = (cur.vw[w >> 1][w & 1] >> (2 * k)) & 0x03030303u;
          const uint32_t lb = perm(tv.lo0, tv.lo0, y), hb = perm(tv.hi0, tv.hi0, y);
          lo_[w] = perm(hb, lb, 0x06020400u);  // code block k
          hi_[w] = perm(hb, lb, 0x07030501u);  // code block k + 4
        }
        Bop[k] = from_dwords(lo_[0], lo_[1], lo_[2], lo_[3]);
        Bop[k + 4] = from_dwords(hi_[0], hi_[1], hi_[2], hi_[3]);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int ci = (D == 128) ? nb : (4 * (c & 1) + nb);  // code index inside the token's 8-coordinate piece
        if constexpr (VB == 2) {
          const int sh = 2 * ci;
          Bop[nb] = from_dwords(lut_v2_pair(cur.vw[0][0] >> sh, tv), lut_v2_pair(cur.vw[0][1] >> sh, tv),
                                lut_v2_pair(cur.vw[1][0] >> sh, tv), lut_v2_pair(cur.vw[1][1] >> sh, tv));
        } else {
          uint16_t hv[8];
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int j = 0; j < 4; ++j) hv[4 * q2 + j] = s_lutv[bits_at<VB>(cur.vw[q2], 8 * VB * j + VB * ci)];
          Bop[nb] = from_halves(hv);
        }
      }
    }
  };

  // FULL: every token of the pair is a cached token of a valid page (no masking needed)
  // PK: the lanes of a head's high column (c < 8) and low column (c ^ 8) hold the same scores once the two partial
  // scores are summed; they then split the softmax by page: the high lane takes page 0 of the pair and the low lane
  // page 1 (its own page), and the two exchange the weights the value MFMA needs at the end. Their reference
  // m_run - ev is the same (every update of it reduces over both lanes), and their softmax sums add up at the merge.
  constexpr int NPG = PK ? 1 : 2;  // pages whose softmax a lane computes
  auto process = [&](const F &cur, int pi, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int pp = p_begin + 2 * pi;
    float rawp[2][4];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      if constexpr (!FULL) {
        if (q2 == 1 && !cur.ok[1]) {  // a run's odd last page: no second page to score (masked below)
#pragma unroll
          for (int j = 0; j < 4; ++j) rawp[1][j] = 0.f;
          continue;
        }
      }
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
      floatx4_t acc2 = {0.f, 0.f, 0.f, 0.f};  // sketched K: <q_s, z>
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) {
        half8_t A;
        if constexpr (LUT1) {
          // byte kb of the code word and of the sketch word: coordinates 8 kb .. 8 kb + 7, one table row each
          const uint4 ks = lut_read4(perm(cur.kw[q2][0], lut1_off, 0x0C0C0400u + ((uint32_t)kb << 8)));
          const uint4 zs = lut_read4(perm(cur.zb[q2], lut1_off, 0x0C0C0400u + ((uint32_t)kb << 8)));
          A = from_dwords(ks.x, ks.y, ks.z, ks.w);
          const half8_t Z = from_dwords(zs.x, zs.y, zs.z, zs.w);
          acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Z, shi[kb], acc2, 0, 0, 0);
          if constexpr (!PK) acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Z, slo[kb], acc2, 0, 0, 0);
        } else if constexpr (LUT) {
          // dword j of the operand: the levels of coordinates 2j, 2j + 1 (code byte j) from table row byte j
          const uint32_t w = cur.kw[q2][kb];
          A = from_dwords(lut_read(perm(w, lut_kb, 0x0C0C0400u)), lut_read(perm(w, lut_kb, 0x0C0C0500u)),
                          lut_read(perm(w, lut_kb, 0x0C0C0600u)), lut_read(perm(w, lut_kb, 0x0C0C0700u)));
        } else if constexpr (KB == 4) {
          A = lut_k4(cur.kw[q2][kb], tk);
        } else if constexpr (LUT3) {
          // dword k of the operand: the levels of coordinates 2k, 2k + 1 (code pair k), natural order
          const uint32_t g = k3_field(cur.kw[q2], kb);
          A = from_dwords(lut_read(lut3_addr(g, 0, lut_kb)), lut_read(lut3_addr(g, 1, lut_kb)),
                          lut_read(lut3_addr(g, 2, lut_kb)), lut_read(lut3_addr(g, 3, lut_kb)));
        } else if constexpr (KB == 3) {
          A = lut_k3(k3_field(cur.kw[q2], kb), tk);
        } else if constexpr (KB == 1) {
          A = signs_to_half8(cur.kw[q2][0], 8 * kb, lev1_hitab, lev1_lo4);
        } else {
          uint16_t hv[8];
#pragma unroll
          for (int p = 0; p < 8; ++p) hv[p] = s_lutk[bits_at<KB>(cur.kw[q2], KB * (8 * kb + p))];
          A = from_halves(hv);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qhi[kb], acc, 0, 0, 0);
        if constexpr (!PK) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qlo[kb], acc, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) rawp[q2][j] = acc[j];
      if constexpr (KPROD) {
        if constexpr (!LUT1) {
#pragma unroll
          for (int kb = 0; kb < KBLK; ++kb) {
            const half8_t A = signs_to_half8(cur.zb[q2], 8 * kb, 0x3CBCu, 0u);  // -1 (0xBC00); a set bit: +1 (0x3C00)
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, shi[kb], acc2, 0, 0, 0);
            if constexpr (!PK) acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, slo[kb], acc2, 0, 0, 0);
          }
        }
        float gam[4];
        unpack4(cur.gm[q2], gam);
#pragma unroll
        for (int j = 0; j < 4; ++j) rawp[q2][j] = fmaf(gam[j] * skratio, acc2[j], rawp[q2][j]);
      }
    }

    // scores of the lane's page(s), in units of softmax scale * log2 e: the fp16 norms enter mixed-precision FMAs
    // directly (fma with a zero addend, not folded to a multiply since signed zeros are kept)
    float s[NPG][4];
    half4_t nv[NPG];
    bool okp[NPG];
    int tpg[NPG];  // first token (sequence position) of the lane's page
    if constexpr (PK) {
      // the partial scores of the high (column c) and low (column c ^ 8) query parts of both pages: both lanes get
      // the sums, each keeps its own page's
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float t0 = rawp[0][j] + xor_lane<8>(rawp[0][j]);
        const float t1 = rawp[1][j] + xor_lane<8>(rawp[1][j]);
        rawp[0][j] = lo_part ? t1 : t0;
      }
      const half4_t nk = as_half4(lo_part ? cur.nk[1] : cur.nk[0]);
      nv[0] = as_half4(lo_part ? cur.nv[1] : cur.nv[0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) s[0][j] = fmaf((float)nk[j], rawp[0][j], 0.f);
      okp[0] = lo_part ? cur.ok[1] : cur.ok[0];
      tpg[0] = (pp + (lo_part ? 1 : 0)) * TQ_PAGE_TOKENS;
    } else {
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const half4_t nk = as_half4(cur.nk[q2]);
        nv[q2] = as_half4(cur.nv[q2]);
#pragma unroll
        for (int j = 0; j < 4; ++j) s[q2][j] = fmaf((float)nk[j], rawp[q2][j], 0.f);
        okp[q2] = cur.ok[q2];
        tpg[q2] = (pp + q2) * TQ_PAGE_TOKENS;
      }
    }

    // tokens past the sequence end or in an invalid page: weight 0 (their bytes are not read as numbers).
    // A masked score is a finite, very negative value so that a zero softmax scale never meets an infinity.
    bool okm[NPG][4];
    if constexpr (!FULL) {
#pragma unroll
      for (int q2 = 0; q2 < NPG; ++q2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          okm[q2][j] = okp[q2] && tpg[q2] + 4 * g4 + j < seq_mem;
          s[q2][j] = okm[q2][j] ? s[q2][j] : -3.0e38f;
          nv[q2][j] = okm[q2][j] ? nv[q2][j] : (_Float16)0.f;
        }
    }

    // online softmax in base 2 (m_run is in units of scale * log2 e); this lane holds head column c,
    // tokens 4*g4 .. 4*g4+3 of its page(s)
    float mxl = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
    if constexpr (NPG == 2) mxl = fmaxf(mxl, fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    // m_run bounds the scores seen so far. When a score passes it, the new reference is set kHeadroom above
    // the new maximum, so the rescale (which any reference allows: it cancels between the sums and the
    // weights) runs only on real jumps of the maximum. The test is taken on the lane's own scores; the
    // column's maximum (over its four lanes, and PK: the other page's lanes) only when some lane passes.
    if (__any(colscale * mxl > m_run)) {
      // O holds head column c in this lane, as do m_run and l_part: the rescale stays in the lane
      float mc = max_xor32(max_xor16(mxl));
      if constexpr (PK) mc = fmaxf(mc, xor_lane<8>(mc));
      const float m_new = colscale * mc;
      const bool up = m_new > m_run;
      const float m_ref = up ? m_new + kHeadroom : m_run;
      const float alpha = up ? ((m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_ref)) : 1.f;
      l_part *= alpha;
      wmax *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) O[nb] *= alpha;
      m_run = m_ref;
    }
    // weights against the effective reference m_run - ev: p <= 2^ev, value weights P' = p ||v||
    const float m_eff = m_run - ev;
    float pv[NPG][4];
#pragma unroll
    for (int q2 = 0; q2 < NPG; ++q2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p = fast_exp2(fmaf(s[q2][j], colscale, -m_eff));
        if constexpr (!FULL) p = okm[q2][j] ? p : 0.f;
        l_part += p;
        pv[q2][j] = fmaf((float)nv[q2][j], p, 0.f);
      }
    }
    float pvl = fmaxf(fmaxf(pv[0][0], pv[0][1]), fmaxf(pv[0][2], pv[0][3]));
    if constexpr (NPG == 2) pvl = fmaxf(pvl, fmaxf(fmaxf(pv[1][0], pv[1][1]), fmaxf(pv[1][2], pv[1][3])));
    wmax = fmaxf(wmax, pvl);
    if (__any(pvl > kWeightHigh || (wmax < kWeightLow && pvl > 0.f))) {
      float wc = max_xor32(max_xor16(wmax));
      if constexpr (PK) wc = fmaxf(wc, xor_lane<8>(wc));
      const float f = weight_shift(wc, ev, wmax);
      l_part *= f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) O[nb] *= f;
#pragma unroll
      for (int q2 = 0; q2 < NPG; ++q2)
#pragma unroll
        for (int j = 0; j < 4; ++j) pv[q2][j] *= f;
    }
    half8_t phi, plo;
    if constexpr (PK) {
      // the lane's four weights as fp16 hi + lo; the high column takes the high parts of both pages, the low column
      // the low parts: each lane keeps one of its own and receives the other page's from lane c ^ 8 (a row rotation
      // by 8 written only to the lanes of one half-row: bank mask 0x3 = lanes 0..7 of each 16-lane row, 0xC = 8..15)
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const float2_t pw = {pv[0][j], pv[0][j + 1]};
        const half2_t h = __builtin_convertvector(pw, half2_t);
        const float2_t hf = __builtin_convertvector(h, float2_t);
        // pw - hi as one mixed-precision FMA per element (the fp16 high part read directly)
        const float2_t t = {fmaf(neg_one, hf[0], pw[0]), fmaf(neg_one, hf[1], pw[1])};
        const half2_t l = __builtin_convertvector(t, half2_t);
        hw[j / 2] = __builtin_bit_cast(uint32_t, h);
        lw[j / 2] = __builtin_bit_cast(uint32_t, l);
      }
      uint32_t d[4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        // page 0 part: high lanes keep their own high part, low lanes take the low part of lane c - 8
        d[k] = (uint32_t)__builtin_amdgcn_update_dpp((int)hw[k], (int)lw[k], 0x128, 0xF, 0xC, false);
        // page 1 part: low lanes keep their own low part, high lanes take the high part of lane c + 8
        d[2 + k] = (uint32_t)__builtin_amdgcn_update_dpp((int)lw[k], (int)hw[k], 0x128, 0xF, 0x3, false);
      }
      phi = from_dwords(d[0], d[1], d[2], d[3]);
    } else {
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const float2_t pw = {pv[q2][j], pv[q2][j + 1]};
          const half2_t h = __builtin_convertvector(pw, half2_t);
          const half2_t l = __builtin_convertvector(pw - __builtin_convertvector(h, float2_t), half2_t);
          phi[4 * q2 + j] = h[0];
          phi[4 * q2 + j + 1] = h[1];
          plo[4 * q2 + j] = l[0];
          plo[4 * q2 + j + 1] = l[1];
        }
      }
    }

    // values, transposed: O^T[coords][head columns] += Vhat^T[coords][32 tokens] * P'^T[32 tokens][heads].
    // The V operand registers are the same as for Vhat as the right-hand operand; swapping the operands
    // of the MFMA puts the query heads in the columns, next to their softmax state.
    half8_t Bop[NB];
    v_operands(cur, Bop);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Bop[nb], phi, O[nb], 0, 0, 0);
      if constexpr (!PK) O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Bop[nb], plo, O[nb], 0, 0, 0);
    }
  };

  // ring of R fragments: R - 1 page pairs in flight while one is processed
  for (int i = wave; i < npairs; i += R * kWaves) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int ii = i + r * kWaves;
      const int nx = ii + (R - 1) * kWaves;
      const int2 pg = *(const int2 *)&s_pid[2 * nx];  // pages p_begin + 2 nx and the next
      load_pages_id<D, KB, KPROD, VB>(a, lo, pg, f[(r + R - 1) % R]);
      if (ii < n_full) process(f[r], ii, std::true_type{});
      else if (ii < npairs) process(f[r], ii, std::false_type{});
    }
  }

  // ---- 4. merge the wavefronts of this work-group: rescale to the work-group max, then sum over the
  //         waves in a fixed order (deterministic). Lane (c, g4) holds head c (real when c < G) and,
  //         in O[nb][j], coordinate (D / 16) * (4 * g4 + j) + nb of its rotated value sum.
  if constexpr (PK) {
    // value sums of the high and low columns of each head: lanes c < 8 hold the total
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) O[nb][j] += xor_lane<8>(O[nb][j]);
  }
  // the sums are in units of the effective reference m_run - ev
  const float m_eff = m_run - ev;
  {
    // PK: the high and low lanes of a column summed the weights of different pages
    const float l_tot = sum_xor16_32(PK ? l_part + xor_lane<8>(l_part) : l_part);
    if (g4 == 0) {
      s_m[wave][c] = m_eff;
      s_l[wave][c] = l_tot;
    }
  }
  __syncthreads();  // also: every wave is past its use of s_q / s_qs
  if (c < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][c]);
    const float e = (M == -INFINITY || m_eff == -INFINITY) ? 0.f : fast_exp2(m_eff - M);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) O[nb] *= e;
  }
  if (tid < G) {
    const int row = tid;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][row]);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (s_m[w][row] != -INFINITY) L = fmaf(fast_exp2(s_m[w][row] - M), s_l[w][row], L);
    }
    s_rowm[row] = M;
    s_rowl[row] = L;
  }
  // this lane's 4 x NB sums as float4 runs of consecutive coordinates of row (head) c
  auto put_rows = [&](float *row_base) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; nb += 4)
        *(float4 *)(row_base + (D / 16) * (4 * g4 + j) + nb) = float4{O[nb][j], O[nb + 1][j], O[nb + 2][j], O[nb + 3][j]};
  };
  auto add_rows = [&](const float *row_base) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nb = 0; nb < NB; nb += 4) {
        const float4 t = *(const float4 *)(row_base + (D / 16) * (4 * g4 + j) + nb);
        O[nb][j] += t.x;
        O[nb + 1][j] += t.y;
        O[nb + 2][j] += t.z;
        O[nb + 3][j] += t.w;
      }
  };
  // every wave deposits its real rows; one fixed-order pass sums them
  constexpr int RMAX = (4 * QF) / (kWaves * D);  // rows that fit in the arena per wave (8)
  float acc_out[(16 * D + NT - 1) / NT];         // this thread's merged elements (row-major over G x D)
  if (G <= RMAX) {
    float(*dep)[RMAX][D] = (float(*)[RMAX][D])arena;
    if (c < G) put_rows(dep[wave][c]);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < (16 * D + NT - 1) / NT; ++q) {
      const int idx = tid + q * NT;
      float t = 0.f;
      if (idx < G * D) {
        const int row = idx / D, k = idx % D;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t += dep[w][row][k];
      }
      acc_out[q] = t;
    }
  } else {
    float(*tree)[16][D] = (float(*)[16][D])arena;  // [kWaves / 2][16][D]
#pragma unroll
    for (int half = kWaves / 2; half >= 1; half >>= 1) {
      if (wave >= half && wave < 2 * half) put_rows(tree[wave - half][c]);
      __syncthreads();
      if (wave < half) add_rows(tree[wave][c]);
      __syncthreads();
    }
    if (wave == 0) put_rows(tree[0][c]);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < (16 * D + NT - 1) / NT; ++q) {
      const int idx = tid + q * NT;
      acc_out[q] = idx < G * D ? tree[0][idx / D][idx % D] : 0.f;
    }
  }

  // ---- 5. one run: finish here; several runs: write this run's partial for the combine kernel
  const int64_t S = a.n_splits;
  if (S > 1) {
#pragma unroll
    for (int q = 0; q < (16 * D + NT - 1) / NT; ++q) {
      const int idx = tid + q * NT;
      if (idx < G * D) {
        const int row = idx / D, k = idx % D;
        const int64_t bh = (int64_t)b * a.Hq + head0 + row;
        a.part_o[(bh * S + split) * D + k] = acc_out[q];
      }
    }
    if (tid < G) {
      const int64_t bh = (int64_t)b * a.Hq + head0 + tid;
      a.part_ml[(bh * S + split) * 2] = s_rowm[tid];
      a.part_ml[(bh * S + split) * 2 + 1] = s_rowl[tid];
    }
    return;
  }
  __syncthreads();  // the deposit buffer is read before it becomes the output buffer
  float(*fin)[D] = (float(*)[D])arena;
#pragma unroll
  for (int q = 0; q < (16 * D + NT - 1) / NT; ++q) {
    const int idx = tid + q * NT;
    if (idx < G * D) {
      const int row = idx / D, k = idx % D;
      const float L = s_rowl[row];
      fin[row][k] = L > 0.f ? acc_out[q] / L : 0.f;
    }
  }
  __syncthreads();
  lds_wht<D, NT>(fin, G, tid);
  {
    const uint32_t *vsw = (const uint32_t *)(a.vcb + a.vo.signs);
    for (int idx = tid; idx < G * D; idx += NT) {
      const int row = idx / D, k = idx % D;
      float o = fin[row][k] * (1.0f / D);
      if ((vsw[k >> 5] >> (k & 31)) & 1u) o = -o;
      a.out[((int64_t)b * a.Hq + head0 + row) * D + k] = o;
    }
  }
}

// Merge of the runs of one (sequence, query head): log-sum-exp weights, weighted sum of the value sums,
// division by the total weight, then (ROT: sums in the rotated domain) R_V^T by butterflies across one
// wavefront, and the fp32 row.
template <int D, bool ROT>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  constexpr int NT = 256;
  constexpr int ITEMS = D / 4;        // float4 columns of a row
  constexpr int GROUPS = NT / ITEMS;  // runs are strided over this many thread groups
  constexpr int PRE = 8;              // partial rows per thread loaded before the weights are known
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int S = a.n_splits;
  __shared__ float s_w[kMlCap], s_lw[kMlCap];
  __shared__ __align__(16) float red[GROUPS][D];
  __shared__ float s_L;
  const int k4 = tid % ITEMS, grp = tid / ITEMS;
  const float4 *po = (const float4 *)(a.part_o + bh * S * D) + k4;
  float4 pre[PRE];
#pragma unroll
  for (int q = 0; q < PRE; ++q) {
    const int s2 = grp + q * GROUPS;
    pre[q] = s2 < S ? po[(int64_t)s2 * ITEMS] : float4{0.f, 0.f, 0.f, 0.f};
  }
  // wavefront 0: the runs' maxima and sums, the log-sum-exp weights of the runs and the total weight
  // (cross-lane reductions in registers, no LDS round trips)
  if (tid < 64) {
    float M = -INFINITY;
    for (int s2 = lane; s2 < S; s2 += 64) {
      const float m = a.part_ml[(bh * S + s2) * 2];
      s_w[s2] = m;
      s_lw[s2] = a.part_ml[(bh * S + s2) * 2 + 1];
      M = fmaxf(M, m);
    }
    M = wave_max(M, lane);
    float L = 0.f;
    for (int s2 = lane; s2 < S; s2 += 64) {
      const float ms = s_w[s2];
      const float e = (M == -INFINITY || ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
      s_w[s2] = e;
      L = fmaf(e, s_lw[s2], L);
    }
    L = wave_sum(L, lane);
    if (lane == 0) s_L = L;
  }
  __syncthreads();
  float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < PRE; ++q) {
    const int s2 = grp + q * GROUPS;
    const float e = s2 < S ? s_w[s2] : 0.f;
    acc.x = fmaf(e, pre[q].x, acc.x);
    acc.y = fmaf(e, pre[q].y, acc.y);
    acc.z = fmaf(e, pre[q].z, acc.z);
    acc.w = fmaf(e, pre[q].w, acc.w);
  }
  for (int s2 = grp + PRE * GROUPS; s2 < S; s2 += GROUPS) {
    const float e = s_w[s2];
    const float4 v = po[(int64_t)s2 * ITEMS];
    acc.x = fmaf(e, v.x, acc.x);
    acc.y = fmaf(e, v.y, acc.y);
    acc.z = fmaf(e, v.z, acc.z);
    acc.w = fmaf(e, v.w, acc.w);
  }
  *(float4 *)&red[grp][4 * k4] = acc;
  __syncthreads();
  if (tid >= 64) return;
  // wavefront 0: the group sums of coordinates lane (and lane + 64), divided by the total weight, then
  // (ROT) R_V^T = diag(s) H / sqrt(d) on the levels' N(0,1) units (another 1 / sqrt(d)) by butterflies
  const float inv = s_L > 0.f ? 1.0f / s_L : 0.f;
  float x0 = 0.f, x1 = 0.f;
#pragma unroll
  for (int g = 0; g < GROUPS; ++g) {
    x0 += red[g][lane];
    if constexpr (D == 128) x1 += red[g][lane + 64];
  }
  x0 *= inv;
  x1 *= inv;
  if constexpr (ROT) {
    x0 = wht_stage<1>(x0, lane);
    x1 = wht_stage<1>(x1, lane);
    x0 = wht_stage<2>(x0, lane);
    x1 = wht_stage<2>(x1, lane);
    x0 = wht_stage<4>(x0, lane);
    x1 = wht_stage<4>(x1, lane);
    x0 = wht_stage<8>(x0, lane);
    x1 = wht_stage<8>(x1, lane);
    x0 = wht_stage<16>(x0, lane);
    x1 = wht_stage<16>(x1, lane);
    x0 = wht_stage<32>(x0, lane);
    x1 = wht_stage<32>(x1, lane);
    if (D == 128) {
      const float u = x0;
      x0 = u + x1;
      x1 = u - x1;
    }
    const uint32_t *sw = (const uint32_t *)(a.vcb + a.vo.signs);
    x0 *= (1.0f / D);
    if ((sw[lane >> 5] >> (lane & 31)) & 1u) x0 = -x0;
    if (D == 128) {
      x1 *= (1.0f / D);
      if ((sw[(lane + 64) >> 5] >> (lane & 31)) & 1u) x1 = -x1;
    }
  }
  a.out[bh * D + lane] = x0;
  if (D == 128) a.out[bh * D + lane + 64] = x1;
}

template <int D, int KB, bool KPROD, int VB, bool PK>
void launch(const DecodeArgs &a, hipStream_t stream) {
  if (a.passes & kPassScan) {
    dim3 grid(a.n_splits, a.Hkv, a.B);
    if constexpr (!KPROD && KB <= 4 && VB <= 4) {
      if (a.k_new) {
        hipLaunchKernelGGL((decode_kernel<D, KB, KPROD, VB, true, PK>), grid, dim3(64 * kWaves), 0, stream, a);
      } else {
        hipLaunchKernelGGL((decode_kernel<D, KB, KPROD, VB, false, PK>), grid, dim3(64 * kWaves), 0, stream, a);
      }
    } else {
      hipLaunchKernelGGL((decode_kernel<D, KB, KPROD, VB, false, PK>), grid, dim3(64 * kWaves), 0, stream, a);
    }
  }
  if ((a.passes & kPassCombine) && a.n_splits > 1)
    hipLaunchKernelGGL((combine_kernel<D, true>), dim3(a.B * a.Hq), dim3(256), 0, stream, a);
}

template <int D, int KB, bool KPROD, bool PK>
bool dispatch_v(int vb, const DecodeArgs &a, hipStream_t s) {
  switch (vb) {
    case 1: launch<D, KB, KPROD, 1, PK>(a, s); return true;
    case 2: launch<D, KB, KPROD, 2, PK>(a, s); return true;
    case 3: launch<D, KB, KPROD, 3, PK>(a, s); return true;
    case 4: launch<D, KB, KPROD, 4, PK>(a, s); return true;
    case 8: launch<D, KB, KPROD, 8, PK>(a, s); return true;
  }
  return false;
}

template <int D, bool PK>
bool dispatch_k(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s) {
  if (kprod) {
    switch (kb) {
      case 1: return dispatch_v<D, 1, true, PK>(vb, a, s);
      case 2: return dispatch_v<D, 2, true, PK>(vb, a, s);
      case 3: return dispatch_v<D, 3, true, PK>(vb, a, s);
    }
    return false;
  }
  switch (kb) {
    case 1: return dispatch_v<D, 1, false, PK>(vb, a, s);
    case 2: return dispatch_v<D, 2, false, PK>(vb, a, s);
    case 3: return dispatch_v<D, 3, false, PK>(vb, a, s);
    case 4: return dispatch_v<D, 4, false, PK>(vb, a, s);
    case 8: return dispatch_v<D, 8, false, PK>(vb, a, s);
  }
  return false;
}

}  // namespace

// The kernels are instantiated in four objects (this file is compiled once per part, in parallel):
// part 1 holds head_dim 128 with packed columns (at most 8 query heads per KV head) and the launcher,
// part 2 head_dim 128 with one column per query head, parts 3 and 4 the same for head_dim 64; no part = all.
bool decode_dispatch_d128_pk(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s);
bool decode_dispatch_d128(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s);
bool decode_dispatch_d64_pk(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s);
bool decode_dispatch_d64(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s);

#if !defined(TQ_DECODE_PART) || TQ_DECODE_PART == 1
bool decode_dispatch_d128_pk(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s) {
  return dispatch_k<128, true>(kb, kprod, vb, a, s);
}
#endif
#if !defined(TQ_DECODE_PART) || TQ_DECODE_PART == 2
bool decode_dispatch_d128(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s) {
  return dispatch_k<128, false>(kb, kprod, vb, a, s);
}
#endif
#if !defined(TQ_DECODE_PART) || TQ_DECODE_PART == 3
bool decode_dispatch_d64_pk(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s) {
  return dispatch_k<64, true>(kb, kprod, vb, a, s);
}
#endif
#if !defined(TQ_DECODE_PART) || TQ_DECODE_PART == 4
bool decode_dispatch_d64(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s) {
  return dispatch_k<64, false>(kb, kprod, vb, a, s);
}
#endif

#if !defined(TQ_DECODE_PART) || TQ_DECODE_PART == 1
// Split partials of tq_decode_attention_noalloc: a fixed array in the library's code object, one copy per device.
// Host code never uses this name as an address (on the host it is only a handle of the device symbol): the
// address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

int decode_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return TQ_ENOTSUP;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TQ_EHIP;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return TQ_OK;
}

int launch_combine_plain(const float *part_o, const float *part_ml, int n_splits, int64_t rows, int head_dim,
                         float *out, hipStream_t stream) {
  DecodeArgs a{};
  a.part_o = const_cast<float *>(part_o);
  a.part_ml = const_cast<float *>(part_ml);
  a.n_splits = n_splits;
  a.out = out;
  if (head_dim == 128) {
    hipLaunchKernelGGL((combine_kernel<128, false>), dim3(rows), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((combine_kernel<64, false>), dim3(rows), dim3(256), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

int launch_decode(const PageGeom &g, const DecodeWs &ws, const void *pages, int64_t num_pages,
                  const void *q, int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                  int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                  const void *k_cb, const void *v_cb, void *workspace, float *out,
                  int passes, const void *k_new, const void *v_new, int kv_dtype, hipStream_t stream) {
  DecodeArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.kv_dtype = kv_dtype;
  a.pages = (const unsigned char *)pages;
  a.num_pages = num_pages;
  a.num_pages32 = (int)std::min<int64_t>(num_pages, 0x7FFFFFFF);
  a.page_bytes = g.page_bytes;
  a.k_codes = g.k_codes;
  a.k_norms = g.k_norms;
  a.k_qjl = g.k_qjl;
  a.k_gamma = g.k_gamma;
  a.v_codes = g.v_codes;
  a.v_norms = g.v_norms;
  a.q = q;
  a.q_dtype = q_dtype;
  a.B = batch;
  a.Hq = num_q_heads;
  a.Hkv = g.num_kv_heads;
  a.G = num_q_heads / g.num_kv_heads;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.scale_log2 = softmax_scale * kLog2e;
  a.kcb = (const unsigned char *)k_cb;
  a.vcb = (const unsigned char *)v_cb;
  a.ko = g.kcb;
  a.vo = g.vcb;
  unsigned char *w = (unsigned char *)workspace;
  a.part_o = (float *)(w + ws.part_o_off);
  a.part_ml = (float *)(w + ws.part_ml_off);
  a.n_splits = ws.n_splits;
  a.pps = ws.pages_per_split;
  a.out = out;
  a.passes = passes;
  const bool kprod = g.k_mode == TQ_PROD;
  const int kb = g.k_mse_bits, vb = g.v_mse_bits;
  const bool pk = a.G <= 8;
  const bool ok = g.head_dim == 128
                      ? (pk ? decode_dispatch_d128_pk(kb, kprod, vb, a, stream) : decode_dispatch_d128(kb, kprod, vb, a, stream))
                      : (pk ? decode_dispatch_d64_pk(kb, kprod, vb, a, stream) : decode_dispatch_d64(kb, kprod, vb, a, stream));
  if (!ok) return TQ_ENOTSUP;
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}
#endif

}  // namespace tq
