// Uncompressed comparators of the decode path: the same paged GQA decode attention over a bf16 cache and
// over an FP8 (E4M3) cache with one scale per tensor, so that the compressed path can be measured against
// the bytes it saves ("Where This Fits in the Inference Stack", "What Changes When KV Cache Is 4x Smaller":
// decode reads the whole cache from HBM every step, and a 4x smaller cache moves 4x fewer bytes; "Who
// Should Care", "The Three Layers of Compression": an FP8 cache is the hardware-native 2x baseline; "Why
// the KV Cache Exists", "The KV Cache Solution": the new query attends over every cached token).
//
// Page layout (16 token slots per page, every KV head of the layer): K as [head][slot][d], then V as
// [head][d][slot] (each head's values of a page stored coordinate-major, as paged-attention caches lay
// them out, so that one lane reads consecutive tokens of one coordinate), 2-byte bf16 or 1-byte E4M3
// elements. An E4M3 byte stands for scale * its value: the K scale is folded into the logit scale and the
// V scale into the output; the bytes are widened to bf16 (exactly: every E4M3 value is a bf16 value) with
// v_cvt_scalef32_pk_bf16_fp8 and go through the same bf16 MFMAs.
//
// The kernel mirrors the compressed split-K kernel: grid (runs, KV heads, batch), 8 wavefronts per
// work-group walking page pairs (32 tokens); scores S^T = K Q and values O^T += V^T P^T on
// v_mfma_f32_16x16x32_bf16 with the query and the weights as bf16 high + low parts (one column each
// when a KV head has at most 8 query heads); online softmax in base 2; wavefront merge in LDS; split
// partials merged by the shared combine kernel. No rotation anywhere.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "tq_common.h"
#include "tq_internal.h"
#include "tq_lanes.h"
#include "tq_quant_common.h"

namespace tq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kDWaves = 8;
constexpr float kDHeadroom = 4.0f;  // log2 units between the running maximum and the weight reference

struct DenseArgs {
  const unsigned char *pages;
  int num_pages32;
  uint32_t page_bytes, v_off;
  const void *q;
  int q_dtype;
  int Hq, Hkv, G;
  const int32_t *page_table;
  int max_pages;
  const int32_t *seq_lens;
  float scale_log2;  // softmax scale * log2(e), times the K scale for E4M3 pages
  float v_scale;     // E4M3 pages: V scale, applied to the outputs
  float *part_o, *part_ml;
  int n_splits, pps;
  float *out;
};

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  const __bf16 h = (__bf16)x;  // round to nearest even
  uint16_t u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}

// One thread per (token, head, 8-coordinate group): K as one 16-byte store, V as 8 strided 2-byte stores.
__global__ __launch_bounds__(256) void dense_write_kernel(unsigned char *pages, int64_t num_slots, uint32_t page_bytes,
                                                          uint32_t v_off, int D, int H, const void *k, const void *v,
                                                          int dtype, int64_t n_tok, const int64_t *slots) {
  const int groups = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_tok * H * groups) return;
  const int g = (int)(gid % groups);
  const int64_t th = gid / groups;
  const int h = (int)(th % H);
  const int64_t t = th / H;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;  // skipped slot
  float xk[8], xv[8];
  load8(k, (t * H + h) * D + 8 * g, dtype, xk);
  load8(v, (t * H + h) * D + 8 * g, dtype, xv);
  unsigned char *pg = pages + (slot / TQ_PAGE_TOKENS) * (int64_t)page_bytes;
  const int s = (int)(slot % TQ_PAGE_TOKENS);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = bf16_bits(xk[2 * i]) | ((uint32_t)bf16_bits(xk[2 * i + 1]) << 16);
  *(uint4 *)(pg + ((int64_t)(h * TQ_PAGE_TOKENS + s) * D + 8 * g) * 2) = uint4{w[0], w[1], w[2], w[3]};
  uint16_t *vcol = (uint16_t *)(pg + v_off) + ((int64_t)h * D + 8 * g) * TQ_PAGE_TOKENS + s;
#pragma unroll
  for (int i = 0; i < 8; ++i) vcol[i * TQ_PAGE_TOKENS] = bf16_bits(xv[i]);
}

// E4M3 byte of y, rounded to nearest, ties to even, saturated to +-448 (bias 7; below 2^-6 the grid step is
// 2^-9, above it 8 steps per binade; a carry out of the mantissa moves to the next exponent by itself).
// Finite inputs only.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const int e = (int)(__float_as_uint(a) >> 23) - 127;  // floor(log2 a), -6 .. 8
    code = (uint32_t)((e + 7) * 8) + (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e)) - 8u;
  }
  return sign | code;
}

// E4M3 pages: one thread per (token, head, 8-coordinate group): K as one 8-byte store, V as 8 strided byte
// stores; each element is the fp32 quotient x / scale, correctly rounded, then encoded.
__global__ __launch_bounds__(256) void dense_write_fp8_kernel(unsigned char *pages, int64_t num_slots,
                                                              uint32_t page_bytes, uint32_t v_off, int D, int H,
                                                              const void *k, const void *v, int dtype,
                                                              int64_t n_tok, const int64_t *slots, float k_scale,
                                                              float v_scale) {
  const int groups = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_tok * H * groups) return;
  const int g = (int)(gid % groups);
  const int64_t th = gid / groups;
  const int h = (int)(th % H);
  const int64_t t = th / H;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;  // skipped slot
  float xk[8], xv[8];
  load8(k, (t * H + h) * D + 8 * g, dtype, xk);
  load8(v, (t * H + h) * D + 8 * g, dtype, xv);
  unsigned char *pg = pages + (slot / TQ_PAGE_TOKENS) * (int64_t)page_bytes;
  const int s = (int)(slot % TQ_PAGE_TOKENS);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i >> 2] |= e4m3_rne(__fdiv_rn(xk[i], k_scale)) << (8 * (i & 3));
  *(uint2 *)(pg + (int64_t)(h * TQ_PAGE_TOKENS + s) * D + 8 * g) = uint2{w[0], w[1]};
  unsigned char *vcol = pg + v_off + ((int64_t)h * D + 8 * g) * TQ_PAGE_TOKENS + s;
#pragma unroll
  for (int i = 0; i < 8; ++i) vcol[i * TQ_PAGE_TOKENS] = (unsigned char)e4m3_rne(__fdiv_rn(xv[i], v_scale));
}

__device__ __forceinline__ bf16x8_t bf16x8_of(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Eight E4M3 bytes (w0 bytes 0-3, then w1) widened to bf16, exactly.
__device__ __forceinline__ bf16x8_t bf16x8_of_fp8(uint32_t w0, uint32_t w1) {
  const uint4 u{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
  return __builtin_bit_cast(bf16x8_t, u);
}

// Register fragment of one page pair: K rows (token c, the lane's D/4 coordinates) and, per 16-coordinate
// block, V of coordinate row c for the lane's 4 tokens of page 0 and of page 1. bf16: the value operand as
// loaded (page 0 in x, y; page 1 in z, w). E4M3: 4 bytes per page (page 0 in x, page 1 in y).
template <int D, bool F8>
struct DFrag {
  uint4 k[2][D / 32];
  uint4 v[D / 16];
  bool ok[2];
};
template <int D>
struct DFrag<D, true> {
  uint4 k[2][D / 64];
  uint2 v[D / 16];
  bool ok[2];
};

template <int D>
__device__ __forceinline__ void dense_load_pages(const DenseArgs &a, int kvh, int c, int g4, int pg0, int pg1,
                                                 DFrag<D, true> &f) {
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int pg = __builtin_amdgcn_readfirstlane(q2 ? pg1 : pg0);
    const bool ok = pg >= 0 && pg < a.num_pages32;
    f.ok[q2] = ok;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.pages + (int64_t)(ok ? pg : 0) * a.page_bytes), (short)0, ok ? (int)a.page_bytes : 0, 0x00020000);
    const uint32_t koff = (uint32_t)(kvh * TQ_PAGE_TOKENS + c) * D + (D / 4) * g4;
#pragma unroll
    for (int kb = 0; kb < D / 64; ++kb)
      f.k[q2][kb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, koff + 16 * kb, 0, 0));
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      const uint32_t voff = a.v_off + (uint32_t)(kvh * D + 16 * nb + c) * TQ_PAGE_TOKENS + 4 * g4;
      const uint32_t t = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
      if (q2) f.v[nb].y = t;
      else f.v[nb].x = t;
    }
  }
}

template <int D>
__device__ __forceinline__ void dense_load_pages(const DenseArgs &a, int kvh, int c, int g4, int pg0, int pg1,
                                                 DFrag<D, false> &f) {
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int pg = __builtin_amdgcn_readfirstlane(q2 ? pg1 : pg0);
    const bool ok = pg >= 0 && pg < a.num_pages32;
    f.ok[q2] = ok;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.pages + (int64_t)(ok ? pg : 0) * a.page_bytes), (short)0, ok ? (int)a.page_bytes : 0, 0x00020000);
    const uint32_t koff = ((uint32_t)(kvh * TQ_PAGE_TOKENS + c) * D + (D / 4) * g4) * 2;
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb)
      f.k[q2][kb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, koff + 16 * kb, 0, 0));
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      const uint32_t voff = a.v_off + ((uint32_t)(kvh * D + 16 * nb + c) * TQ_PAGE_TOKENS + 4 * g4) * 2;
      const uint2 t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
      if (q2) {
        f.v[nb].z = t.x;
        f.v[nb].w = t.y;
      } else {
        f.v[nb].x = t.x;
        f.v[nb].y = t.y;
      }
    }
  }
}

// MFMA operands of a fragment: the K rows of 32-coordinate block kb of page q2, and the V rows of
// 16-coordinate block nb of both pages.
template <int D>
__device__ __forceinline__ bf16x8_t k_operand(const DFrag<D, false> &f, int q2, int kb) { return bf16x8_of(f.k[q2][kb]); }
template <int D>
__device__ __forceinline__ bf16x8_t k_operand(const DFrag<D, true> &f, int q2, int kb) {
  const uint4 u = f.k[q2][kb >> 1];
  return (kb & 1) ? bf16x8_of_fp8(u.z, u.w) : bf16x8_of_fp8(u.x, u.y);
}
template <int D>
__device__ __forceinline__ bf16x8_t v_operand(const DFrag<D, false> &f, int nb) { return bf16x8_of(f.v[nb]); }
template <int D>
__device__ __forceinline__ bf16x8_t v_operand(const DFrag<D, true> &f, int nb) {
  return bf16x8_of_fp8(f.v[nb].x, f.v[nb].y);
}

// PK (at most 8 query heads per KV head): MFMA column c carries query head c & 7, its high bf16 part in
// columns 0-7 and its low part in columns 8-15; otherwise column c is head c and each product is a high +
// low pair of MFMAs.
template <int D, bool PK, bool F8>
__global__ __launch_bounds__(64 * kDWaves) void dense_decode_kernel(DenseArgs a) {
  constexpr int NT = 64 * kDWaves;
  constexpr int KBLK = D / 32;  // 32-coordinate blocks of the score contraction
  constexpr int NB = D / 16;    // 16-coordinate blocks of the value contraction
  constexpr int QS = D + 4;
  // fragments in the ring: R - 1 pairs in flight while one is processed (a deeper ring measured slower
  // for E4M3 pages too, though their fragments would fit)
  constexpr int R = 2;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g4 = lane >> 4;
  const int hc = PK ? (c & 7) : c;
  const bool lo_part = PK && c >= 8;
  const float lo_neg = lo_part ? -1.f : 0.f;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.G;
  const int head0 = kvh * G;

  __shared__ __align__(16) float s_q[16][QS];
  __shared__ int s_pid[kDecodePidCap];
  __shared__ float s_m[kDWaves][16], s_l[kDWaves][16];
  __shared__ float s_rowm[16], s_rowl[16];
  __shared__ __align__(16) float dep[kDWaves][16][D];

  const bool last_run = split == a.n_splits - 1;
  const int p_begin = split * a.pps;
  const int p_cap = last_run ? a.max_pages : min(p_begin + a.pps, a.max_pages);
  typedef const __attribute__((address_space(4))) int32_t *const_i32;  // read through the scalar cache
  const const_i32 ptab = (const_i32)a.page_table + (int64_t)b * a.max_pages;
  int seq_len = ((const_i32)a.seq_lens)[b];
  seq_len = seq_len < 0 ? 0 : min(seq_len, a.max_pages * TQ_PAGE_TOKENS);
  const int npages = (seq_len + TQ_PAGE_TOKENS - 1) / TQ_PAGE_TOKENS;
  const int p_end = last_run ? npages : min(p_begin + a.pps, npages);
  const int npairs = p_end > p_begin ? (p_end - p_begin + 1) / 2 : 0;

  // this wavefront's first pair in flight (page ids through the scalar cache), then the run's page ids
  // and the queries into LDS
  DFrag<D, F8> f[R];
#pragma unroll
  for (int j = 0; j < R - 1; ++j) {
    const int pp = p_begin + 2 * (wave + j * kDWaves);
    const int id0 = pp < p_end ? ptab[pp] : -1;
    const int id1 = pp + 1 < p_end ? ptab[pp + 1] : -1;
    dense_load_pages<D>(a, kvh, c, g4, id0, id1, f[j]);
  }
  int pids_ok = 1;
  for (int j = tid; j < p_end - p_begin; j += NT) {
    const int pg = a.page_table[(int64_t)b * a.max_pages + p_begin + j];
    s_pid[j] = pg;
    pids_ok &= (pg >= 0 && pg < a.num_pages32) ? 1 : 0;
  }
  for (int idx = tid; idx < G * D; idx += NT)
    s_q[idx / D][idx % D] = load_elem(a.q, ((int64_t)b * a.Hq + head0 + idx / D) * D + idx % D, a.q_dtype);
  const bool all_ok = __syncthreads_and(pids_ok);
  const int full_end = min(p_end, seq_len / TQ_PAGE_TOKENS);
  const int n_full = (all_ok && full_end > p_begin) ? (full_end - p_begin) / 2 : 0;

  // query operands: column c = head hc, contraction rows 8 * g4 .. of each 32-block = coordinates
  // (D / 4) * g4 + 8 * kb + p (the same order as the K rows the lane loads)
  bf16x8_t qop[KBLK], qlo[PK ? 1 : KBLK];
  {
    const bool real = hc < G;
    const int r = real ? hc : 0;
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const float x = real ? s_q[r][(D / 4) * g4 + 8 * kb + p] : 0.f;
        const __bf16 h = (__bf16)x;
        const __bf16 l = (__bf16)(x - (float)h);
        if constexpr (PK) {
          qop[kb][p] = lo_part ? l : h;
        } else {
          qop[kb][p] = h;
          qlo[kb][p] = l;
        }
      }
    }
  }
  const float colscale = hc < G ? a.scale_log2 : 0.f;

  float m_run = -INFINITY, l_part = 0.f;
  floatx4_t O[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) O[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const DFrag<D, F8> &cur, int pi, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int pp = p_begin + 2 * pi;
    float s[2][4];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) {
        const bf16x8_t A = k_operand<D>(cur, q2, kb);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qop[kb], acc, 0, 0, 0);
        if constexpr (!PK) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qlo[kb], acc, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) s[q2][j] = PK ? acc[j] + xor_lane<8>(acc[j]) : acc[j];
    }
    bool okm[2][4];
    if constexpr (!FULL) {
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = (pp + q2) * TQ_PAGE_TOKENS + 4 * g4 + j;
          okm[q2][j] = cur.ok[q2] && t < seq_len;
          s[q2][j] = okm[q2][j] ? s[q2][j] : -3.0e38f;
        }
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = max_xor32(max_xor16(mx));
    const float m_new = colscale * mx;
    if (__any(m_new > m_run)) {
      const bool up = m_new > m_run;
      const float m_ref = up ? m_new + kDHeadroom : m_run;
      const float alpha = up ? ((m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_ref)) : 1.f;
      l_part *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) O[nb] *= alpha;
      m_run = m_ref;
    }
    bf16x8_t phi, plo;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p = fast_exp2(fmaf(s[q2][j], colscale, -m_run));
        if constexpr (!FULL) p = okm[q2][j] ? p : 0.f;
        l_part += p;
        const __bf16 h = (__bf16)p;
        if constexpr (PK) {
          phi[4 * q2 + j] = (__bf16)fmaf(lo_neg, (float)h, p);  // high column: p; low column: p - bf16(p)
          (void)plo;
        } else {
          phi[4 * q2 + j] = h;
          plo[4 * q2 + j] = (__bf16)(p - (float)h);
        }
      }
    }
    // values, transposed: O^T[coords][heads] += V^T[coords][32 tokens] P^T[32 tokens][heads]; contraction
    // row 8 * g4 + p is token 4 * g4 + (p & 3) of page p >> 2, as the score rows of this lane
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8_t A = v_operand<D>(cur, nb);
      O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, phi, O[nb], 0, 0, 0);
      if constexpr (!PK) O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, plo, O[nb], 0, 0, 0);
    }
  };

  for (int i = wave; i < npairs; i += R * kDWaves) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int ii = i + r * kDWaves;
      const int nx = ii + (R - 1) * kDWaves;
      const int pp = p_begin + 2 * nx;
      dense_load_pages<D>(a, kvh, c, g4, pp < p_end ? s_pid[min(pp, p_end - 1) - p_begin] : -1,
                          pp + 1 < p_end ? s_pid[min(pp + 1, p_end - 1) - p_begin] : -1, f[(r + R - 1) % R]);
      if (ii < n_full) process(f[r], ii, std::true_type{});
      else if (ii < npairs) process(f[r], ii, std::false_type{});
    }
  }

  // ---- merge the wavefronts: rescale to the work-group max, then sum over the waves in a fixed order
  if constexpr (PK) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) O[nb][j] += xor_lane<8>(O[nb][j]);
  }
  {
    const float l_tot = sum_xor16_32(l_part);
    if (g4 == 0) {
      s_m[wave][c] = m_run;
      s_l[wave][c] = l_tot;
    }
  }
  __syncthreads();
  if (c < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDWaves; ++w) M = fmaxf(M, s_m[w][c]);
    const float e = (M == -INFINITY || m_run == -INFINITY) ? 0.f : fast_exp2(m_run - M);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      O[nb] *= e;
      *(float4 *)&dep[wave][c][16 * nb + 4 * g4] = float4{O[nb][0], O[nb][1], O[nb][2], O[nb][3]};
    }
  }
  if (tid < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDWaves; ++w) M = fmaxf(M, s_m[w][tid]);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDWaves; ++w)
        if (s_m[w][tid] != -INFINITY) L = fmaf(fast_exp2(s_m[w][tid] - M), s_l[w][tid], L);
    }
    s_rowm[tid] = M;
    s_rowl[tid] = L;
  }
  __syncthreads();
  const int64_t S = a.n_splits;
  for (int idx = tid; idx < G * D; idx += NT) {
    const int row = idx / D, k = idx % D;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kDWaves; ++w) t += dep[w][row][k];
    if constexpr (F8) t *= a.v_scale;
    const int64_t bh = (int64_t)b * a.Hq + head0 + row;
    if (S > 1) {
      a.part_o[(bh * S + split) * D + k] = t;
    } else {
      const float L = s_rowl[row];
      a.out[bh * D + k] = L > 0.f ? t / L : 0.f;
    }
  }
  if (S > 1 && tid < G) {
    const int64_t bh = (int64_t)b * a.Hq + head0 + tid;
    a.part_ml[(bh * S + split) * 2] = s_rowm[tid];
    a.part_ml[(bh * S + split) * 2 + 1] = s_rowl[tid];
  }
}

}  // namespace

int launch_dense_write(int head_dim, int num_kv_heads, const DenseFormat &fmt, void *pages, int64_t num_pages,
                       const void *k, const void *v, int dtype, int64_t n_tok, const int64_t *slots,
                       hipStream_t stream) {
  const uint32_t half = (uint32_t)((fmt.fp8 ? 1 : 2) * num_kv_heads * TQ_PAGE_TOKENS * head_dim);
  const int64_t threads = n_tok * num_kv_heads * (head_dim / 8);
  if (threads == 0) return TQ_OK;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return TQ_EINVAL;
  if (fmt.fp8)
    hipLaunchKernelGGL(dense_write_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (unsigned char *)pages,
                       num_pages * TQ_PAGE_TOKENS, 2 * half, half, head_dim, num_kv_heads, k, v, dtype, n_tok, slots,
                       fmt.k_scale, fmt.v_scale);
  else
    hipLaunchKernelGGL(dense_write_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (unsigned char *)pages,
                       num_pages * TQ_PAGE_TOKENS, 2 * half, half, head_dim, num_kv_heads, k, v, dtype, n_tok, slots);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

template <int D, bool F8>
static void launch_dense_scan(const DenseArgs &a, dim3 grid, hipStream_t stream) {
  if (a.G <= 8) hipLaunchKernelGGL((dense_decode_kernel<D, true, F8>), grid, dim3(64 * kDWaves), 0, stream, a);
  else hipLaunchKernelGGL((dense_decode_kernel<D, false, F8>), grid, dim3(64 * kDWaves), 0, stream, a);
}

int launch_dense_decode(int head_dim, int num_kv_heads, const DenseFormat &fmt, const DecodeWs &ws,
                        const void *pages, int64_t num_pages, const void *q, int q_dtype, int batch,
                        int num_q_heads, const int32_t *page_table, int max_pages_per_seq, const int32_t *seq_lens,
                        float softmax_scale, void *workspace, float *out, int passes, hipStream_t stream) {
  DenseArgs a;
  const uint32_t half = (uint32_t)((fmt.fp8 ? 1 : 2) * num_kv_heads * TQ_PAGE_TOKENS * head_dim);
  a.pages = (const unsigned char *)pages;
  a.num_pages32 = (int)std::min<int64_t>(num_pages, 0x7FFFFFFF);
  a.page_bytes = 2 * half;
  a.v_off = half;
  a.q = q;
  a.q_dtype = q_dtype;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.G = num_q_heads / num_kv_heads;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  if (fmt.fp8) a.scale_log2 *= fmt.k_scale;
  a.v_scale = fmt.v_scale;
  unsigned char *w = (unsigned char *)workspace;
  a.part_o = (float *)(w + ws.part_o_off);
  a.part_ml = (float *)(w + ws.part_ml_off);
  a.n_splits = ws.n_splits;
  a.pps = ws.pages_per_split;
  a.out = out;
  if (passes & kPassScan) {
    const dim3 grid(a.n_splits, num_kv_heads, batch);
    if (head_dim == 128) {
      if (fmt.fp8) launch_dense_scan<128, true>(a, grid, stream);
      else launch_dense_scan<128, false>(a, grid, stream);
    } else {
      if (fmt.fp8) launch_dense_scan<64, true>(a, grid, stream);
      else launch_dense_scan<64, false>(a, grid, stream);
    }
    if (hipGetLastError() != hipSuccess) return TQ_EHIP;
  }
  if ((passes & kPassCombine) && a.n_splits > 1)
    return launch_combine_plain(a.part_o, a.part_ml, a.n_splits, (int64_t)batch * num_q_heads, head_dim, out, stream);
  return TQ_OK;
}

}  // namespace tq
