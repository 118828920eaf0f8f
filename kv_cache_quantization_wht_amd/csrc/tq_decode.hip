// Decode attention over the packed cache ("Where This Fits in the Inference Stack", "TensorRT-LLM: Why
// Integration Is a Kernel Problem": dequantize in registers while the K/V tiles stream in; "Why the KV
// Cache Exists", "The KV Cache Solution": one new query per sequence attends over every cached token).
//
// Three kernels on the caller's stream:
//   prologue  per (batch, query head): q_rot = R q = H (s * q) / sqrt(d), stored scaled by 1/sqrt(d)
//             (the stored levels are in N(0,1) units); for a sketched K also q_s = S q_rot * sqrt(pi/2)/m.
//             A power-of-two range factor per head makes the fp16 hi/lo split below exact to 2^-22.
//   split     one wavefront per (batch, KV head, run of pages). For each pair of 16-token pages:
//               scores  S^T[16 tokens, 16 cols] = Khat[16, d] * Q[d, 16] on MFMA 16x16x32 f16, where the
//                       K operand holds the fp16 levels looked up from the codes and Q holds the G query
//                       heads of this KV head as fp16 hi + lo parts (two MFMAs per 32 coordinates);
//               softmax running max / sum per head (base-2 exponent);
//               values  O[16 rows, d] += P'[rows, 32 tokens] * Vhat[32 tokens, d], P' = p * ||v|| split
//                       into fp16 hi + lo rows, Vhat the fp16 V levels.
//             Writes the run's (max, sum, O) partial. Everything stays in the rotated domain.
//   combine   per (batch, query head): log-sum-exp merge of the partials, then one inverse rotation
//             R_V^T (Walsh-Hadamard butterflies in LDS) and the fp32 output.
#include <hip/hip_runtime.h>

#include "tq_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const unsigned char *pages;
  int64_t num_pages;
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
  float *qrot, *qsk, *qscale, *part_o, *part_ml;
  int n_splits, pps;
  float *out;
};

__device__ __forceinline__ int clamp_len(const DecodeArgs &a, int b) {
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : L;
  int cap = a.max_pages * TQ_PAGE_TOKENS;
  return L > cap ? cap : L;
}

// Largest power of two sigma with max|x| * sigma < 256 (1 if x is all zero).
__device__ __forceinline__ float range_factor(float maxabs) {
  if (!(maxabs > 0.f)) return 1.0f;
  int e;
  frexpf(maxabs, &e);  // maxabs in [2^(e-1), 2^e)
  return ldexpf(1.0f, 8 - e);
}

// ------------------------------------------------------------------------------------------------
// prologue
// ------------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void prologue_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int i = threadIdx.x;
  __shared__ float v[D];
  __shared__ float red[D];
  const tq_codebook_header *hk = (const tq_codebook_header *)a.kcb;
  const uint32_t *sw = (const uint32_t *)(a.kcb + hk->signs_off);
  float x = load_elem(a.q, (int64_t)bh * D + i, a.q_dtype);
  if ((sw[i >> 5] >> (i & 31)) & 1u) x = -x;
  v[i] = x;
  __syncthreads();
  for (int hs = 1; hs < D; hs <<= 1) {
    float u = v[i], w = v[i ^ hs];
    __syncthreads();
    v[i] = (i & hs) ? (w - u) : (u + w);
    __syncthreads();
  }
  const float qr = v[i] * (1.0f / D);  // (R q)_i / sqrt(d)
  a.qrot[(int64_t)bh * D + i] = qr;
  red[i] = fabsf(qr);
  __syncthreads();
  for (int s = D / 2; s > 0; s >>= 1) {
    if (i < s) red[i] = fmaxf(red[i], red[i + s]);
    __syncthreads();
  }
  if (i == 0) a.qscale[(int64_t)bh * 2] = range_factor(red[0]);
  if (hk->mode == TQ_PROD) {
    // q_s = S (R q) * sqrt(pi/2) / m, with (R q)_k = v_k / sqrt(d)
    const float *S = (const float *)(a.kcb + hk->proj_off);
    const float c = 1.2533141373155003f / (float)hk->qjl_rows * (D == 128 ? 0.088388347648318440f : 0.125f);
    float acc = 0.f;
    for (int k = 0; k < D; ++k) acc = fmaf(S[(int64_t)i * D + k], v[k], acc);
    const float qs = acc * c;
    a.qsk[(int64_t)bh * D + i] = qs;
    __syncthreads();
    red[i] = fabsf(qs);
    __syncthreads();
    for (int s = D / 2; s > 0; s >>= 1) {
      if (i < s) red[i] = fmaxf(red[i], red[i + s]);
      __syncthreads();
    }
    if (i == 0) a.qscale[(int64_t)bh * 2 + 1] = range_factor(red[0]);
  }
}

// ------------------------------------------------------------------------------------------------
// split
// ------------------------------------------------------------------------------------------------

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

__device__ __forceinline__ half8_t pack8(const uint16_t *hv) {
  half8_t r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    _Float16 h;
    __builtin_memcpy(&h, &hv[i], 2);
    r[i] = h;
  }
  return r;
}

__device__ __forceinline__ void split_hi_lo(float x, _Float16 &hi, _Float16 &lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

template <int D, int KB, bool KPROD, int VB>
__global__ __launch_bounds__(64) void split_kernel(DecodeArgs a) {
  constexpr int KBLK = D / 32;           // 32-coordinate blocks of the score contraction
  constexpr int NB = D / 16;             // 16-coordinate blocks of the value contraction
  constexpr int KCH = D / 4 * KB / 8;    // bytes of K codes per lane per token (D/4 coordinates)
  constexpr int KREC = D * KB / 8;       // bytes of one K record
  constexpr int VCH = 4 * VB;            // bytes of V codes per lane per page (4 tokens x one piece)
  constexpr int KW = (KCH + 3) / 4 + 1;  // dwords (one spare for bit extraction across a boundary)
  constexpr int VW = VCH / 4 + 1;

  const int lane = threadIdx.x;
  const int c = lane & 15;   // MFMA row/column index inside a 16-block
  const int g4 = lane >> 4;  // which 8-deep slice of the contraction this lane holds
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.G;
  const int head0 = kvh * G;

  __shared__ uint16_t lut_k[1 << KB];
  __shared__ uint16_t lut_v[1 << VB];
  {
    const tq_codebook_header *hk = (const tq_codebook_header *)a.kcb;
    const tq_codebook_header *hv = (const tq_codebook_header *)a.vcb;
    for (int i = lane; i < (1 << KB); i += 64) lut_k[i] = ((const uint16_t *)(a.kcb + hk->levels_off))[i];
    for (int i = lane; i < (1 << VB); i += 64) lut_v[i] = ((const uint16_t *)(a.vcb + hv->levels_off))[i];
  }
  __syncthreads();

  // Query operands: lane holds column c (query head head0 + c) for contraction rows
  // 8*g4 .. 8*g4+7 of each 32-coordinate block, i.e. coordinates cbase + 8*kb + e.
  const int cbase = (D / 4) * g4;
  half8_t qhi[KBLK], qlo[KBLK];
  half8_t shi[KPROD ? KBLK : 1], slo[KPROD ? KBLK : 1];
  float colscale = 0.f, skratio = 0.f;
  {
    const bool real = c < G;
    const int64_t bh = (int64_t)b * a.Hq + head0 + (real ? c : 0);
    const float sig = real ? a.qscale[bh * 2] : 1.f;
    const float sig2 = (KPROD && real) ? a.qscale[bh * 2 + 1] : 1.f;
    colscale = real ? a.scale_log2 / sig : 0.f;
    skratio = sig / sig2;
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int coord = cbase + 8 * kb + e;
        float x = real ? a.qrot[bh * D + coord] * sig : 0.f;
        _Float16 h, l;
        split_hi_lo(x, h, l);
        qhi[kb][e] = h;
        qlo[kb][e] = l;
        if constexpr (KPROD) {
          float y = real ? a.qsk[bh * D + coord] * sig2 : 0.f;
          split_hi_lo(y, h, l);
          shi[kb][e] = h;
          slo[kb][e] = l;
        }
      }
    }
  }

  const int seq_len = clamp_len(a, b);
  const int npages = (seq_len + TQ_PAGE_TOKENS - 1) / TQ_PAGE_TOKENS;
  const int p_begin = split * a.pps;
  const int p_end = min(p_begin + a.pps, npages);

  float m_run = -INFINITY;
  float l_part = 0.f;
  floatx4_t O[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) O[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  for (int pp = p_begin; pp < p_end; pp += 2) {
    float s[2][4], nv[2][4];
    uint32_t vw[2][VW];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int pi = pp + q2;
      int pg = pi < p_end ? a.page_table[(int64_t)b * a.max_pages + pi] : -1;
      const bool pvalid = pg >= 0 && pg < a.num_pages;
      const unsigned char *base = a.pages + (int64_t)(pvalid ? pg : 0) * a.page_bytes;

      // ---- scores for the 16 tokens of this page
      uint32_t kw[KW];
      kw[KW - 1] = 0;
      load_bytes<KCH, (KCH % 16 == 0) ? 16 : ((KCH % 8 == 0) ? 8 : ((KCH % 4 == 0) ? 4 : 2))>(
          base + a.k_codes + (int64_t)(kvh * TQ_PAGE_TOKENS + c) * KREC + g4 * KCH, kw);
      floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) {
        uint16_t hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = lut_k[bits_at<KB>(kw, KB * (8 * kb + e))];
        const half8_t A = pack8(hv);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qhi[kb], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qlo[kb], acc, 0, 0, 0);
      }
      floatx4_t acc2 = {0.f, 0.f, 0.f, 0.f};
      float gam[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (KPROD) {
        // sketch bits of token c for coordinates cbase .. cbase + D/4 - 1
        uint32_t zb;
        const unsigned char *zp = base + a.k_qjl + (int64_t)(kvh * TQ_PAGE_TOKENS + c) * (D / 8) + g4 * (D / 32);
        if constexpr (D == 128) zb = *(const uint32_t *)zp;
        else zb = *(const uint16_t *)zp;
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) {
          uint16_t hv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = ((zb >> (8 * kb + e)) & 1u) ? 0x3C00 : 0xBC00;  // +1 / -1
          const half8_t A = pack8(hv);
          acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, shi[kb], acc2, 0, 0, 0);
          acc2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, slo[kb], acc2, 0, 0, 0);
        }
        const uint2 gw = *(const uint2 *)(base + a.k_gamma + (int64_t)(kvh * TQ_PAGE_TOKENS + 4 * g4) * 2);
        gam[0] = half_bits_to_float(gw.x & 0xFFFF);
        gam[1] = half_bits_to_float(gw.x >> 16);
        gam[2] = half_bits_to_float(gw.y & 0xFFFF);
        gam[3] = half_bits_to_float(gw.y >> 16);
      }
      const uint2 nkw = *(const uint2 *)(base + a.k_norms + (int64_t)(kvh * TQ_PAGE_TOKENS + 4 * g4) * 2);
      const uint2 nvw = *(const uint2 *)(base + a.v_norms + (int64_t)(kvh * TQ_PAGE_TOKENS + 4 * g4) * 2);
      const float nk[4] = {half_bits_to_float(nkw.x & 0xFFFF), half_bits_to_float(nkw.x >> 16),
                           half_bits_to_float(nkw.y & 0xFFFF), half_bits_to_float(nkw.y >> 16)};
      nv[q2][0] = half_bits_to_float(nvw.x & 0xFFFF);
      nv[q2][1] = half_bits_to_float(nvw.x >> 16);
      nv[q2][2] = half_bits_to_float(nvw.y & 0xFFFF);
      nv[q2][3] = half_bits_to_float(nvw.y >> 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = pi * TQ_PAGE_TOKENS + 4 * g4 + j;
        const bool ok = pvalid && t < seq_len && c < G;
        float raw = acc[j];
        if constexpr (KPROD) raw = fmaf(gam[j] * skratio, acc2[j], raw);
        s[q2][j] = ok ? colscale * nk[j] * raw : -INFINITY;
      }

      // ---- V codes: piece holding coordinates (D/16)*c .. +NB-1, slots 4*g4 .. 4*g4+3
      const int piece = (D / 16) * c / 8;
      vw[q2][VW - 1] = 0;
      load_bytes<VCH, 4>(base + a.v_codes + ((int64_t)(kvh * (D / 8) + piece) * TQ_PAGE_TOKENS + 4 * g4) * VB,
                         vw[q2]);
    }

    // ---- online softmax over the 32 tokens (this lane: head column c, tokens 4*g4 .. +3 of each page)
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    if (__any(m_new > m_run)) {
      const float alpha = (m_new > m_run) ? ((m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new)) : 1.f;
      l_part *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float aj = __shfl(alpha, 4 * g4 + j);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nb][j] *= aj;
      }
      m_run = m_new;
    }
    half8_t phi, plo;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = (s[q2][j] == -INFINITY) ? 0.f : exp2f(s[q2][j] - m_run);
        l_part += p;
        const float pv = p > 0.f ? p * nv[q2][j] : 0.f;
        _Float16 h, l;
        split_hi_lo(pv, h, l);
        phi[4 * q2 + j] = h;
        plo[4 * q2 + j] = l;
      }
    }

    // ---- values: O[rows][coords] += P'[rows][32 tokens] * Vhat[32 tokens][coords]
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int ci = (D == 128) ? nb : (4 * (c & 1) + nb);  // code index inside the 8-coordinate piece
      uint16_t hv[8];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int j = 0; j < 4; ++j) hv[4 * q2 + j] = lut_v[bits_at<VB>(vw[q2], 8 * VB * j + VB * ci)];
      const half8_t Bv = pack8(hv);
      O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi, Bv, O[nb], 0, 0, 0);
      O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo, Bv, O[nb], 0, 0, 0);
    }
  }

  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const int64_t S = a.n_splits;
  if (g4 == 0 && c < G) {
    const int64_t bh = (int64_t)b * a.Hq + head0 + c;
    a.part_ml[(bh * S + split) * 2] = m_run;
    a.part_ml[(bh * S + split) * 2 + 1] = l_tot;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 4 * g4 + j;
    if (row < G) {
      const int64_t bh = (int64_t)b * a.Hq + head0 + row;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) a.part_o[(bh * S + split) * D + (D / 16) * c + nb] = O[nb][j];
    }
  }
}

// ------------------------------------------------------------------------------------------------
// combine
// ------------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(DecodeArgs a) {
  const int64_t bh = blockIdx.x;
  const int i = threadIdx.x;
  const int S = a.n_splits;
  __shared__ float v[D];
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_ml[(bh * S + s) * 2]);
  float L = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ms = a.part_ml[(bh * S + s) * 2];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - M);
      L = fmaf(w, a.part_ml[(bh * S + s) * 2 + 1], L);
      acc = fmaf(w, a.part_o[(bh * S + s) * D + i], acc);
    }
  }
  v[i] = L > 0.f ? acc / L : 0.f;
  __syncthreads();
  for (int hs = 1; hs < D; hs <<= 1) {
    float u = v[i], w = v[i ^ hs];
    __syncthreads();
    v[i] = (i & hs) ? (w - u) : (u + w);
    __syncthreads();
  }
  const tq_codebook_header *hv = (const tq_codebook_header *)a.vcb;
  const uint32_t *sw = (const uint32_t *)(a.vcb + hv->signs_off);
  float o = v[i] * (1.0f / D);
  if ((sw[i >> 5] >> (i & 31)) & 1u) o = -o;
  a.out[bh * D + i] = o;
}

template <int D, int KB, bool KPROD, int VB>
void launch_split(const DecodeArgs &a, hipStream_t stream) {
  dim3 grid(a.n_splits, a.Hkv, a.B);
  hipLaunchKernelGGL((split_kernel<D, KB, KPROD, VB>), grid, dim3(64), 0, stream, a);
}

template <int D, int KB, bool KPROD>
bool dispatch_v(int vb, const DecodeArgs &a, hipStream_t s) {
  switch (vb) {
    case 1: launch_split<D, KB, KPROD, 1>(a, s); return true;
    case 2: launch_split<D, KB, KPROD, 2>(a, s); return true;
    case 3: launch_split<D, KB, KPROD, 3>(a, s); return true;
    case 4: launch_split<D, KB, KPROD, 4>(a, s); return true;
    case 8: launch_split<D, KB, KPROD, 8>(a, s); return true;
  }
  return false;
}

template <int D>
bool dispatch_k(int kb, bool kprod, int vb, const DecodeArgs &a, hipStream_t s) {
  if (kprod) {
    switch (kb) {
      case 1: return dispatch_v<D, 1, true>(vb, a, s);
      case 2: return dispatch_v<D, 2, true>(vb, a, s);
      case 3: return dispatch_v<D, 3, true>(vb, a, s);
    }
    return false;
  }
  switch (kb) {
    case 1: return dispatch_v<D, 1, false>(vb, a, s);
    case 2: return dispatch_v<D, 2, false>(vb, a, s);
    case 3: return dispatch_v<D, 3, false>(vb, a, s);
    case 4: return dispatch_v<D, 4, false>(vb, a, s);
    case 8: return dispatch_v<D, 8, false>(vb, a, s);
  }
  return false;
}

}  // namespace

int launch_decode(const PageGeom &g, const DecodeWs &ws, const void *pages, int64_t num_pages,
                  const void *q, int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                  int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                  const void *k_cb, const void *v_cb, void *workspace, float *out,
                  hipStream_t stream) {
  DecodeArgs a;
  a.pages = (const unsigned char *)pages;
  a.num_pages = num_pages;
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
  unsigned char *w = (unsigned char *)workspace;
  a.qrot = (float *)(w + ws.qrot_off);
  a.qsk = (float *)(w + ws.qsk_off);
  a.qscale = (float *)(w + ws.qscale_off);
  a.part_o = (float *)(w + ws.part_o_off);
  a.part_ml = (float *)(w + ws.part_ml_off);
  a.n_splits = ws.n_splits;
  a.pps = ws.pages_per_split;
  a.out = out;
  const int bhq = batch * num_q_heads;
  const bool kprod = g.k_mode == TQ_PROD;
  bool ok;
  if (g.head_dim == 128) {
    hipLaunchKernelGGL(prologue_kernel<128>, dim3(bhq), dim3(128), 0, stream, a);
    ok = dispatch_k<128>(g.k_mse_bits, kprod, g.v_mse_bits, a, stream);
    if (ok) hipLaunchKernelGGL(combine_kernel<128>, dim3(bhq), dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL(prologue_kernel<64>, dim3(bhq), dim3(64), 0, stream, a);
    ok = dispatch_k<64>(g.k_mse_bits, kprod, g.v_mse_bits, a, stream);
    if (ok) hipLaunchKernelGGL(combine_kernel<64>, dim3(bhq), dim3(64), 0, stream, a);
  }
  if (!ok) return TQ_ENOTSUP;
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // namespace tq
