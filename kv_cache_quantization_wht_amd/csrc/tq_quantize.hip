// Quantize-on-write ("Closing - The Three-Step Summary", Steps 1-3): for every K and V vector,
//   n = ||x||, y' = H (s * x) / n   (the rotated unit vector in N(0,1) units),
//   idx_i = #{j : y'_i >= t_j}      (Gaussian Lloyd-Max thresholds, midpoints of the fp16 levels),
//   code_i = sign-magnitude form of idx_i, pack the b-bit codes, store n as fp16, and in prod mode also
//   r = (y' - level[code]) / sqrt(d), gamma = ||r||, z_j = [(S r)_j >= 0].
// One vector is handled by d/8 lanes that each own 8 consecutive coordinates: the three lowest
// Walsh-Hadamard stages run in registers, the others exchange values between lanes with DPP moves inside
// 16-lane rows. A lane's 8 codes are exactly b whole bytes of the vector's bit stream, so each lane writes
// its own bytes: a contiguous run for K records and one V piece. The vectors of a work-group are
// consecutive tokens of one head, so the records they write are neighbours in a page.
#include <hip/hip_runtime.h>

#include "tq_common.h"
#include "tq_internal.h"
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
};

constexpr int kQuantVectorsPerLane = 1;

// One vector: norm, signs, rotation, codes, record write (and the prod-mode residual sketch).
template <int D, bool PROD>
__device__ __forceinline__ void quantize_vector(const QuantArgs &a, int which, float *x, int64_t slot, bool active,
                                                int h, int lane, int vl, uint32_t sword, const PosThresholds &P,
                                                const float *s_th, const float *s_lv, float (*s_r)[D]) {
  constexpr int LANES = D / 8;
  const unsigned char *cb = a.cb[which];
  const BlobOffsets bo = a.cbo[which];
  const int b = a.bits[which];
  const int half = (1 << b) >> 1;
  const bool valid = active && slot >= 0 && slot < a.num_slots;

  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss = fmaf(x[k], x[k], ss);
  ss = group_sum<LANES>(ss);
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / n : 0.f;

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

  // Lloyd-Max index (ties to the upper cell) in its stored sign-magnitude form: the top bit marks the
  // non-negative half, the low bits count the rank away from zero. For y < 0 the rank counts thresholds
  // strictly below |y|, i.e. thresholds at or below the next float under |y|.
  int code[8];
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    y[k] = x[k] * inv;
    const bool neg = y[k] < 0.f;
    const int z = (int)(__float_as_uint(y[k]) & 0x7FFFFFFFu) - (neg ? 1 : 0);
    int mag;
    if (b <= 4) {
      switch (b) {
        case 1: mag = magnitude<1>(z, P); break;
        case 2: mag = magnitude<2>(z, P); break;
        case 3: mag = magnitude<3>(z, P); break;
        default: mag = magnitude<4>(z, P); break;
      }
    } else {
      // wide codes: binary search over all thresholds in LDS, then the sign-magnitude form
      int c = 0;
      for (int st = half; st > 0; st >>= 1)
        if (y[k] >= s_th[c + st - 1]) c += st;
      mag = c >= half ? c - half : half - 1 - c;
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

  if constexpr (PROD) {
    const float inv_sqrt_d = D == 128 ? 0.088388347648318440f : 0.125f;
    float r[8];
    float g2 = 0.f;
    __syncthreads();  // the previous vector's residuals have been read
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // ascending index of the stored code
      const int idx = (code[k] & half) ? code[k] : half - 1 - code[k];
      r[k] = (y[k] - s_lv[idx]) * inv_sqrt_d;
      g2 = fmaf(r[k], r[k], g2);
      s_r[vl][8 * lane + k] = r[k];
    }
    g2 = group_sum<LANES>(g2);
    __syncthreads();
    const float *S = (const float *)(cb + bo.proj);
    uint32_t zbits = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float *row = S + (int64_t)(8 * lane + k) * D;
      float acc = 0.f;
      for (int i = 0; i < D; ++i) acc = fmaf(row[i], s_r[vl][i], acc);
      zbits |= (acc >= 0.f ? 1u : 0u) << k;
    }
    if (valid) {
      pg[a.qjl_off[which] + (int64_t)(h * TQ_PAGE_TOKENS + off) * (D / 8) + lane] = (unsigned char)zbits;
      if (lane == 0)
        *(uint16_t *)(pg + a.gamma_off[which] + (int64_t)(h * TQ_PAGE_TOKENS + off) * 2) =
            float_to_half_bits(sqrtf(g2));
    }
  }
}

// A work-group holds NV * VPB consecutive tokens of one head (K or V by blockIdx.y); each lane group
// takes NV of them and issues all their loads before computing any, to keep bytes in flight.
template <int D>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  constexpr int LANES = D / 8;
  constexpr int VPB = 256 / LANES;
  constexpr int NV = kQuantVectorsPerLane;
  const int which = blockIdx.y;  // 0 = K, 1 = V
  const unsigned char *cb = a.cb[which];
  const BlobOffsets bo = a.cbo[which];
  const int b = a.bits[which];
  const int mode = a.mode[which];
  const int nl = 1 << b;
  const int half = nl >> 1;

  __shared__ float s_th[256];
  __shared__ float s_lv[256];
  __shared__ float s_r[VPB][D];

  const int lane = threadIdx.x % LANES;
  const int vl = threadIdx.x / LANES;
  const int h = blockIdx.x % a.H;
  const int64_t tok0 = (int64_t)(blockIdx.x / a.H) * (VPB * NV) + vl;

  const uint32_t sword = ((const uint32_t *)(cb + bo.signs))[(8 * lane) >> 5];
  // positive thresholds (t[half-1] is 0 by symmetry), as integer bit patterns
  PosThresholds P{};
  if (b <= 4) P = pos_thresholds((const_i32)(cb + bo.thresholds), half);
  if (b > 4 || mode == TQ_PROD) {
    for (int i = threadIdx.x; i < nl - 1; i += 256) s_th[i] = ((const float *)(cb + bo.thresholds))[i];
    for (int i = threadIdx.x; i < nl; i += 256) s_lv[i] = half_bits_to_float(((const uint16_t *)(cb + bo.levels))[i]);
    __syncthreads();
  }
  if (mode == TQ_PROD) {
    // the residual sketch reads the same rows of S for every vector: one vector at a time, so that the
    // compiler does not hold those rows across vectors
#pragma unroll 1
    for (int j = 0; j < NV; ++j) {
      const int64_t t = tok0 + (int64_t)j * VPB;
      const int64_t tc = t < a.n_tok ? t : 0;
      float x[8];
      load8(a.in[which], tc * a.stride[which] + (int64_t)h * D + 8 * lane, a.dtype, x);
      quantize_vector<D, true>(a, which, x, a.slots[tc], t < a.n_tok, h, lane, vl, sword, P, s_th, s_lv, s_r);
    }
    return;
  }
  // every input read issued before the first use: slots and the lane's 8 inputs of each vector
  int64_t slot[NV];
  float x[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t t = tok0 + (int64_t)j * VPB;
    const int64_t tc = t < a.n_tok ? t : 0;
    slot[j] = a.slots[tc];
    load8(a.in[which], tc * a.stride[which] + (int64_t)h * D + 8 * lane, a.dtype, x[j]);
  }
#pragma unroll
  for (int j = 0; j < NV; ++j)
    quantize_vector<D, false>(a, which, x[j], slot[j], tok0 + (int64_t)j * VPB < a.n_tok, h, lane, vl, sword, P,
                              s_th, s_lv, s_r);
}

}  // namespace

int launch_quantize(const PageGeom &g, void *pages, int64_t num_pages, const void *k, const void *v,
                    int dtype, int64_t n_tok, int64_t k_stride, int64_t v_stride,
                    const int64_t *slots, const void *k_cb, const void *v_cb, hipStream_t stream) {
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
  // work-groups: (token groups x heads, K/V)
  const int vpb = (g.head_dim == 128 ? 16 : 32) * kQuantVectorsPerLane;
  const int64_t blocks = (n_tok + vpb - 1) / vpb * g.num_kv_heads;
  if (blocks > 0x7FFFFFFF) return TQ_EINVAL;
  dim3 grid((unsigned)blocks, 2);
  if (g.head_dim == 128) hipLaunchKernelGGL(quantize_kernel<128>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(quantize_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // namespace tq
