// Quantize-on-write ("Closing - The Three-Step Summary", Steps 1-3): for every K and V vector,
//   n = ||x||, y' = H (s * x) / n   (the rotated unit vector in N(0,1) units),
//   idx_i = #{j : y'_i >= t_j}      (Gaussian Lloyd-Max thresholds, midpoints of the fp16 levels),
//   code_i = sign-magnitude form of idx_i, pack the b-bit codes, store n as fp16, and in prod mode also
//   r = (y' - level[code]) / sqrt(d), gamma = ||r||, z_j = [(S r)_j >= 0].
// One vector is handled by d/8 lanes that each own 8 consecutive coordinates: the three lowest
// Walsh-Hadamard stages run in registers, the others exchange values between lanes. A lane's 8 codes
// are exactly b whole bytes of the vector's bit stream, so each lane writes its own bytes: that is a
// contiguous run for K records and one V piece.
#include <hip/hip_runtime.h>

#include "tq_common.h"
#include "tq_internal.h"

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
        x[2 * k] = bf16_bits_to_float((uint16_t)(d[k] & 0xFFFF));
        x[2 * k + 1] = bf16_bits_to_float((uint16_t)(d[k] >> 16));
      } else {
        x[2 * k] = half_bits_to_float((uint16_t)(d[k] & 0xFFFF));
        x[2 * k + 1] = half_bits_to_float((uint16_t)(d[k] >> 16));
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  constexpr int LANES = D / 8;
  constexpr int VPB = 256 / LANES;
  const int which = blockIdx.y;  // 0 = K, 1 = V
  const unsigned char *cb = a.cb[which];
  const BlobOffsets bo = a.cbo[which];
  const int b = a.bits[which];
  const int mode = a.mode[which];
  const int nl = 1 << b;

  __shared__ float s_th[256];
  __shared__ float s_lv[256];
  __shared__ float s_r[VPB][D];

  const int lane = threadIdx.x % LANES;
  const int vl = threadIdx.x / LANES;
  const int64_t vid = (int64_t)blockIdx.x * VPB + vl;
  const bool active = vid < a.n_tok * a.H;
  const int64_t tok = active ? vid / a.H : 0;
  const int h = active ? (int)(vid % a.H) : 0;

  // every global read issued before the first wait: slot, the lane's 8 inputs, its 8 sign bits, tables
  const int64_t slot = active ? a.slots[tok] : -1;
  float x[8];
  if (active) load8(a.in[which], tok * a.stride[which] + (int64_t)h * D + 8 * lane, a.dtype, x);
  else
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = 0.f;
  const uint32_t sword = ((const uint32_t *)(cb + bo.signs))[(8 * lane) >> 5];
  for (int i = threadIdx.x; i < nl - 1; i += 256) s_th[i] = ((const float *)(cb + bo.thresholds))[i];
  for (int i = threadIdx.x; i < nl; i += 256) s_lv[i] = half_bits_to_float(((const uint16_t *)(cb + bo.levels))[i]);
  const bool valid = active && slot >= 0 && slot < a.num_slots;
  __syncthreads();

  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss = fmaf(x[k], x[k], ss);
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) ss += __shfl_xor(ss, o, LANES);
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
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float p = __shfl_xor(x[k], o, LANES);
      x[k] = (lane & o) ? (p - x[k]) : (x[k] + p);
    }
  }

  // Lloyd-Max index (ties to the upper cell), then the stored sign-magnitude code: the top bit marks
  // the non-negative half, the low bits count the rank away from zero.
  int idx[8], code[8];
  float y[8];
  const int half = nl >> 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    y[k] = x[k] * inv;
    int c = 0;
    for (int s = nl >> 1; s > 0; s >>= 1)
      if (y[k] >= s_th[c + s - 1]) c += s;
    idx[k] = c;
    code[k] = c >= half ? c : half - 1 - c;
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

  if (mode == TQ_PROD) {
    const float inv_sqrt_d = D == 128 ? 0.088388347648318440f : 0.125f;
    float r[8];
    float g2 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      r[k] = (y[k] - s_lv[idx[k]]) * inv_sqrt_d;
      g2 = fmaf(r[k], r[k], g2);
      s_r[vl][8 * lane + k] = r[k];
    }
#pragma unroll
    for (int o = 1; o < LANES; o <<= 1) g2 += __shfl_xor(g2, o, LANES);
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
  const int64_t nvec = n_tok * g.num_kv_heads;
  if (g.head_dim == 128) {
    dim3 grid((unsigned)((nvec + 15) / 16), 2);
    hipLaunchKernelGGL(quantize_kernel<128>, grid, dim3(256), 0, stream, a);
  } else {
    dim3 grid((unsigned)((nvec + 31) / 32), 2);
    hipLaunchKernelGGL(quantize_kernel<64>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // namespace tq
