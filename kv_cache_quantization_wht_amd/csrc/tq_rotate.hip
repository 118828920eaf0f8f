// Rotation of rows by a dense d x d matrix on the matrix cores: y[r] = A x[r] for every row r, fp32 out
// ("What the Paper Doesn't Tell You", Finding 4: the paper's own rotation is a dense random orthogonal
// matrix, d x d storage and O(d^2) work per vector, against the WHT's sign vector and O(d log d)).
//
// y^T = A x^T is a genuine dense contraction, so it runs on v_mfma_f32_16x16x32_f16: the matrix blocks are
// the A operand (held in registers for the whole launch), 16 rows of x are the B operand. fp32 accuracy
// comes from splitting both into fp16 high and low parts and accumulating hi.hi + hi.lo + lo.hi in fp32
// (the dropped lo.lo term is below 2^-22 of each product). Before the split the matrix is scaled by 16 and
// each row of x by a power of two that brings its largest magnitude to [2^13, 2^14), so that the low parts
// stay normal fp16 numbers; the scales come off exactly at the end.
//
// Work split: a work-group of 4 wavefronts takes 16 rows at a time; wavefront w computes the output
// coordinates of the 16-row blocks w, w + 4, ... (two blocks at d = 128, one at d = 64), so every wavefront
// loads the same 16 rows (cache hits after the first) and holds only its share of the matrix.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_common.h"
#include "tq_internal.h"
#include "tq_lanes.h"
#include "tq_quant_common.h"

namespace tq {
namespace {

constexpr int kRotWaves = 4;
constexpr float kMatScale = 16.f;

__device__ __forceinline__ void split_fp16(float s, _Float16 &h, _Float16 &l) {
  h = (_Float16)s;
  l = (_Float16)(s - (float)h);
}

template <int D>
__global__ __launch_bounds__(64 * kRotWaves) void rotate_rows_kernel(const float *mat, const void *x, int x_dtype,
                                                                     int64_t rows, float *y) {
  constexpr int JB = D / 32;              // 32-wide blocks of the contraction
  constexpr int IB = D / 16 / kRotWaves;  // 16-row output blocks of one wavefront
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15, g4 = lane >> 4;

  // this wavefront's matrix operands: row 16 * (wave + 4 * ib) + c, columns 32 * jb + 8 * g4 .. + 7
  half8_t ahi[IB][JB], alo[IB][JB];
#pragma unroll
  for (int ib = 0; ib < IB; ++ib)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const float *src = mat + (16 * (wave + kRotWaves * ib) + c) * D + 32 * jb + 8 * g4;
      const float4 u0 = *(const float4 *)src;
      const float4 u1 = *(const float4 *)(src + 4);
      const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        _Float16 h, l;
        split_fp16(v[p] * kMatScale, h, l);
        ahi[ib][jb][p] = h;
        alo[ib][jb][p] = l;
      }
    }

  for (int64_t r0 = (int64_t)blockIdx.x * 16; r0 < rows; r0 += (int64_t)gridDim.x * 16) {
    const int64_t r = r0 + c;
    const bool live = r < rows;
    float xv[JB][8];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      if (live) {
        load8(x, r * D + 32 * jb + 8 * g4, x_dtype, xv[jb]);
      } else {
#pragma unroll
        for (int p = 0; p < 8; ++p) xv[jb][p] = 0.f;
      }
    }
    // the row's largest magnitude (its 4 lanes: c, c + 16, c + 32, c + 48) sets its power-of-two scale
    float mx = 0.f;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int p = 0; p < 8; ++p) mx = fmaxf(mx, fabsf(xv[jb][p]));
    mx = max_xor32(max_xor16(mx));
    int e = 0;
    (void)frexpf(mx, &e);
    const float sc = mx > 0.f ? ldexpf(1.f, 14 - e) : 1.f;
    const float back = 1.f / (kMatScale * sc);  // a power of two: exact
    half8_t xhi[JB], xlo[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        _Float16 h, l;
        split_fp16(xv[jb][p] * sc, h, l);
        xhi[jb][p] = h;
        xlo[jb][p] = l;
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
      // lane (c, g4) holds output coordinates 16 * block + 4 * g4 + j of row r0 + c
      if (live)
        *(float4 *)(y + r * D + 16 * (wave + kRotWaves * ib) + 4 * g4) =
            float4{acc[0] * back, acc[1] * back, acc[2] * back, acc[3] * back};
    }
  }
}

}  // namespace

int launch_rotate_rows(int head_dim, const float *mat, const void *x, int x_dtype, int64_t rows, float *y,
                       hipStream_t stream) {
  if (rows <= 0) return TQ_OK;
  const int64_t tiles = (rows + 15) / 16;
  const unsigned grid = (unsigned)std::min<int64_t>(tiles, 1024);
  if (head_dim == 128)
    hipLaunchKernelGGL(rotate_rows_kernel<128>, dim3(grid), dim3(64 * kRotWaves), 0, stream, mat, x, x_dtype, rows, y);
  else
    hipLaunchKernelGGL(rotate_rows_kernel<64>, dim3(grid), dim3(64 * kRotWaves), 0, stream, mat, x, x_dtype, rows, y);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // namespace tq
