// Dense random (QR) rotation ("What the Paper Doesn't Tell You", Finding 4: the paper rotates with a dense
// random orthogonal matrix from a QR decomposition - d x d storage, O(d^2) work per vector - where the WHT
// needs one sign vector and O(d log d)): the host factorization that builds the rotation, and the entry
// points that run the compressed path with it.
//
// The quantize and decode kernels apply W = H diag(s) / sqrt(d) (H Sylvester's Hadamard matrix, s the
// codebook's signs). For the dense rotation Q the rows are first rotated by M = W^T Q on the matrix cores;
// the kernels then apply W, and W M = Q, so the codes are those of Q u. For MSE keys and values the rotation
// runs inside the quantize kernel (rows through LDS); a sketched tensor takes a separate rotation pass. The
// queries go through the same M of the keys (scores <W M q, yhat> = <Q q, yhat>), and the decode output -
// returned by the unchanged kernels in the coordinates of M x - is brought back by the transpose of the
// values' M.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "tq_internal.h"

namespace {

size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

bool valid_dtype(int t) { return t == TQ_F32 || t == TQ_BF16 || t == TQ_F16; }

}  // namespace

extern "C" {

int tq_qr_rotation(int head_dim, const double *gauss, const uint32_t *sign_words, float *fwd, float *inv) {
  if ((head_dim != 64 && head_dim != 128) || !gauss || !fwd) return TQ_EINVAL;
  const int d = head_dim;
  // Householder QR of G (row-major), in fp64: A becomes T (upper triangular), Q accumulates the
  // reflectors, G = Q T
  std::vector<double> A(gauss, gauss + (size_t)d * d);
  std::vector<double> Q((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) Q[(size_t)i * d + i] = 1.0;
  std::vector<double> v(d);
  for (int k = 0; k < d; ++k) {
    double nrm = 0.0;
    for (int i = k; i < d; ++i) nrm += A[(size_t)i * d + k] * A[(size_t)i * d + k];
    nrm = std::sqrt(nrm);
    if (!(nrm > 0.0) || !std::isfinite(nrm)) return TQ_EINVAL;  // singular or non-finite draw
    // reflect column k onto alpha e_k, alpha of the opposite sign to the pivot (no cancellation in v)
    const double alpha = A[(size_t)k * d + k] > 0.0 ? -nrm : nrm;
    double vn = 0.0;
    for (int i = k; i < d; ++i) {
      v[i] = A[(size_t)i * d + k] - (i == k ? alpha : 0.0);
      vn += v[i] * v[i];
    }
    if (vn == 0.0) continue;
    for (int j = k; j < d; ++j) {  // A <- (I - 2 v v^T / |v|^2) A
      double t = 0.0;
      for (int i = k; i < d; ++i) t += v[i] * A[(size_t)i * d + j];
      t *= 2.0 / vn;
      for (int i = k; i < d; ++i) A[(size_t)i * d + j] -= t * v[i];
    }
    for (int i = 0; i < d; ++i) {  // Q <- Q (I - 2 v v^T / |v|^2)
      double t = 0.0;
      for (int l = k; l < d; ++l) t += Q[(size_t)i * d + l] * v[l];
      t *= 2.0 / vn;
      for (int l = k; l < d; ++l) Q[(size_t)i * d + l] -= t * v[l];
    }
  }
  // the convention diag(T) > 0 makes the factorization unique: flip column k of Q where T_kk < 0
  for (int k = 0; k < d; ++k)
    if (A[(size_t)k * d + k] < 0.0)
      for (int i = 0; i < d; ++i) Q[(size_t)i * d + k] = -Q[(size_t)i * d + k];
  // M = W^T Q = diag(s) H Q / sqrt(d), with H[i][l] = (-1)^popcount(i & l)
  const double rs = 1.0 / std::sqrt((double)d);
  for (int i = 0; i < d; ++i) {
    const bool neg = sign_words && ((sign_words[i >> 5] >> (i & 31)) & 1u);
    for (int j = 0; j < d; ++j) {
      double t = 0.0;
      for (int l = 0; l < d; ++l) {
        const double q = Q[(size_t)l * d + j];
        t += (__builtin_popcount((unsigned)(i & l)) & 1) ? -q : q;
      }
      const float m = (float)((neg ? -t : t) * rs);
      fwd[(size_t)i * d + j] = m;
      if (inv) inv[(size_t)j * d + i] = m;
    }
  }
  return TQ_OK;
}

int tq_rotate_rows(int head_dim, const float *mat, const void *x, int x_dtype, int64_t rows, float *y, void *stream) {
  if ((head_dim != 64 && head_dim != 128) || !valid_dtype(x_dtype) || rows < 0) return TQ_EINVAL;
  if (rows == 0) return TQ_OK;
  if (!mat || !x || !y) return TQ_EINVAL;
  if (((uintptr_t)mat | (uintptr_t)x | (uintptr_t)y) & 15) return TQ_EINVAL;
  return tq::launch_rotate_rows(head_dim, mat, x, x_dtype, rows, y, (hipStream_t)stream);
}

int tq_quantize_kv_qr_workspace_bytes(const tq_layout *layout, int64_t n_tok, size_t *out) {
  tq::PageGeom g;
  const int st = tq::make_geom(layout, &g);
  if (st) return st;
  if (!out || n_tok < 0) return TQ_EINVAL;
  *out = 2 * align16((size_t)n_tok * layout->num_kv_heads * layout->head_dim * 4);
  return TQ_OK;
}

int tq_quantize_kv_qr(const tq_layout *layout, void *pages, int64_t num_pages, const void *k, const void *v,
                      int dtype, int64_t n_tok, const int64_t *slots, const void *k_cb, const void *v_cb,
                      const float *k_rot, const float *v_rot, void *workspace, size_t workspace_bytes,
                      void *stream) {
  size_t need = 0;
  int st = tq_quantize_kv_qr_workspace_bytes(layout, n_tok, &need);
  if (st) return st;
  if (!valid_dtype(dtype)) return TQ_EINVAL;
  if (n_tok == 0) return TQ_OK;
  if (!pages || !k || !v || !slots || !k_cb || !v_cb || !k_rot || !v_rot || !workspace) return TQ_EINVAL;
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)k_rot | (uintptr_t)v_rot | (uintptr_t)workspace) & 15) return TQ_EINVAL;
  if (workspace_bytes < need) return TQ_ENOSPC;
  const int d = layout->head_dim;
  if (layout->k_mode != TQ_PROD && layout->v_mode != TQ_PROD) {
    // MSE keys and values: the rotation fused into the quantize kernel (same bytes as the two passes below)
    tq::PageGeom g;
    if ((st = tq::make_geom(layout, &g))) return st;
    if (n_tok * layout->num_kv_heads >= ((int64_t)1 << 35)) return TQ_EINVAL;
    return tq::launch_quantize_qr(g, pages, num_pages, k, v, dtype, n_tok, slots, k_cb, v_cb, k_rot, v_rot,
                                  (hipStream_t)stream);
  }
  // a sketched tensor: the rows rotated in their own pass, then tq_quantize_kv over the fp32 rows
  const int64_t rows = n_tok * layout->num_kv_heads;
  float *wk = (float *)workspace;
  float *wv = (float *)((unsigned char *)workspace + need / 2);
  hipStream_t s = (hipStream_t)stream;
  if ((st = tq::launch_rotate_rows(d, k_rot, k, dtype, rows, wk, s))) return st;
  if ((st = tq::launch_rotate_rows(d, v_rot, v, dtype, rows, wv, s))) return st;
  const int64_t stride = (int64_t)layout->num_kv_heads * d;
  return tq_quantize_kv(layout, pages, num_pages, wk, wv, TQ_F32, n_tok, stride, stride, slots, k_cb, v_cb, stream);
}

int tq_decode_qr_workspace_bytes(const tq_layout *layout, int batch, int num_q_heads, int max_pages_per_seq,
                                 int pages_per_split, size_t *out) {
  if (!out) return TQ_EINVAL;
  size_t dec = 0;
  const int st = tq_decode_workspace_bytes(layout, batch, num_q_heads, max_pages_per_seq, pages_per_split, &dec);
  if (st) return st;
  *out = align16(dec) + 2 * align16((size_t)batch * num_q_heads * layout->head_dim * 4);
  return TQ_OK;
}

int tq_decode_attention_qr(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q, int q_dtype,
                           int batch, int num_q_heads, const int32_t *page_table, int max_pages_per_seq,
                           const int32_t *seq_lens, float softmax_scale, int pages_per_split, const void *k_cb,
                           const void *v_cb, const float *k_rot, const float *v_inv, void *workspace,
                           size_t workspace_bytes, float *out, void *stream) {
  size_t need = 0, dec = 0;
  int st = tq_decode_qr_workspace_bytes(layout, batch, num_q_heads, max_pages_per_seq, pages_per_split, &need);
  if (st) return st;
  st = tq_decode_workspace_bytes(layout, batch, num_q_heads, max_pages_per_seq, pages_per_split, &dec);
  if (st) return st;
  if (!valid_dtype(q_dtype) || batch < 0) return TQ_EINVAL;
  if (batch == 0) return TQ_OK;
  if (!q || !k_rot || !v_inv || !workspace || !out) return TQ_EINVAL;
  if (((uintptr_t)q | (uintptr_t)k_rot | (uintptr_t)v_inv | (uintptr_t)workspace | (uintptr_t)out) & 15) return TQ_EINVAL;
  if (workspace_bytes < need) return TQ_ENOSPC;
  const int d = layout->head_dim;
  const int64_t rows = (int64_t)batch * num_q_heads;
  unsigned char *w = (unsigned char *)workspace;
  float *q_in = (float *)(w + align16(dec));
  float *o_in = (float *)(w + align16(dec) + align16((size_t)rows * d * 4));
  hipStream_t s = (hipStream_t)stream;
  if ((st = tq::launch_rotate_rows(d, k_rot, q, q_dtype, rows, q_in, s))) return st;
  st = tq_decode_attention(layout, pages, num_pages, q_in, TQ_F32, batch, num_q_heads, page_table, max_pages_per_seq,
                           seq_lens, softmax_scale, pages_per_split, k_cb, v_cb, workspace, dec, o_in, stream);
  if (st) return st;
  return tq::launch_rotate_rows(d, v_inv, o_in, TQ_F32, rows, out, s);
}

}  // extern "C"
