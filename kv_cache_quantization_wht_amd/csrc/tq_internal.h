// Internal declarations shared by the library's translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

// Everything a kernel needs to address one layer's page pool.
struct PageGeom {
  int64_t page_bytes;
  int64_t k_codes, k_norms, k_qjl, k_gamma;
  int64_t v_codes, v_norms, v_qjl, v_gamma;
  int head_dim, num_kv_heads;
  int k_mse_bits, k_mode, v_mse_bits, v_mode;
};

// Fills `g` from a validated layout; returns TQ_OK or TQ_EINVAL.
int make_geom(const tq_layout *L, PageGeom *g);

// Workspace carve-up of tq_decode_attention.
struct DecodeWs {
  int n_splits;
  int pages_per_split;
  size_t qrot_off;     // float [B][Hq][d]   rotated, 1/sqrt(d)-scaled query
  size_t qsk_off;      // float [B][Hq][d]   sketch-domain query (prod K only)
  size_t qscale_off;   // float [B][Hq][2]   power-of-two range factors for the fp16 split
  size_t part_o_off;   // float [B][Hq][n_splits][d]
  size_t part_ml_off;  // float [B][Hq][n_splits][2]
  size_t total;
};

int plan_decode(const PageGeom &g, int batch, int num_q_heads, int max_pages_per_seq,
                int pages_per_split, DecodeWs *ws);

int launch_quantize(const PageGeom &g, void *pages, int64_t num_pages, const void *k, const void *v,
                    int dtype, int64_t n_tok, int64_t k_stride, int64_t v_stride,
                    const int64_t *slots, const void *k_cb, const void *v_cb, hipStream_t stream);

int launch_decode(const PageGeom &g, const DecodeWs &ws, const void *pages, int64_t num_pages,
                  const void *q, int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                  int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                  const void *k_cb, const void *v_cb, void *workspace, float *out,
                  hipStream_t stream);

}  // namespace tq
