// Internal declarations shared by the library's translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

// Byte offsets of the sections of a codebook blob; a pure function of (head_dim, bits, mode), so kernels
// take them as arguments instead of reading the blob header first.
struct BlobOffsets {
  uint32_t levels, thresholds, signs, proj;
  int qjl_rows;
};
BlobOffsets blob_offsets(int head_dim, int bits, int mode);

// Everything a kernel needs to address one layer's page pool.
struct PageGeom {
  int64_t page_bytes;
  int64_t k_codes, k_norms, k_qjl, k_gamma;
  int64_t v_codes, v_norms, v_qjl, v_gamma;
  int head_dim, num_kv_heads;
  int k_mse_bits, k_mode, v_mse_bits, v_mode;
  BlobOffsets kcb, vcb;
};


// Fills `g` from a validated layout; returns TQ_OK or TQ_EINVAL.
int make_geom(const tq_layout *L, PageGeom *g);

// Workspace carve-up of tq_decode_attention (split partials, used when a sequence is cut into runs).
struct DecodeWs {
  int n_splits;
  int pages_per_split;
  size_t part_o_off;    // float [B][Hq][n_splits][d]   un-normalised rotated value sums
  size_t part_ml_off;   // float [B][Hq][n_splits][2]   (running max in log2 units, sum of weights)
  size_t total;
};

// Limits of one decode launch: page ids of one run held in LDS, runs merged by one combine work-group.
constexpr int kDecodePidCap = 4096;
constexpr int kDecodeMaxSplits = 2048;

int plan_decode(const PageGeom &g, int batch, int num_q_heads, int max_pages_per_seq,
                int pages_per_split, DecodeWs *ws);

// Plain streaming read of `bytes` (a multiple of 16) bytes at `buf` by `blocks` work-groups.
int launch_stream_read(const void *buf, int64_t bytes, int blocks, uint32_t *sink, hipStream_t stream);

// The allocation-free decode entry point keeps its split partials in one fixed device array of this many
// bytes (per device, for the life of the process); decode_scratch gives its address on the current device.
constexpr size_t kDecodeScratchBytes = TQ_DECODE_NOALLOC_MAX_BYTES;
int decode_scratch(void **ptr);

int launch_quantize(const PageGeom &g, void *pages, int64_t num_pages, const void *k, const void *v,
                    int dtype, int64_t n_tok, int64_t k_stride, int64_t v_stride,
                    const int64_t *slots, const void *k_cb, const void *v_cb, hipStream_t stream);

// Passes of one decode launch: the split-K scan, the merge of the runs, or both in order.
constexpr int kPassScan = 1;
constexpr int kPassCombine = 2;

int launch_decode(const PageGeom &g, const DecodeWs &ws, const void *pages, int64_t num_pages,
                  const void *q, int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                  int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                  const void *k_cb, const void *v_cb, void *workspace, float *out,
                  int passes, const void *k_new, const void *v_new, int kv_dtype, hipStream_t stream);

// Merge of split partials into fp32 rows with no inverse rotation (the uncompressed comparator): rows =
// batch * query heads, partials laid out as in DecodeWs.
int launch_combine_plain(const float *part_o, const float *part_ml, int n_splits, int64_t rows, int head_dim,
                         float *out, hipStream_t stream);

// Uncompressed comparators: pages of K [head][16][d] then V [head][d][16] (each head's V block of a page
// transposed), one element = bf16 (page bytes = 4 * num_kv_heads * 16 * head_dim) or, with `fp8`, one
// E4M3 byte standing for scale * its value (page bytes = 2 * num_kv_heads * 16 * head_dim).
struct DenseFormat {
  bool fp8;
  float k_scale, v_scale;  // 1 for bf16
};
int launch_dense_write(int head_dim, int num_kv_heads, const DenseFormat &fmt, void *pages, int64_t num_pages,
                       const void *k, const void *v, int dtype, int64_t n_tok, const int64_t *slots,
                       hipStream_t stream);
int launch_dense_decode(int head_dim, int num_kv_heads, const DenseFormat &fmt, const DecodeWs &ws,
                        const void *pages, int64_t num_pages, const void *q, int q_dtype, int batch,
                        int num_q_heads, const int32_t *page_table, int max_pages_per_seq, const int32_t *seq_lens,
                        float softmax_scale, void *workspace, float *out, int passes, hipStream_t stream);

// Quantize with the dense rotation fused ahead of the MSE steps (K and V in MSE mode; TQ_ENOTSUP otherwise):
// k, v contiguous [n_tok][num_kv_heads][head_dim]; k_rot, v_rot the fp32 matrices M (row-major).
int launch_quantize_qr(const PageGeom &g, void *pages, int64_t num_pages, const void *k, const void *v, int dtype,
                       int64_t n_tok, const int64_t *slots, const void *k_cb, const void *v_cb, const float *k_rot,
                       const float *v_rot, hipStream_t stream);

// Rows of x (rows x head_dim, dtype TQ_F32 / TQ_BF16 / TQ_F16, contiguous) times a dense row-major
// head_dim x head_dim fp32 matrix: y[r] = mat x[r], fp32 (matrix cores, three fp16 hi/lo products).
int launch_rotate_rows(int head_dim, const float *mat, const void *x, int x_dtype, int64_t rows, float *y,
                       hipStream_t stream);

// Causal attention of a chunk of chunk_len new tokens per sequence over the packed cache (K and V in MSE
// mode; TQ_ENOTSUP otherwise): q [batch][chunk_len][num_q_heads][head_dim], out fp32 of the same shape.
int launch_prefill(const PageGeom &g, const void *pages, int64_t num_pages, const void *q, int q_dtype, int batch,
                   int chunk_len, int num_q_heads, const int32_t *page_table, int max_pages_per_seq,
                   const int32_t *prefix_lens, float softmax_scale, const void *k_cb, const void *v_cb, float *out,
                   hipStream_t stream);

}  // namespace tq
