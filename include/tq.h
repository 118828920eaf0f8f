/*
 * tq.h - C ABI of the TurboQuant KV-cache library for MI355X (gfx950).
 *
 * The library does three things, each named after the step of the method it runs:
 *   tq_build_codebook   builds the per-layer, per-tensor codebook blob: Gaussian Lloyd-Max levels
 *                       and thresholds, the rotation's random sign vector and (prod mode) the QJL
 *                       projection ("Closing - The Three-Step Summary", Step 2 and "The One-Slide
 *                       Version"; "Why the KV Cache Exists", "Prefix Caching": the rotation is
 *                       fixed per model load).
 *   tq_quantize_kv      quantize-on-write of K and V vectors into 16-token pages: norm, random
 *                       signs, Walsh-Hadamard transform, Lloyd-Max index, bit packing, and for
 *                       prod mode the 1-bit QJL sketch of the residual ("Closing - The Three-Step
 *                       Summary", Steps 1-3; "Where This Fits in the Inference Stack", "Production
 *                       Deployment: Tensor Parallelism": quantize on the owning GPU before the
 *                       write to HBM).
 *   tq_decode_attention GQA decode attention that reads the packed pages and dequantizes inside
 *                       the kernel ("Where This Fits in the Inference Stack", "TensorRT-LLM: Why
 *                       Integration Is a Kernel Problem"), with scores and value sums formed in the
 *                       rotated domain and one inverse rotation per output ("Closing - The
 *                       Three-Step Summary", Step 1: the rotation keeps inner products).
 *   tq_decode_step, tq_decode_step_partial
 *                       one decode step: append the new token of each sequence (quantized by the
 *                       work-group that owns its page) and decode attention over the cache; and its
 *                       first pass alone.
 *   tq_decode_partial, tq_decode_combine
 *                       the two passes of tq_decode_attention, callable one by one: the split-K
 *                       scan over the pages, then the merge of the runs and the inverse rotation.
 *   tq_qr_rotation, tq_rotate_rows, tq_quantize_kv_qr, tq_decode_attention_qr
 *                       the dense random (QR) rotation in place of the WHT: the same codes and
 *                       attention with a d x d orthogonal matrix, for the comparison of the two.
 *   tq_prefill_attention, tq_prefill_chunk
 *                       chunked prefill: a chunk of new tokens attends causally to the packed cache
 *                       (its own keys and values written there first), on the matrix cores.
 *   tq_dense_*          the uncompressed comparators: the same paged decode attention over a bf16
 *                       cache and (tq_dense_fp8_*) over an FP8 E4M3 cache with per-tensor scales, to
 *                       measure the compressed path against the bytes it saves.
 *
 * Conventions for every call:
 *   - Returns TQ_OK (0) or a negative TQ_E* status; never aborts, never allocates device memory.
 *   - Argument checks happen on the host, synchronously, before anything is launched; a failed
 *     check launches nothing and leaves every buffer untouched.
 *   - "device" pointers are caller-owned GPU memory (for instance PyTorch tensors); "host"
 *     pointers are caller-owned CPU memory. The library keeps no pointer after a call returns.
 *   - Kernels run asynchronously on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream). A launch error reported by the HIP runtime returns TQ_EHIP.
 *   - The library holds no global state; calls on different streams may run concurrently as long
 *     as they do not write the same bytes.
 *   - NaN or infinite inputs give unspecified (but in-bounds) results.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------------- */
#define TQ_OK 0
#define TQ_EINVAL (-1)   /* null pointer, unsupported shape, bit width or mode, bad blob */
#define TQ_ENOSPC (-2)   /* a caller buffer is smaller than required */
#define TQ_ENOTSUP (-3)  /* a valid combination this library does not implement */
#define TQ_EHIP (-4)     /* the HIP runtime reported an error */

/* ---- modes and dtypes ------------------------------------------------------------------ */
#define TQ_MSE 0   /* b-bit Lloyd-Max index ("b >= 3: rotate, quantize with b bits") */
#define TQ_PROD 1  /* (b-1)-bit Lloyd-Max index + 1-bit QJL residual sketch ("b <= 2") */

#define TQ_F32 0
#define TQ_BF16 1
#define TQ_F16 2

#define TQ_PAGE_TOKENS 16
#define TQ_CODEBOOK_MAGIC 0x42435154u /* "TQCB" little-endian */
#define TQ_CODEBOOK_VERSION 1u

/* One layer's cache layout. head_dim is 64 or 128; bits is 1, 2, 3, 4 or 8 in MSE mode and
 * 2, 3 or 4 in prod mode; page_tokens must be 16. */
typedef struct tq_layout {
  int32_t head_dim;
  int32_t num_kv_heads;
  int32_t page_tokens;
  int32_t k_bits;
  int32_t k_mode;
  int32_t v_bits;
  int32_t v_mode;
} tq_layout;

/* Byte offsets of the sub-arrays inside one page, and the page size. A page holds 16 token slots
 * of every KV head of one layer; every sub-array starts on a 16-byte boundary:
 *   k_codes [head][slot][head_dim*bK/8]   natural little-endian bit stream, code i at bits b*i..
 *   k_norms [head][slot] fp16             vector norm
 *   k_qjl   [head][slot][head_dim/8]      sketch bit j = [(S r)_j >= 0]          (prod mode)
 *   k_gamma [head][slot] fp16             residual norm                          (prod mode)
 *   v_codes [head][head_dim/8][slot][bV]  the bit stream cut into pieces of bV bytes
 *                                         (8 coordinates each), piece-major
 *   v_norms, v_qjl, v_gamma               as for K (the V code pieces are the only difference)
 * bK, bV are the Lloyd-Max index widths (bits, or bits-1 in prod mode). Offsets of absent
 * sub-arrays are 0. Token t of sequence b is stored at global slot
 * page_table[b][t/16]*16 + t%16, i.e. page slot/16, offset slot%16. */
typedef struct tq_page_offsets {
  uint64_t k_codes, k_norms, k_qjl, k_gamma;
  uint64_t v_codes, v_norms, v_qjl, v_gamma;
  uint64_t page_bytes;
} tq_page_offsets;

/* Codebook blob header (little-endian). The blob is `total_bytes` long and holds, at the given
 * byte offsets from its start:
 *   levels      n_levels fp16: the Lloyd-Max levels for N(0,1) with 2^mse_bits levels, rounded
 *               to fp16, ascending (the 1/sqrt(head_dim) scale is applied in arithmetic)
 *   thresholds  n_levels-1 fp32: exact midpoints of consecutive stored levels
 *   signs       head_dim/32 uint32: bit i of word i/32 set = coordinate i negated before the
 *               Walsh-Hadamard transform
 *   proj        qjl_rows*head_dim fp32, row-major: the QJL projection S (prod mode only)
 * The host builds it once per model load; the caller copies it to device memory and passes the
 * device copy to tq_quantize_kv / tq_decode_attention. */
typedef struct tq_codebook_header {
  uint32_t magic;
  uint32_t version;
  int32_t head_dim;
  int32_t bits;
  int32_t mode;
  int32_t mse_bits;
  int32_t n_levels;
  int32_t qjl_rows;
  uint32_t levels_off;
  uint32_t thresholds_off;
  uint32_t signs_off;
  uint32_t proj_off;
  uint32_t total_bytes;
  uint32_t reserved[3];
} tq_codebook_header;

/* Human-readable text of a status code (static storage). */
const char *tq_strerror(int status);

/* Size in bytes of the codebook blob for (head_dim, bits, mode). Host only.
 * Errors: TQ_EINVAL for a null `out` or an unsupported combination. */
int tq_codebook_bytes(int head_dim, int bits, int mode, size_t *out);

/* Build a codebook blob in caller-owned host memory `blob` of `blob_bytes` bytes. Host only,
 * synchronous, deterministic. The Lloyd-Max levels are solved in fp64 (Gaussian centroid and
 * midpoint conditions, "Closing - The Three-Step Summary", Step 2).
 *   sign_words  host, head_dim/32 uint32: the rotation's random signs (drawn by the caller once per
 *               model load, "Why the KV Cache Exists", "Prefix Caching")
 *   qjl_proj    host, head_dim*head_dim fp32 row-major iid N(0,1) projection S; required in prod
 *               mode, ignored (may be NULL) in MSE mode ("Closing - The Three-Step Summary",
 *               Step 3: the 1-bit QJL sketch)
 * Errors: TQ_EINVAL (null pointers, unsupported combination), TQ_ENOSPC (blob too small). */
int tq_build_codebook(int head_dim, int bits, int mode, const uint32_t *sign_words,
                      const float *qjl_proj, void *blob, size_t blob_bytes);

/* tq_build_codebook with the random objects drawn by the library from one 64-bit seed ("Why the KV Cache Exists",
 * "Prefix Caching": the rotation is fixed per model load; "What the Paper Doesn't Tell You", Finding 4: the WHT
 * rotation is one random sign vector, 16 bytes at head_dim 128). Use one seed per layer (the same for its K and V
 * blobs, so that they share a rotation). Host only, synchronous, deterministic.
 *   signs  bit i of the sign vector is bit i % 64 of output i / 64 of SplitMix64 (Steele, Lea, Flood 2014)
 *          started from state seed ^ 0x5349474E ("SIGN"); set = coordinate negated
 *   S      (prod mode) head_dim x head_dim, row-major: outputs 2k, 2k + 1 of SplitMix64 from seed ^ 0x514A4C53
 *          ("QJLS") give u = ((x >> 11) + 0.5) * 2^-53, and the Box-Muller pair sqrt(-2 ln u1) * (cos, sin)(2 pi u2)
 *          fills entries 2k, 2k + 1 (fp64, rounded to fp32)
 * The blob equals tq_build_codebook's for those signs and S.
 * Errors: those of tq_build_codebook. */
int tq_build_codebook_seeded(int head_dim, int bits, int mode, uint64_t seed, void *blob, size_t blob_bytes);

/* Page layout of one layer. Host only. Errors: TQ_EINVAL for an invalid layout or null pointer. */
int tq_page_layout(const tq_layout *layout, tq_page_offsets *out);

/* Quantize n_tok tokens of K and V into the page pool ("Closing - The Three-Step Summary",
 * Steps 1-3; "Where This Fits in the Inference Stack", tensor-parallel section: per-vector
 * state only, nothing crosses a vector boundary).
 *   pages       device, num_pages * page_bytes bytes: the layer's page pool (written)
 *   k, v        device, element (t, h, i) at [t*k_stride_tok + h*head_dim + i] of dtype `dtype`
 *               (TQ_F32, TQ_BF16 or TQ_F16); 16-byte aligned, token strides a multiple of 8
 *   slots       device int64 [n_tok]: global slot of each token; a slot < 0 or >= num_pages*16 is
 *               skipped. Two tokens of one call must not share a slot.
 *   k_cb, v_cb  device copies of blobs built for (head_dim, k_bits, k_mode) and (head_dim, v_bits,
 *               v_mode)
 * Each vector's record (codes, norm, and in prod mode sketch and residual norm) is written in full;
 * no other byte of the pool is touched. n_tok = 0 launches nothing; n_tok * num_kv_heads must stay
 * below 2^35 (one launch).
 * Errors: TQ_EINVAL (layout, dtype, strides, null pointers), TQ_ENOTSUP, TQ_EHIP. */
int tq_quantize_kv(const tq_layout *layout, void *pages, int64_t num_pages, const void *k,
                   const void *v, int dtype, int64_t n_tok, int64_t k_stride_tok,
                   int64_t v_stride_tok, const int64_t *slots, const void *k_cb, const void *v_cb,
                   void *stream);

/* Workspace bytes needed by tq_decode_attention for these arguments (same `pages_per_split`
 * rule; 0 = automatic choice for the current device). Host only. */
int tq_decode_workspace_bytes(const tq_layout *layout, int batch, int num_q_heads,
                              int max_pages_per_seq, int pages_per_split, size_t *out);

/* Decode attention for one new query per sequence over the packed cache ("Why the KV Cache
 * Exists", "The KV Cache Solution": each step reads every cached K/V of the sequence).
 *   q           device [batch][num_q_heads][head_dim] of q_dtype
 *   page_table  device int32 [batch][max_pages_per_seq]: physical page of each 16-token block
 *   seq_lens    device int32 [batch]: cached tokens per sequence (clamped to
 *               max_pages_per_seq*16); 0 gives a zero output row. Page-table entries < 0 or
 *               >= num_pages inside a sequence are treated as empty pages.
 *   softmax_scale    >= 0 (usually 1/sqrt(head_dim))
 *   pages_per_split  pages of one run, handled by one work-group before the runs are merged
 *               (rounded up to even, at most 2048; 0 = automatic). A sequence's runs start every
 *               pages_per_split pages and its last run also takes the remainder (fewer than
 *               pages_per_split more pages). The result does not depend on it beyond fp32 rounding.
 *   workspace   device scratch of at least tq_decode_workspace_bytes(...) bytes (no initial
 *               contents needed). Calls that share a workspace must not overlap in time.
 *   out         device fp32 [batch][num_q_heads][head_dim]
 * Query head h reads KV head h / (num_q_heads / num_kv_heads) (grouped-query attention, "Why the
 * KV Cache Exists", "What's in the KV Cache"); out = sum_t softmax_t(softmax_scale * q.khat_t)
 * vhat_t over the sequence's tokens, with khat, vhat the dequantized vectors.
 * Errors: TQ_EINVAL, TQ_ENOSPC (workspace), TQ_ENOTSUP, TQ_EHIP. */
int tq_decode_attention(const tq_layout *layout, const void *pages, int64_t num_pages,
                        const void *q, int q_dtype, int batch, int num_q_heads,
                        const int32_t *page_table, int max_pages_per_seq, const int32_t *seq_lens,
                        float softmax_scale, int pages_per_split, const void *k_cb,
                        const void *v_cb, void *workspace, size_t workspace_bytes, float *out,
                        void *stream);

/* A plain streaming read of `bytes` bytes of device memory at `buf` (16-byte aligned, a multiple of 16) by
 * `blocks` work-groups of 512 threads, each lane four 16-byte loads in flight with a grid stride: the practical
 * HBM ceiling the decode kernels are measured against ("Where This Fits in the Inference Stack", "What Changes
 * When KV Cache Is 4x Smaller": decode reads the whole cache from HBM, so its bound is the streaming rate).
 * `sink`: device uint32, written only for one data value that keeps the loads live (contents unspecified).
 * Asynchronous on `stream`. Errors: TQ_EINVAL (null, misaligned or empty buffer, blocks outside
 * 1 .. 2^20), TQ_EHIP. */
int tq_stream_read(const void *buf, size_t bytes, int blocks, uint32_t *sink, void *stream);

/* Largest split-partial buffer tq_decode_attention_noalloc can use: the bytes of the fixed device array it keeps
 * them in (compare with tq_decode_workspace_bytes for the same arguments). */
#define TQ_DECODE_NOALLOC_MAX_BYTES ((size_t)4 << 20)

/* tq_decode_attention for callers that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Same arguments, layout, result and errors as
 * tq_decode_attention without `workspace` / `workspace_bytes`; the split partials live in a fixed device array
 * of TQ_DECODE_NOALLOC_MAX_BYTES bytes that the library's code object holds on each device it runs on until the
 * process ends. Allocates nothing: no hipMalloc, no hipFree, no allocating library call. The array's address on
 * the current device is looked up on the first call on that device (thread-safe).
 * Every call on one device shares that device's array and leaves the last call's partials in it (no initial
 * contents are needed): calls that overlap in time on one device (two streams, two threads) race and must be
 * ordered by the caller.
 * Errors: those of tq_decode_attention; TQ_ENOSPC when the plan's partials (tq_decode_workspace_bytes for the
 * same arguments) exceed TQ_DECODE_NOALLOC_MAX_BYTES - a larger pages_per_split needs fewer;
 * TQ_ENOTSUP on a device index >= 64. */
int tq_decode_attention_noalloc(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q,
                                int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                                int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                                int pages_per_split, const void *k_cb, const void *v_cb, float *out, void *stream);

/* One decode step ("Where This Fits in the Inference Stack", "Production Deployment: Tensor Parallelism":
 * quantize the new K/V before it reaches HBM; "Why the KV Cache Exists", "The KV Cache Solution": the new
 * query attends over every cached token including its own): appends the new token of each sequence and
 * runs decode attention, with the same page bytes and output as tq_quantize_kv of the new tokens into
 * their slots followed by tq_decode_attention.
 *   pages       device page pool (written: the new token's records)
 *   k_new, v_new device [batch][num_kv_heads][head_dim] of kv_dtype (TQ_F32, TQ_BF16 or TQ_F16), 16-byte
 *               aligned: K and V of the new token of each sequence
 *   seq_lens    device int32 [batch], counting the new token: sequence b's new token is position
 *               seq_lens[b] - 1, written to slot page_table[b][(seq_lens[b]-1)/16]*16 + (seq_lens[b]-1)%16
 *               (skipped, and not attended, if that page id is outside [0, num_pages)); 0 appends
 *               nothing and gives a zero row
 * All other arguments as for tq_decode_attention. The work-group that owns the new token's page
 * quantizes it and scores it from its codes, so the step is one split-K launch plus the merge.
 * Errors: as tq_decode_attention; TQ_ENOTSUP unless K and V use MSE codes of at most 4 bits. */
int tq_decode_step(const tq_layout *layout, void *pages, int64_t num_pages, const void *k_new,
                   const void *v_new, int kv_dtype, const void *q, int q_dtype, int batch, int num_q_heads,
                   const int32_t *page_table, int max_pages_per_seq, const int32_t *seq_lens,
                   float softmax_scale, int pages_per_split, const void *k_cb, const void *v_cb,
                   void *workspace, size_t workspace_bytes, float *out, void *stream);

/* The first pass of tq_decode_step (append + split-K scan); tq_decode_combine with the same arguments
 * (its own argument list) completes it, exactly as tq_decode_partial / tq_decode_combine complete
 * tq_decode_attention. Arguments and errors as tq_decode_step. */
int tq_decode_step_partial(const tq_layout *layout, void *pages, int64_t num_pages, const void *k_new,
                           const void *v_new, int kv_dtype, const void *q, int q_dtype, int batch,
                           int num_q_heads, const int32_t *page_table, int max_pages_per_seq,
                           const int32_t *seq_lens, float softmax_scale, int pages_per_split, const void *k_cb,
                           const void *v_cb, void *workspace, size_t workspace_bytes, float *out, void *stream);

/* The two passes of tq_decode_attention. Called in this order on one stream with the same arguments,
 * they produce exactly the bytes tq_decode_attention produces (which is this pair of calls).
 *   tq_decode_partial  the split-K scan: every work-group reads one run of pages of one (sequence, KV
 *                      head) and writes its (max, sum of weights, rotated value sums) to `workspace`;
 *                      when the plan has a single run per sequence it finishes the rows into `out`.
 *   tq_decode_combine  merges the runs of each (sequence, query head) with log-sum-exp weights and
 *                      applies the inverse rotation into `out`; launches nothing when the plan has a
 *                      single run per sequence.
 * Argument rules and errors as for tq_decode_attention. */
int tq_decode_partial(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q,
                      int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                      int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                      int pages_per_split, const void *k_cb, const void *v_cb, void *workspace,
                      size_t workspace_bytes, float *out, void *stream);
int tq_decode_combine(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q,
                      int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                      int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                      int pages_per_split, const void *k_cb, const void *v_cb, void *workspace,
                      size_t workspace_bytes, float *out, void *stream);

/* ------------------------------------------------------------------------------------------------
 * Chunked prefill over the packed cache ("Where This Fits in the Inference Stack", "Decode Throughput
 * vs. Time to First Token": over long inputs the attention of prefill reads the cache too, and a cache
 * 4x smaller shortens it; "Why the KV Cache Exists", "The KV Cache Solution" and "Prefix Caching": the
 * prompt's keys and values are stored once and later tokens attend to the stored prefix).
 *
 * A chunk of chunk_len new tokens of each of `batch` sequences: token i of sequence b sits at position
 * prefix_lens[b] + i and attends causally to positions 0 .. prefix_lens[b] + i of its sequence, itself
 * included. Every key and value is read from the packed pages, the chunk's own included (they must have
 * been written there first: tq_prefill_chunk does both), so row i equals tq_decode_attention of its
 * query at sequence length prefix_lens[b] + i + 1 up to fp32 rounding.
 *   q            device [batch][chunk_len][num_q_heads][head_dim], dtype q_dtype, contiguous
 *   page_table   device int32 [batch][max_pages_per_seq]; entries < 0 or >= num_pages are empty pages
 *                (their tokens get no weight), as are positions >= max_pages_per_seq * 16
 *   prefix_lens  device int32 [batch]: cached tokens ahead of the chunk (negative values count as 0)
 *   out          device fp32 [batch][chunk_len][num_q_heads][head_dim] (written); a row that sees no
 *                key (every visible page empty) is zero
 * K may be in either mode (a sketched K adds the QJL term to every score, as in decode); V must be in MSE
 * mode (prod-mode V: TQ_ENOTSUP, as in decode); num_q_heads / num_kv_heads <= 16.
 * Errors: TQ_EINVAL (layout, dtype, shapes, null or misaligned pointers: pages and the codebooks
 * 16-byte aligned, q and out element-aligned), TQ_ENOTSUP, TQ_EHIP. batch or chunk_len 0 launches
 * nothing. */
int tq_prefill_attention(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q,
                         int q_dtype, int batch, int chunk_len, int num_q_heads, const int32_t *page_table,
                         int max_pages_per_seq, const int32_t *prefix_lens, float softmax_scale,
                         const void *k_cb, const void *v_cb, float *out, void *stream);

/* One prefill chunk: quantize its keys and values into the pages (tq_quantize_kv of the batch * chunk_len
 * tokens), then tq_prefill_attention, on `stream` in that order.
 *   k, v   device [batch][chunk_len][num_kv_heads][head_dim], dtype kv_dtype, contiguous, 16-byte aligned
 *   slots  device int64 [batch * chunk_len]: the global slot of each token, which must be the one the
 *          page table gives its position (page_table[b][t / 16] * 16 + t % 16 for t = prefix_lens[b] + i)
 * Every argument is checked before the first launch. Errors as for tq_quantize_kv and
 * tq_prefill_attention. */
int tq_prefill_chunk(const tq_layout *layout, void *pages, int64_t num_pages, const void *k, const void *v,
                     int kv_dtype, const int64_t *slots, const void *q, int q_dtype, int batch, int chunk_len,
                     int num_q_heads, const int32_t *page_table, int max_pages_per_seq,
                     const int32_t *prefix_lens, float softmax_scale, const void *k_cb, const void *v_cb,
                     float *out, void *stream);

/* ------------------------------------------------------------------------------------------------
 * Uncompressed comparator ("Where This Fits in the Inference Stack", "What Changes When KV Cache Is
 * 4x Smaller": decode reads the entire KV cache from HBM at every step, so a cache 4x smaller moves
 * 4x fewer bytes). The same paged, split-K GQA decode attention over a bf16 cache, with no quantization
 * and no rotation: the baseline the compressed path is measured against on the same GPU.
 *
 * Dense page layout (one pool per layer, 16 token slots per page, every KV head): K as
 * [head][slot][head_dim] bf16, then V as [head][head_dim][slot] bf16 (each head's values of a page stored
 * coordinate-major). Page bytes = 4 * num_kv_heads * 16 * head_dim. Token t of sequence b lives in page
 * page_table[b][t / 16], slot t % 16.
 *
 * head_dim must be 64 or 128, num_kv_heads >= 1; errors as for the compressed calls.
 * ------------------------------------------------------------------------------------------------ */

/* Bytes of one dense page. */
int tq_dense_page_bytes(int head_dim, int num_kv_heads, size_t *out);

/* Write n_tok tokens' K and V into dense pages, rounded to bf16 (nearest even).
 *   k, v   device [n_tok][num_kv_heads][head_dim] of `dtype` (TQ_F32, TQ_BF16 or TQ_F16), contiguous,
 *          16-byte aligned
 *   slots  device int64 [n_tok]: global slot (page * 16 + offset); a slot < 0 or >= num_pages * 16 is
 *          skipped
 * Errors: TQ_EINVAL for a bad head_dim / dtype, null or misaligned pointers, n_tok < 0. */
int tq_dense_write_kv(int head_dim, int num_kv_heads, void *pages, int64_t num_pages, const void *k,
                      const void *v, int dtype, int64_t n_tok, const int64_t *slots, void *stream);

/* Workspace bytes of tq_dense_decode_attention for these sizes (the split plan is the compressed
 * path's: same pages_per_split rule). */
int tq_dense_decode_workspace_bytes(int head_dim, int num_kv_heads, int batch, int num_q_heads,
                                    int max_pages_per_seq, int pages_per_split, size_t *out);

/* out[b][h][:] = sum_t softmax_t(scale * <q[b][h], k_t>) v_t over the seq_lens[b] cached tokens of
 * sequence b, query head h reading KV head h / (num_q_heads / num_kv_heads); fp32 out
 * [batch][num_q_heads][head_dim]. Arguments as for tq_decode_attention (q of TQ_F32 / TQ_BF16 /
 * TQ_F16, page_table, seq_lens, workspace), with the dense pool in place of the packed one.
 * Errors as for tq_decode_attention; TQ_ENOTSUP for more than 16 query heads per KV head. */
int tq_dense_decode_attention(int head_dim, int num_kv_heads, const void *pages, int64_t num_pages,
                              const void *q, int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                              int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                              int pages_per_split, void *workspace, size_t workspace_bytes, float *out,
                              void *stream);

/* ------------------------------------------------------------------------------------------------
 * FP8 comparator ("Who Should Care", its KV8 line; "The Three Layers of Compression", the KV cache layer;
 * "Quality vs. Compression: The Full Comparison": an 8-bit floating-point KV cache is the
 * hardware-native 2x baseline that serving stacks ship). The pages fix no format: the cache holds OCP
 * E4M3 bytes (bias 7, no infinities, 0x7F / 0xFF are NaN, largest finite 448) with one scale per tensor,
 * a byte standing for scale * its value. Same page layout and calls as the bf16 comparator with 1-byte
 * elements: page bytes = 2 * num_kv_heads * 16 * head_dim; workspace from
 * tq_dense_decode_workspace_bytes (the split plan does not depend on the element size).
 * k_scale, v_scale must be finite and > 0 (else TQ_EINVAL).
 * ------------------------------------------------------------------------------------------------ */

/* Bytes of one FP8 dense page. */
int tq_dense_fp8_page_bytes(int head_dim, int num_kv_heads, size_t *out);

/* Write n_tok tokens' K and V into FP8 pages: each element is the fp32 quotient x / scale (correctly
 * rounded), rounded to the nearest E4M3 value, ties to even, saturated to +-448. Arguments and errors as
 * for tq_dense_write_kv; inputs must be finite (a NaN input stores an unspecified byte). */
int tq_dense_fp8_write_kv(int head_dim, int num_kv_heads, void *pages, int64_t num_pages, const void *k,
                          const void *v, int dtype, int64_t n_tok, const int64_t *slots, float k_scale,
                          float v_scale, void *stream);

/* tq_dense_decode_attention over FP8 pages: keys and values are k_scale * byte value and v_scale * byte
 * value. Arguments and errors as for tq_dense_decode_attention. */
int tq_dense_fp8_decode_attention(int head_dim, int num_kv_heads, const void *pages, int64_t num_pages,
                                  const void *q, int q_dtype, int batch, int num_q_heads,
                                  const int32_t *page_table, int max_pages_per_seq, const int32_t *seq_lens,
                                  float softmax_scale, float k_scale, float v_scale, int pages_per_split,
                                  void *workspace, size_t workspace_bytes, float *out, void *stream);

/* ------------------------------------------------------------------------------------------------
 * Dense random (QR) rotation ("What the Paper Doesn't Tell You", Finding 4: the paper's rotation is a
 * dense random orthogonal matrix from a QR decomposition, d x d storage and O(d^2) work per vector; the
 * WHT with random signs replaces it). The rotation is Q, the orthogonal factor of G = Q T for a caller-drawn
 * iid N(0,1) matrix G, unique under diag(T) > 0. Codes, norms, page layout and attention are those of the
 * compressed path with R = Q in place of H diag(s) / sqrt(d).
 *
 * Realisation: the kernels of the WHT path apply W = H diag(s) / sqrt(d) with the codebook's signs s. The
 * rows are first rotated on the matrix cores by M = W^T Q, so that W M = Q: keys and values inside the
 * quantize kernel when both are in MSE mode (otherwise by tq_rotate_rows ahead of tq_quantize_kv), queries
 * (by the keys' M) before tq_decode_attention and its output by the transpose of the values' M
 * (tq_rotate_rows).
 * ------------------------------------------------------------------------------------------------ */

/* Host only. Q from the Householder QR of `gauss` (host fp64, row-major head_dim x head_dim, iid N(0,1)) in
 * fp64 with the sign convention diag(T) > 0, then fwd = M = diag(s) H Q / sqrt(head_dim) as fp32 row-major
 * (host, head_dim^2 floats) and, if `inv` is not null, its transpose. `sign_words`: host, the head_dim/32
 * sign words of the codebook that M will be used with (null: no signs). head_dim 64 or 128.
 * Errors: TQ_EINVAL (head_dim, null gauss / fwd, a singular or non-finite matrix). */
int tq_qr_rotation(int head_dim, const double *gauss, const uint32_t *sign_words, float *fwd, float *inv);

/* y[r] = mat x[r] for rows r < rows: x device [rows][head_dim] of x_dtype (TQ_F32, TQ_BF16, TQ_F16),
 * contiguous; mat device fp32 row-major head_dim x head_dim; y device fp32 [rows][head_dim] (not
 * overlapping x). All 16-byte aligned. Matrix cores with fp16 high/low splits of both operands (three
 * products): about 2^-22 relative error per product. rows = 0 launches nothing.
 * Errors: TQ_EINVAL (head_dim, dtype, null or misaligned pointers, rows < 0), TQ_EHIP. */
int tq_rotate_rows(int head_dim, const float *mat, const void *x, int x_dtype, int64_t rows, float *y, void *stream);

/* Workspace bytes of tq_quantize_kv_qr for n_tok tokens (two fp32 copies of the rotated rows, used when a
 * tensor is in prod mode; MSE keys and values need none but the size is the same). Host only. */
int tq_quantize_kv_qr_workspace_bytes(const tq_layout *layout, int64_t n_tok, size_t *out);

/* tq_quantize_kv with the dense rotation: k, v device [n_tok][num_kv_heads][head_dim] of `dtype`, contiguous,
 * 16-byte aligned; k_rot, v_rot device fp32 `fwd` matrices of tq_qr_rotation built with the sign words of
 * k_cb and v_cb respectively; workspace device, at least tq_quantize_kv_qr_workspace_bytes bytes. Other
 * arguments, the bytes written and the errors as for tq_quantize_kv (TQ_ENOSPC for a small workspace). */
int tq_quantize_kv_qr(const tq_layout *layout, void *pages, int64_t num_pages, const void *k, const void *v,
                      int dtype, int64_t n_tok, const int64_t *slots, const void *k_cb, const void *v_cb,
                      const float *k_rot, const float *v_rot, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Workspace bytes of tq_decode_attention_qr (tq_decode_workspace_bytes plus two fp32 rows per query head).
 * Host only. */
int tq_decode_qr_workspace_bytes(const tq_layout *layout, int batch, int num_q_heads, int max_pages_per_seq,
                                 int pages_per_split, size_t *out);

/* tq_decode_attention over a cache written by tq_quantize_kv_qr: k_rot the keys' `fwd` matrix, v_inv the
 * values' `inv` matrix (device fp32, 16-byte aligned); q and out 16-byte aligned; workspace at least
 * tq_decode_qr_workspace_bytes bytes. Other arguments and errors as for tq_decode_attention. */
int tq_decode_attention_qr(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q, int q_dtype,
                           int batch, int num_q_heads, const int32_t *page_table, int max_pages_per_seq,
                           const int32_t *seq_lens, float softmax_scale, int pages_per_split, const void *k_cb,
                           const void *v_cb, const float *k_rot, const float *v_inv, void *workspace,
                           size_t workspace_bytes, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
