// Host side of the C ABI: argument checks, the Gaussian Lloyd-Max solver that builds codebook blobs,
// the page layout, the decode workspace plan, and dispatch to the HIP launchers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace {

constexpr int kPageTokens = TQ_PAGE_TOKENS;

bool valid_head_dim(int d) { return d == 64 || d == 128; }

// Bits accepted per mode: MSE 1,2,3,4,8; prod 2,3,4 (a 1..3-bit Lloyd-Max index plus one sketch bit).
bool valid_bits(int bits, int mode) {
  if (mode == TQ_MSE) return bits == 1 || bits == 2 || bits == 3 || bits == 4 || bits == 8;
  if (mode == TQ_PROD) return bits == 2 || bits == 3 || bits == 4;
  return false;
}

int index_bits(int bits, int mode) { return mode == TQ_PROD ? bits - 1 : bits; }

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// ------------------------------------------------------------------------------------------
// Gaussian Lloyd-Max levels (fp64). The positive half p_0 < ... < p_{K-1} of a symmetric
// 2K-level quantizer satisfies, with cell edges e_0 = 0, e_k = (p_{k-1} + p_k)/2, e_K = inf:
//     p_k * (Q(e_k) - Q(e_{k+1})) = phi(e_k) - phi(e_{k+1})          (conditional mean)
// where Q is the Gaussian upper tail. Lloyd sweeps from equiprobable cells get close; damped
// Newton with a tridiagonal Jacobian finishes the solve.
// ------------------------------------------------------------------------------------------
const double kInvSqrt2Pi = 0.39894228040143267794;

double gauss_pdf(double x) { return std::isinf(x) ? 0.0 : kInvSqrt2Pi * std::exp(-0.5 * x * x); }
double gauss_upper(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }

// x >= 0 with Q(x) = target (target in (0, 0.5]) by bisection.
double gauss_upper_inverse(double target) {
  double lo = 0.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    double mid = 0.5 * (lo + hi);
    if (gauss_upper(mid) > target) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

void cell_edges(const std::vector<double> &p, std::vector<double> &e) {
  size_t K = p.size();
  e.assign(K + 1, 0.0);
  for (size_t k = 1; k < K; ++k) e[k] = 0.5 * (p[k - 1] + p[k]);
  e[K] = INFINITY;
}

void lloyd_sweep(std::vector<double> &p) {
  std::vector<double> e;
  cell_edges(p, e);
  for (size_t k = 0; k < p.size(); ++k)
    p[k] = (gauss_pdf(e[k]) - gauss_pdf(e[k + 1])) / (gauss_upper(e[k]) - gauss_upper(e[k + 1]));
}

std::vector<double> positive_levels(int index_bits_) {
  const int L = 1 << index_bits_;
  const int K = L / 2;
  std::vector<double> p(K);
  for (int k = 0; k < K; ++k) p[k] = gauss_upper_inverse(0.5 - (k + 0.5) / L);
  for (int it = 0; it < 100; ++it) lloyd_sweep(p);
  std::vector<double> e, F(K), lo(K), di(K), up(K), step(K), cp(K), dp(K);
  for (int it = 0; it < 200; ++it) {
    cell_edges(p, e);
    for (int k = 0; k < K; ++k) {
      double mass = gauss_upper(e[k]) - gauss_upper(e[k + 1]);
      F[k] = p[k] * mass - (gauss_pdf(e[k]) - gauss_pdf(e[k + 1]));
      di[k] = mass;
      lo[k] = up[k] = 0.0;
      if (k >= 1) {
        double g = (e[k] - p[k]) * gauss_pdf(e[k]);
        di[k] += 0.5 * g;
        lo[k] = 0.5 * g;
      }
      if (k <= K - 2) {
        double g = (p[k] - e[k + 1]) * gauss_pdf(e[k + 1]);
        di[k] += 0.5 * g;
        up[k] = 0.5 * g;
      }
    }
    // Thomas algorithm for J * step = -F
    cp[0] = up[0] / di[0];
    dp[0] = -F[0] / di[0];
    for (int k = 1; k < K; ++k) {
      double den = di[k] - lo[k] * cp[k - 1];
      cp[k] = up[k] / den;
      dp[k] = (-F[k] - lo[k] * dp[k - 1]) / den;
    }
    step[K - 1] = dp[K - 1];
    for (int k = K - 2; k >= 0; --k) step[k] = dp[k] - cp[k] * step[k + 1];
    double lam = 1.0;
    std::vector<double> cand(K);
    for (int tries = 0; tries < 60; ++tries) {
      bool ok = true;
      for (int k = 0; k < K; ++k) cand[k] = p[k] + lam * step[k];
      if (cand[0] <= 0) ok = false;
      for (int k = 1; k < K && ok; ++k) ok = cand[k] > cand[k - 1];
      if (ok) break;
      lam *= 0.5;
    }
    double rel = 0.0;
    for (int k = 0; k < K; ++k) rel = std::max(rel, std::fabs(lam * step[k]) / std::max(1.0, std::fabs(cand[k])));
    p = cand;
    if (rel < 1e-15) break;
  }
  lloyd_sweep(p);
  return p;
}

// Round to IEEE binary16, ties to even (current rounding mode is assumed round-to-nearest).
uint16_t to_half_bits(double x) {
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs(x);
  if (std::isnan(x)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;
  int e;
  std::frexp(a, &e);  // a = m * 2^e, m in [0.5, 1)
  int E = e - 1;      // a in [2^E, 2^(E+1))
  if (a == 0.0) return sign;
  if (E >= -14) {
    double r = std::nearbyint(std::ldexp(a, 10 - E));  // [1024, 2048]
    if (r >= 2048.0) { r = 1024.0; E += 1; }
    if (E > 15) return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)r - 1024));
  }
  double r = std::nearbyint(std::ldexp(a, 24));  // subnormal count of 2^-24
  return sign | (uint16_t)r;
}

double half_bits_to_double(uint16_t h) {
  int s = h >> 15, E = (h >> 10) & 31, M = h & 1023;
  double v;
  if (E == 0) v = std::ldexp((double)M, -24);
  else if (E == 31) v = M ? NAN : INFINITY;
  else v = std::ldexp(1024.0 + M, E - 25);
  return s ? -v : v;
}

struct BlobPlan {
  int n_levels, rows;
  uint32_t levels_off, thresholds_off, signs_off, proj_off, total;
};

BlobPlan plan_blob(int head_dim, int bits, int mode) {
  BlobPlan b{};
  b.n_levels = 1 << index_bits(bits, mode);
  b.rows = mode == TQ_PROD ? head_dim : 0;
  size_t off = sizeof(tq_codebook_header);
  b.levels_off = (uint32_t)off;
  off = align16(off + 2 * (size_t)b.n_levels);
  b.thresholds_off = (uint32_t)off;
  off = align16(off + 4 * (size_t)(b.n_levels - 1));
  b.signs_off = (uint32_t)off;
  off = align16(off + 4 * (size_t)(head_dim / 32));
  b.proj_off = 0;
  if (b.rows) {
    b.proj_off = (uint32_t)off;
    off = align16(off + 4 * (size_t)b.rows * head_dim);
  }
  b.total = (uint32_t)off;
  return b;
}

bool valid_layout(const tq_layout *L) {
  return L && valid_head_dim(L->head_dim) && L->num_kv_heads >= 1 && L->num_kv_heads <= 4096 &&
         L->page_tokens == kPageTokens && valid_bits(L->k_bits, L->k_mode) &&
         valid_bits(L->v_bits, L->v_mode);
}

}  // namespace

namespace tq {

BlobOffsets blob_offsets(int head_dim, int bits, int mode) {
  BlobPlan P = plan_blob(head_dim, bits, mode);
  return BlobOffsets{P.levels_off, P.thresholds_off, P.signs_off, P.proj_off, P.rows};
}

int make_geom(const tq_layout *L, PageGeom *g) {
  if (!valid_layout(L) || !g) return TQ_EINVAL;
  const int64_t H = L->num_kv_heads, d = L->head_dim, T = kPageTokens;
  int64_t off = 0;
  auto section = [&](int bits, int mode, int64_t *codes, int64_t *norms, int64_t *qjl, int64_t *gamma,
                     int *b_out) {
    int b = index_bits(bits, mode);
    *b_out = b;
    *codes = off;
    off = (int64_t)align16(off + H * T * d * b / 8);
    *norms = off;
    off = (int64_t)align16(off + H * T * 2);
    *qjl = *gamma = 0;
    if (mode == TQ_PROD) {
      *qjl = off;
      off = (int64_t)align16(off + H * T * d / 8);
      *gamma = off;
      off = (int64_t)align16(off + H * T * 2);
    }
  };
  section(L->k_bits, L->k_mode, &g->k_codes, &g->k_norms, &g->k_qjl, &g->k_gamma, &g->k_mse_bits);
  section(L->v_bits, L->v_mode, &g->v_codes, &g->v_norms, &g->v_qjl, &g->v_gamma, &g->v_mse_bits);
  g->page_bytes = off;
  g->head_dim = (int)d;
  g->num_kv_heads = (int)H;
  g->k_mode = L->k_mode;
  g->v_mode = L->v_mode;
  g->kcb = blob_offsets(L->head_dim, L->k_bits, L->k_mode);
  g->vcb = blob_offsets(L->head_dim, L->v_bits, L->v_mode);
  return TQ_OK;
}

int plan_decode(const PageGeom &g, int batch, int num_q_heads, int max_pages_per_seq,
                int pages_per_split, DecodeWs *ws) {
  if (batch < 0 || num_q_heads < 1 || max_pages_per_seq < 1 || pages_per_split < 0) return TQ_EINVAL;
  if (num_q_heads % g.num_kv_heads) return TQ_EINVAL;
  int pps = pages_per_split;
  if (pps == 0) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
      int v = 0;
      if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    // about one 8-wave work-group per compute unit over all (sequence, KV head) pairs, each run a whole
    // number of 16-page rounds (one page pair per wavefront); the last run takes the remainder
    int64_t units = (int64_t)std::max(batch, 1) * g.num_kv_heads;
    int64_t want_splits = std::max<int64_t>(1, (cus + units - 1) / units);
    pps = (int)std::max<int64_t>(16, (max_pages_per_seq / want_splits) / 16 * 16);
  }
  pps = (pps + 1) & ~1;  // whole page pairs
  // the last run holds fewer than 2 * pps pages
  if (pps > kDecodePidCap / 2) pps = kDecodePidCap / 2;
  if (max_pages_per_seq / pps > kDecodeMaxSplits) {
    pps = (max_pages_per_seq + kDecodeMaxSplits - 1) / kDecodeMaxSplits;
    pps = (pps + 1) & ~1;
    if (pps > kDecodePidCap / 2) return TQ_EINVAL;
  }
  ws->pages_per_split = pps;
  ws->n_splits = std::max(1, max_pages_per_seq / pps);
  const size_t B = (size_t)std::max(batch, 0), Hq = (size_t)num_q_heads, d = (size_t)g.head_dim;
  const size_t S = (size_t)ws->n_splits;
  size_t off = 0;
  ws->part_o_off = off;
  off = align16(off + 4 * B * Hq * S * d);
  ws->part_ml_off = off;
  off = align16(off + 4 * B * Hq * S * 2);
  ws->total = off;
  return TQ_OK;
}

}  // namespace tq

extern "C" {

const char *tq_strerror(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_ENOSPC: return "buffer too small";
    case TQ_ENOTSUP: return "combination not supported";
    case TQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int tq_codebook_bytes(int head_dim, int bits, int mode, size_t *out) {
  if (!out || !valid_head_dim(head_dim) || !valid_bits(bits, mode)) return TQ_EINVAL;
  *out = plan_blob(head_dim, bits, mode).total;
  return TQ_OK;
}

int tq_build_codebook(int head_dim, int bits, int mode, const uint32_t *sign_words,
                      const float *qjl_proj, void *blob, size_t blob_bytes) {
  if (!valid_head_dim(head_dim) || !valid_bits(bits, mode) || !sign_words || !blob) return TQ_EINVAL;
  if (mode == TQ_PROD && !qjl_proj) return TQ_EINVAL;
  BlobPlan P = plan_blob(head_dim, bits, mode);
  if (blob_bytes < P.total) return TQ_ENOSPC;
  unsigned char *base = (unsigned char *)blob;
  std::memset(base, 0, P.total);
  tq_codebook_header h{};
  h.magic = TQ_CODEBOOK_MAGIC;
  h.version = TQ_CODEBOOK_VERSION;
  h.head_dim = head_dim;
  h.bits = bits;
  h.mode = mode;
  h.mse_bits = index_bits(bits, mode);
  h.n_levels = P.n_levels;
  h.qjl_rows = P.rows;
  h.levels_off = P.levels_off;
  h.thresholds_off = P.thresholds_off;
  h.signs_off = P.signs_off;
  h.proj_off = P.proj_off;
  h.total_bytes = P.total;
  std::memcpy(base, &h, sizeof(h));

  std::vector<double> pos = positive_levels(h.mse_bits);
  const int K = P.n_levels / 2;
  std::vector<uint16_t> lv(P.n_levels);
  for (int k = 0; k < K; ++k) {
    uint16_t hb = to_half_bits(pos[k]);
    lv[K + k] = hb;
    lv[K - 1 - k] = (uint16_t)(hb | 0x8000);
  }
  std::memcpy(base + P.levels_off, lv.data(), 2 * lv.size());
  std::vector<float> th(P.n_levels - 1);
  for (int j = 0; j + 1 < P.n_levels; ++j)
    th[j] = (float)(0.5 * (half_bits_to_double(lv[j]) + half_bits_to_double(lv[j + 1])));
  std::memcpy(base + P.thresholds_off, th.data(), 4 * th.size());
  std::memcpy(base + P.signs_off, sign_words, 4 * (size_t)(head_dim / 32));
  if (P.rows) std::memcpy(base + P.proj_off, qjl_proj, 4 * (size_t)P.rows * head_dim);
  return TQ_OK;
}

namespace {

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): the state
// advances by the golden-ratio increment and each output is the state through Stafford's variant-13 mix.
struct SplitMix64 {
  uint64_t state;
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

constexpr uint64_t kSignStream = 0x5349474Eull;  // "SIGN"
constexpr uint64_t kQjlStream = 0x514A4C53ull;   // "QJLS"

// The rotation's signs: the bits of consecutive outputs of stream seed ^ "SIGN", low to high (bit i of the vector
// is bit i % 64 of output i / 64; set = coordinate negated).
void draw_signs(uint64_t seed, int head_dim, uint32_t *words) {
  SplitMix64 g{seed ^ kSignStream};
  for (int w = 0; w < head_dim / 32; w += 2) {
    const uint64_t x = g.next();
    words[w] = (uint32_t)x;
    if (w + 1 < head_dim / 32) words[w + 1] = (uint32_t)(x >> 32);
  }
}

// The QJL projection, rows x head_dim row-major: Box-Muller ("A Note on the Generation of Random Normal Deviates",
// 1958) on output pairs of stream seed ^ "QJLS": u = ((x >> 11) + 1/2) 2^-53 in (0, 1], r = sqrt(-2 ln u1), the
// pair r cos(2 pi u2), r sin(2 pi u2) into entries 2k, 2k + 1 (fp64, then rounded to fp32).
void draw_projection(uint64_t seed, int rows, int head_dim, float *S) {
  SplitMix64 g{seed ^ kQjlStream};
  const int n = rows * head_dim;
  const double two_pi = 2.0 * 3.141592653589793;
  for (int k = 0; k < n; k += 2) {
    const double u1 = ((double)(g.next() >> 11) + 0.5) * 0x1p-53;
    const double u2 = ((double)(g.next() >> 11) + 0.5) * 0x1p-53;
    const double r = std::sqrt(-2.0 * std::log(u1));
    const double t = two_pi * u2;
    const double c = std::cos(t);
    const double sn = std::sin(t);
    S[k] = (float)(r * c);
    if (k + 1 < n) S[k + 1] = (float)(r * sn);
  }
}

}  // namespace

int tq_build_codebook_seeded(int head_dim, int bits, int mode, uint64_t seed, void *blob, size_t blob_bytes) {
  if (!valid_head_dim(head_dim) || !valid_bits(bits, mode) || !blob) return TQ_EINVAL;
  std::vector<uint32_t> signs((size_t)head_dim / 32);
  draw_signs(seed, head_dim, signs.data());
  std::vector<float> S;
  if (mode == TQ_PROD) {
    S.resize((size_t)head_dim * head_dim);
    draw_projection(seed, head_dim, head_dim, S.data());
  }
  return tq_build_codebook(head_dim, bits, mode, signs.data(), S.empty() ? nullptr : S.data(), blob, blob_bytes);
}

int tq_stream_read(const void *buf, size_t bytes, int blocks, uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15) || blocks < 1 || blocks > (1 << 20))
    return TQ_EINVAL;
  return tq::launch_stream_read(buf, (int64_t)bytes, blocks, sink, (hipStream_t)stream);
}

int tq_page_layout(const tq_layout *layout, tq_page_offsets *out) {
  if (!out) return TQ_EINVAL;
  tq::PageGeom g;
  int st = tq::make_geom(layout, &g);
  if (st) return st;
  out->k_codes = g.k_codes;
  out->k_norms = g.k_norms;
  out->k_qjl = g.k_qjl;
  out->k_gamma = g.k_gamma;
  out->v_codes = g.v_codes;
  out->v_norms = g.v_norms;
  out->v_qjl = g.v_qjl;
  out->v_gamma = g.v_gamma;
  out->page_bytes = g.page_bytes;
  return TQ_OK;
}

int tq_quantize_kv(const tq_layout *layout, void *pages, int64_t num_pages, const void *k,
                   const void *v, int dtype, int64_t n_tok, int64_t k_stride_tok,
                   int64_t v_stride_tok, const int64_t *slots, const void *k_cb, const void *v_cb,
                   void *stream) {
  tq::PageGeom g;
  int st = tq::make_geom(layout, &g);
  if (st) return st;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_EINVAL;
  if (n_tok < 0 || num_pages < 0) return TQ_EINVAL;
  if (n_tok == 0) return TQ_OK;
  if (!pages || !k || !v || !slots || !k_cb || !v_cb) return TQ_EINVAL;
  if (((uintptr_t)pages | (uintptr_t)k_cb | (uintptr_t)v_cb) & 15) return TQ_EINVAL;
  const int64_t row = (int64_t)g.num_kv_heads * g.head_dim;
  if (k_stride_tok < row || v_stride_tok < row) return TQ_EINVAL;
  if ((k_stride_tok | v_stride_tok) & 7) return TQ_EINVAL;             // 8-element rows stay 16-byte aligned
  if (((uintptr_t)k | (uintptr_t)v) & 15) return TQ_EINVAL;
  if (n_tok > ((int64_t)1 << 40)) return TQ_EINVAL;
  return tq::launch_quantize(g, pages, num_pages, k, v, dtype, n_tok, k_stride_tok, v_stride_tok,
                             slots, k_cb, v_cb, (hipStream_t)stream);
}

int tq_decode_workspace_bytes(const tq_layout *layout, int batch, int num_q_heads,
                              int max_pages_per_seq, int pages_per_split, size_t *out) {
  if (!out) return TQ_EINVAL;
  tq::PageGeom g;
  int st = tq::make_geom(layout, &g);
  if (st) return st;
  tq::DecodeWs ws;
  st = tq::plan_decode(g, batch, num_q_heads, max_pages_per_seq, pages_per_split, &ws);
  if (st) return st;
  *out = ws.total;
  return TQ_OK;
}

// Every check of a decode call but the workspace's, and its plan. Returns TQ_OK with *launch = false when there is
// nothing to launch (batch 0).
static int decode_prepare(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q, int q_dtype,
                          int batch, int num_q_heads, const int32_t *page_table, int max_pages_per_seq,
                          const int32_t *seq_lens, float softmax_scale, int pages_per_split, const void *k_cb,
                          const void *v_cb, float *out, tq::PageGeom *g, tq::DecodeWs *ws, bool *launch) {
  *launch = false;
  int st = tq::make_geom(layout, g);
  if (st) return st;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return TQ_EINVAL;
  if (batch < 0 || num_q_heads < 1 || num_q_heads % g->num_kv_heads) return TQ_EINVAL;
  if (num_q_heads / g->num_kv_heads > 16) return TQ_ENOTSUP;  // one MFMA column block of query heads
  if (g->v_mode == TQ_PROD) return TQ_ENOTSUP;
  if (max_pages_per_seq < 1 || num_pages < 1 || !std::isfinite(softmax_scale) || softmax_scale < 0.f) return TQ_EINVAL;
  if (batch == 0) return TQ_OK;
  if (!pages || !q || !page_table || !seq_lens || !k_cb || !v_cb || !out) return TQ_EINVAL;
  if (((uintptr_t)pages | (uintptr_t)k_cb | (uintptr_t)v_cb) & 15) return TQ_EINVAL;
  st = tq::plan_decode(*g, batch, num_q_heads, max_pages_per_seq, pages_per_split, ws);
  if (st) return st;
  *launch = true;
  return TQ_OK;
}

static int decode_passes(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q,
                         int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                         int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                         int pages_per_split, const void *k_cb, const void *v_cb, void *workspace,
                         size_t workspace_bytes, float *out, int passes, void *stream,
                         const void *k_new = nullptr, const void *v_new = nullptr, int kv_dtype = TQ_BF16) {
  tq::PageGeom g;
  tq::DecodeWs ws;
  bool launch = false;
  int st = decode_prepare(layout, pages, num_pages, q, q_dtype, batch, num_q_heads, page_table, max_pages_per_seq,
                          seq_lens, softmax_scale, pages_per_split, k_cb, v_cb, out, &g, &ws, &launch);
  if (st || !launch) return st;
  if (!workspace || ((uintptr_t)workspace & 15)) return TQ_EINVAL;
  if (workspace_bytes < ws.total) return TQ_ENOSPC;
  return tq::launch_decode(g, ws, pages, num_pages, q, q_dtype, batch, num_q_heads, page_table,
                           max_pages_per_seq, seq_lens, softmax_scale, k_cb, v_cb, workspace, out, passes,
                           k_new, v_new, kv_dtype, (hipStream_t)stream);
}

int tq_decode_attention(const tq_layout *layout, const void *pages, int64_t num_pages,
                        const void *q, int q_dtype, int batch, int num_q_heads,
                        const int32_t *page_table, int max_pages_per_seq, const int32_t *seq_lens,
                        float softmax_scale, int pages_per_split, const void *k_cb,
                        const void *v_cb, void *workspace, size_t workspace_bytes, float *out,
                        void *stream) {
  return decode_passes(layout, pages, num_pages, q, q_dtype, batch, num_q_heads, page_table, max_pages_per_seq,
                       seq_lens, softmax_scale, pages_per_split, k_cb, v_cb, workspace, workspace_bytes, out,
                       tq::kPassScan | tq::kPassCombine, stream);
}

int tq_decode_attention_noalloc(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q,
                                int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                                int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                                int pages_per_split, const void *k_cb, const void *v_cb, float *out, void *stream) {
  tq::PageGeom g;
  tq::DecodeWs ws;
  bool launch = false;
  int st = decode_prepare(layout, pages, num_pages, q, q_dtype, batch, num_q_heads, page_table, max_pages_per_seq,
                          seq_lens, softmax_scale, pages_per_split, k_cb, v_cb, out, &g, &ws, &launch);
  if (st || !launch) return st;
  if (ws.total > tq::kDecodeScratchBytes) return TQ_ENOSPC;  // the plan's partials do not fit the fixed array
  void *scratch = nullptr;
  st = tq::decode_scratch(&scratch);
  if (st) return st;
  return tq::launch_decode(g, ws, pages, num_pages, q, q_dtype, batch, num_q_heads, page_table, max_pages_per_seq,
                           seq_lens, softmax_scale, k_cb, v_cb, scratch, out, tq::kPassScan | tq::kPassCombine,
                           nullptr, nullptr, TQ_BF16, (hipStream_t)stream);
}

static int decode_step_passes(const tq_layout *layout, void *pages, int64_t num_pages, const void *k_new,
                              const void *v_new, int kv_dtype, const void *q, int q_dtype, int batch,
                              int num_q_heads, const int32_t *page_table, int max_pages_per_seq,
                              const int32_t *seq_lens, float softmax_scale, int pages_per_split,
                              const void *k_cb, const void *v_cb, void *workspace, size_t workspace_bytes,
                              float *out, int passes, void *stream) {
  tq::PageGeom g;
  int st = tq::make_geom(layout, &g);
  if (st) return st;
  if (kv_dtype != TQ_F32 && kv_dtype != TQ_BF16 && kv_dtype != TQ_F16) return TQ_EINVAL;
  if (batch > 0 && (!k_new || !v_new || (((uintptr_t)k_new | (uintptr_t)v_new) & 15))) return TQ_EINVAL;
  // the appending work-group quantizes with register thresholds: MSE codes of up to 4 bits
  if (g.k_mode != TQ_MSE || g.v_mode != TQ_MSE || g.k_mse_bits > 4 || g.v_mse_bits > 4) return TQ_ENOTSUP;
  return decode_passes(layout, pages, num_pages, q, q_dtype, batch, num_q_heads, page_table, max_pages_per_seq,
                       seq_lens, softmax_scale, pages_per_split, k_cb, v_cb, workspace, workspace_bytes, out,
                       passes, stream, k_new, v_new, kv_dtype);
}

int tq_decode_step(const tq_layout *layout, void *pages, int64_t num_pages, const void *k_new,
                   const void *v_new, int kv_dtype, const void *q, int q_dtype, int batch, int num_q_heads,
                   const int32_t *page_table, int max_pages_per_seq, const int32_t *seq_lens,
                   float softmax_scale, int pages_per_split, const void *k_cb, const void *v_cb,
                   void *workspace, size_t workspace_bytes, float *out, void *stream) {
  return decode_step_passes(layout, pages, num_pages, k_new, v_new, kv_dtype, q, q_dtype, batch, num_q_heads,
                            page_table, max_pages_per_seq, seq_lens, softmax_scale, pages_per_split, k_cb, v_cb,
                            workspace, workspace_bytes, out, tq::kPassScan | tq::kPassCombine, stream);
}

int tq_decode_step_partial(const tq_layout *layout, void *pages, int64_t num_pages, const void *k_new,
                           const void *v_new, int kv_dtype, const void *q, int q_dtype, int batch,
                           int num_q_heads, const int32_t *page_table, int max_pages_per_seq,
                           const int32_t *seq_lens, float softmax_scale, int pages_per_split, const void *k_cb,
                           const void *v_cb, void *workspace, size_t workspace_bytes, float *out, void *stream) {
  return decode_step_passes(layout, pages, num_pages, k_new, v_new, kv_dtype, q, q_dtype, batch, num_q_heads,
                            page_table, max_pages_per_seq, seq_lens, softmax_scale, pages_per_split, k_cb, v_cb,
                            workspace, workspace_bytes, out, tq::kPassScan, stream);
}

int tq_decode_partial(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q,
                      int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                      int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                      int pages_per_split, const void *k_cb, const void *v_cb, void *workspace,
                      size_t workspace_bytes, float *out, void *stream) {
  return decode_passes(layout, pages, num_pages, q, q_dtype, batch, num_q_heads, page_table, max_pages_per_seq,
                       seq_lens, softmax_scale, pages_per_split, k_cb, v_cb, workspace, workspace_bytes, out,
                       tq::kPassScan, stream);
}

int tq_decode_combine(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q,
                      int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                      int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                      int pages_per_split, const void *k_cb, const void *v_cb, void *workspace,
                      size_t workspace_bytes, float *out, void *stream) {
  return decode_passes(layout, pages, num_pages, q, q_dtype, batch, num_q_heads, page_table, max_pages_per_seq,
                       seq_lens, softmax_scale, pages_per_split, k_cb, v_cb, workspace, workspace_bytes, out,
                       tq::kPassCombine, stream);
}

// Every check of tq_prefill_attention, before anything is launched (tq_prefill_chunk runs them ahead of its
// quantize launch too).
static int prefill_check(const tq_layout *layout, tq::PageGeom *g, const void *pages, int64_t num_pages,
                         const void *q, int q_dtype, int batch, int chunk_len, int num_q_heads,
                         const int32_t *page_table, int max_pages_per_seq, const int32_t *prefix_lens,
                         float softmax_scale, const void *k_cb, const void *v_cb, const float *out) {
  int st = tq::make_geom(layout, g);
  if (st) return st;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return TQ_EINVAL;
  if (batch < 0 || chunk_len < 0 || num_q_heads < 1 || num_q_heads % g->num_kv_heads) return TQ_EINVAL;
  if (num_q_heads / g->num_kv_heads > 16) return TQ_ENOTSUP;
  if (g->v_mode != TQ_MSE) return TQ_ENOTSUP;
  if (max_pages_per_seq < 1 || max_pages_per_seq > (1 << 26) || num_pages < 1) return TQ_EINVAL;
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return TQ_EINVAL;
  if (batch == 0 || chunk_len == 0) return TQ_OK;
  if (!pages || !q || !page_table || !prefix_lens || !k_cb || !v_cb || !out) return TQ_EINVAL;
  if (((uintptr_t)pages | (uintptr_t)k_cb | (uintptr_t)v_cb) & 15) return TQ_EINVAL;
  if (((uintptr_t)q & (q_dtype == TQ_F32 ? 3 : 1)) || ((uintptr_t)out & 3)) return TQ_EINVAL;
  // work-groups own 64 columns or more; this bound covers every column count
  const int64_t tiles = ((int64_t)chunk_len * (num_q_heads / g->num_kv_heads) + 63) / 64 + 1;
  if (tiles * g->num_kv_heads * batch > 0x7FFFFFFF) return TQ_EINVAL;
  return TQ_OK;
}

int tq_prefill_attention(const tq_layout *layout, const void *pages, int64_t num_pages, const void *q, int q_dtype,
                         int batch, int chunk_len, int num_q_heads, const int32_t *page_table,
                         int max_pages_per_seq, const int32_t *prefix_lens, float softmax_scale, const void *k_cb,
                         const void *v_cb, float *out, void *stream) {
  tq::PageGeom g;
  const int st = prefill_check(layout, &g, pages, num_pages, q, q_dtype, batch, chunk_len, num_q_heads, page_table,
                               max_pages_per_seq, prefix_lens, softmax_scale, k_cb, v_cb, out);
  if (st || batch == 0 || chunk_len == 0) return st;
  return tq::launch_prefill(g, pages, num_pages, q, q_dtype, batch, chunk_len, num_q_heads, page_table,
                            max_pages_per_seq, prefix_lens, softmax_scale, k_cb, v_cb, out, (hipStream_t)stream);
}

int tq_prefill_chunk(const tq_layout *layout, void *pages, int64_t num_pages, const void *k, const void *v,
                     int kv_dtype, const int64_t *slots, const void *q, int q_dtype, int batch, int chunk_len,
                     int num_q_heads, const int32_t *page_table, int max_pages_per_seq, const int32_t *prefix_lens,
                     float softmax_scale, const void *k_cb, const void *v_cb, float *out, void *stream) {
  tq::PageGeom g;
  int st = prefill_check(layout, &g, pages, num_pages, q, q_dtype, batch, chunk_len, num_q_heads, page_table,
                         max_pages_per_seq, prefix_lens, softmax_scale, k_cb, v_cb, out);
  if (st || batch == 0 || chunk_len == 0) return st;
  // the quantize call's own checks, ahead of its launch, so that a failure launches nothing
  if (kv_dtype != TQ_F32 && kv_dtype != TQ_BF16 && kv_dtype != TQ_F16) return TQ_EINVAL;
  if (!k || !v || !slots || (((uintptr_t)k | (uintptr_t)v) & 15)) return TQ_EINVAL;
  const int64_t row = (int64_t)g.num_kv_heads * g.head_dim;
  const int64_t n_tok = (int64_t)batch * chunk_len;
  if ((st = tq_quantize_kv(layout, pages, num_pages, k, v, kv_dtype, n_tok, row, row, slots, k_cb, v_cb, stream)))
    return st;
  return tq::launch_prefill(g, pages, num_pages, q, q_dtype, batch, chunk_len, num_q_heads, page_table,
                            max_pages_per_seq, prefix_lens, softmax_scale, k_cb, v_cb, out, (hipStream_t)stream);
}

static int dense_geom(int head_dim, int num_kv_heads, bool fp8, tq::PageGeom *g) {
  if ((head_dim != 64 && head_dim != 128) || num_kv_heads < 1 || num_kv_heads > 4096) return TQ_EINVAL;
  *g = tq::PageGeom{};
  g->head_dim = head_dim;
  g->num_kv_heads = num_kv_heads;
  g->page_bytes = (int64_t)(fp8 ? 2 : 4) * num_kv_heads * TQ_PAGE_TOKENS * head_dim;
  return TQ_OK;
}

static bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

static int dense_page_bytes(int head_dim, int num_kv_heads, bool fp8, size_t *out) {
  tq::PageGeom g;
  const int st = dense_geom(head_dim, num_kv_heads, fp8, &g);
  if (st) return st;
  if (!out) return TQ_EINVAL;
  *out = (size_t)g.page_bytes;
  return TQ_OK;
}

static int dense_write(int head_dim, int num_kv_heads, const tq::DenseFormat &fmt, void *pages, int64_t num_pages,
                       const void *k, const void *v, int dtype, int64_t n_tok, const int64_t *slots, void *stream) {
  tq::PageGeom g;
  const int st = dense_geom(head_dim, num_kv_heads, fmt.fp8, &g);
  if (st) return st;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_EINVAL;
  if (n_tok < 0 || num_pages < 0) return TQ_EINVAL;
  if (!valid_scale(fmt.k_scale) || !valid_scale(fmt.v_scale)) return TQ_EINVAL;
  if (n_tok == 0) return TQ_OK;
  if (!pages || !k || !v || !slots) return TQ_EINVAL;
  if (((uintptr_t)pages | (uintptr_t)k | (uintptr_t)v) & 15) return TQ_EINVAL;
  return tq::launch_dense_write(head_dim, num_kv_heads, fmt, pages, num_pages, k, v, dtype, n_tok, slots,
                                (hipStream_t)stream);
}

static int dense_decode(int head_dim, int num_kv_heads, const tq::DenseFormat &fmt, const void *pages,
                        int64_t num_pages, const void *q, int q_dtype, int batch, int num_q_heads,
                        const int32_t *page_table, int max_pages_per_seq, const int32_t *seq_lens,
                        float softmax_scale, int pages_per_split, void *workspace, size_t workspace_bytes,
                        float *out, void *stream) {
  tq::PageGeom g;
  int st = dense_geom(head_dim, num_kv_heads, fmt.fp8, &g);
  if (st) return st;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return TQ_EINVAL;
  if (batch < 0 || num_q_heads < 1 || num_q_heads % num_kv_heads) return TQ_EINVAL;
  if (num_q_heads / num_kv_heads > 16) return TQ_ENOTSUP;
  if (max_pages_per_seq < 1 || num_pages < 1 || !std::isfinite(softmax_scale) || softmax_scale < 0.f) return TQ_EINVAL;
  if (!valid_scale(fmt.k_scale) || !valid_scale(fmt.v_scale)) return TQ_EINVAL;
  if (batch == 0) return TQ_OK;
  if (!pages || !q || !page_table || !seq_lens || !workspace || !out) return TQ_EINVAL;
  if (((uintptr_t)pages | (uintptr_t)workspace) & 15) return TQ_EINVAL;
  tq::DecodeWs ws;
  st = tq::plan_decode(g, batch, num_q_heads, max_pages_per_seq, pages_per_split, &ws);
  if (st) return st;
  if (workspace_bytes < ws.total) return TQ_ENOSPC;
  return tq::launch_dense_decode(head_dim, num_kv_heads, fmt, ws, pages, num_pages, q, q_dtype, batch, num_q_heads,
                                 page_table, max_pages_per_seq, seq_lens, softmax_scale, workspace, out,
                                 tq::kPassScan | tq::kPassCombine, (hipStream_t)stream);
}

static const tq::DenseFormat kBf16Format{false, 1.f, 1.f};

int tq_dense_page_bytes(int head_dim, int num_kv_heads, size_t *out) {
  return dense_page_bytes(head_dim, num_kv_heads, false, out);
}

int tq_dense_write_kv(int head_dim, int num_kv_heads, void *pages, int64_t num_pages, const void *k,
                      const void *v, int dtype, int64_t n_tok, const int64_t *slots, void *stream) {
  return dense_write(head_dim, num_kv_heads, kBf16Format, pages, num_pages, k, v, dtype, n_tok, slots, stream);
}

int tq_dense_decode_workspace_bytes(int head_dim, int num_kv_heads, int batch, int num_q_heads,
                                    int max_pages_per_seq, int pages_per_split, size_t *out) {
  if (!out) return TQ_EINVAL;
  tq::PageGeom g;
  int st = dense_geom(head_dim, num_kv_heads, false, &g);
  if (st) return st;
  tq::DecodeWs ws;
  st = tq::plan_decode(g, batch, num_q_heads, max_pages_per_seq, pages_per_split, &ws);
  if (st) return st;
  *out = ws.total;
  return TQ_OK;
}

int tq_dense_decode_attention(int head_dim, int num_kv_heads, const void *pages, int64_t num_pages,
                              const void *q, int q_dtype, int batch, int num_q_heads, const int32_t *page_table,
                              int max_pages_per_seq, const int32_t *seq_lens, float softmax_scale,
                              int pages_per_split, void *workspace, size_t workspace_bytes, float *out,
                              void *stream) {
  return dense_decode(head_dim, num_kv_heads, kBf16Format, pages, num_pages, q, q_dtype, batch, num_q_heads,
                      page_table, max_pages_per_seq, seq_lens, softmax_scale, pages_per_split, workspace,
                      workspace_bytes, out, stream);
}

int tq_dense_fp8_page_bytes(int head_dim, int num_kv_heads, size_t *out) {
  return dense_page_bytes(head_dim, num_kv_heads, true, out);
}

int tq_dense_fp8_write_kv(int head_dim, int num_kv_heads, void *pages, int64_t num_pages, const void *k,
                          const void *v, int dtype, int64_t n_tok, const int64_t *slots, float k_scale,
                          float v_scale, void *stream) {
  return dense_write(head_dim, num_kv_heads, tq::DenseFormat{true, k_scale, v_scale}, pages, num_pages, k, v, dtype,
                     n_tok, slots, stream);
}

int tq_dense_fp8_decode_attention(int head_dim, int num_kv_heads, const void *pages, int64_t num_pages,
                                  const void *q, int q_dtype, int batch, int num_q_heads,
                                  const int32_t *page_table, int max_pages_per_seq, const int32_t *seq_lens,
                                  float softmax_scale, float k_scale, float v_scale, int pages_per_split,
                                  void *workspace, size_t workspace_bytes, float *out, void *stream) {
  return dense_decode(head_dim, num_kv_heads, tq::DenseFormat{true, k_scale, v_scale}, pages, num_pages, q, q_dtype,
                      batch, num_q_heads, page_table, max_pages_per_seq, seq_lens, softmax_scale, pages_per_split,
                      workspace, workspace_bytes, out, stream);
}

}  // extern "C"
