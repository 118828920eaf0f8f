// Chunked prefill attention over the packed cache ("Where This Fits in the Inference Stack", "Decode Throughput
// vs. Time to First Token": over long contexts the attention of prefill reads the cache too, and its traffic
// shrinks with it; "Why the KV Cache Exists", "The KV Cache Solution" and "Prefix Caching": the prompt's keys
// and values are stored once and later tokens attend to the stored prefix).
//
// A chunk of C new tokens of each sequence, at positions P_b .. P_b + C - 1, attends causally to the cached
// tokens 0 .. its own position (its own keys and values already written to the pages, quantized). Where the
// decode kernel gives every byte of a page to G query heads, here a work-group of eight wavefronts owns 256 query
// columns (128 with a sketched K) - the (token, head) pairs of 256 / G consecutive tokens of one KV head - so one
// dequantization serves all of them and the contraction runs on the matrix cores:
//   1. Query rotation as in decode (signs, Walsh-Hadamard butterflies, 1/d, a power-of-two range factor per
//      column), the fp16 hi and lo parts of each column kept in registers as MFMA operands.
//   2. Steps of 32 keys (two pages), in two groups of four wavefronts half a step apart: while one group's
//      wavefronts run a matrix phase the other's run the softmax, on the same SIMDs, with a barrier between phases.
//        matrix phase M_j: values O^T[coordinates, columns] += Vhat^T P'^T of step j - 1 (P' = p * ||v|| as fp16
//                hi + lo, each column's weights shifted by a power of two that keeps them in the fp16 range);
//                scores S^T[16 keys, 16 columns] = Khat Q of step j on MFMA 16x16x32 f16 (hi and lo query parts),
//                plus for a sketched K gamma * <q_s, z> from a tile of the keys' sketch signs; and the group's
//                share of the table lookups: group 0 stores step j's V levels, group 1 step j + 1's K levels
//                and norms, into double-buffered LDS tiles (K as [key][coordinate], V as [coordinate][key] in
//                the key order of the softmax operand), from codes loaded one matrix phase earlier;
//        vector phase V_j: the scores times the key norms, the causal mask (only on steps that reach past a
//                column's position), the running maximum per column (base 2), the weights, their sums and the
//                value weights P' for the next matrix phase.
//   3. Each column's sums divided by its total weight, the inverse rotation by butterflies, fp32 rows out.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "tq_common.h"
#include "tq_internal.h"
#include "tq_lanes.h"
#include "tq_operands.h"

namespace tq {

struct PrefillArgs {
  const unsigned char *pages;
  int num_pages32;  // min(num_pages, INT32_MAX)
  int64_t page_bytes;
  int64_t k_codes, k_norms, v_codes, v_norms;
  int64_t k_qjl, k_gamma;  // prod-mode K: sketch bits and residual norms
  const void *q;  // [B][C][Hq][D]
  int q_dtype;
  int B, C, Hq, Hkv, G, TQ;  // TQ: query tokens per work-group (query columns per work-group / G)
  int tiles;                 // work-groups along the chunk (ceil(C / TQ))
  const int32_t *page_table;
  int max_pages;
  const int32_t *prefix_lens;
  float scale_log2;
  const unsigned char *kcb, *vcb;
  BlobOffsets ko, vo;
  float *out;  // [B][C][Hq][D]
};

namespace {

constexpr int kWavesP = 8;
constexpr int kThreadsP = 64 * kWavesP;
constexpr int kBlocksPerCU = 1;       // work-groups per CU the register budget is set for

// 16-column MFMA blocks of query columns per wavefront: two, or one with a sketched K (whose second query
// operand takes the registers of the second block)
__host__ __device__ constexpr int col_blocks(bool kprod) { return kprod ? 1 : 2; }
__host__ __device__ constexpr int cols_per_group(bool kprod) { return 16 * col_blocks(kprod) * kWavesP; }
constexpr int kStepKeys = 32;         // keys per step: two pages
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kHeadroomP = 4.0f;    // log2 units between a column's running maximum and its weight reference
// a column's running maximum before its first visible key: finite, so that a masked score (-inf) weighs
// exp2(-inf) = 0 and the first rescale factor exp2(kNoMaxP - m) underflows to 0
constexpr float kNoMaxP = -1.0e30f;

typedef _Float16 half4p_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f4at(const float4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
// largest of eight values as three 3-input maxima and one 2-input
__device__ __forceinline__ float max8(const float (&v)[2][4]) {
  const float a = fmaxf(fmaxf(v[0][0], v[0][1]), v[0][2]);
  const float b = fmaxf(fmaxf(a, v[0][3]), v[1][0]);
  const float c = fmaxf(fmaxf(b, v[1][1]), v[1][2]);
  return fmaxf(c, v[1][3]);
}

// LDS of one work-group: the double-buffered level tiles of a step, or (prologue, epilogue) one
// [16][D + 4] fp32 staging block per wavefront.
template <int D, bool KPROD>
struct Tiles {
  _Float16 k[2][kStepKeys][D + 8];  // K levels [key][coordinate]; rows padded so 16 keys hit distinct banks
  _Float16 v[2][D][kStepKeys + 8];  // V levels [coordinate][k'], k' = 8 g + 4 q2 + j <-> key 16 q2 + 4 g + j
  // the step's fp16 norms, widened once by the lane that stores them; buffer step % 2, or step % 3 with a sketched
  // K (whose norms are stored two steps ahead)
  float nk[3][kStepKeys], nv[3][kStepKeys];
  // sketched K: the sketch as fp16 -1 / +1 [key][coordinate], and the fp16 residual norms
  _Float16 z[KPROD ? 2 : 1][KPROD ? kStepKeys : 1][D + 8];
  float gm[3][kStepKeys];
};
template <int D, bool KPROD>
union PrefillLds {
  Tiles<D, KPROD> t;
  float stage[kWavesP][16][D + 4];
};

// Per-thread registers of one step's loads: K codes of 8 keys' coordinate chunk, V codes of 4 slots of one
// piece, one norm.
template <int D, int KB, int VB>
struct StepRegs {
  static constexpr int KBYTES = KB * D / 64;              // bytes of the thread's D/8 K codes
  static constexpr int KW = (KBYTES % 4 == 0) ? KBYTES / 4 : (KBYTES + 3) / 4 + 1;  // dwords covering them
  uint32_t kw[KW];
  uint32_t vw[VB];  // 4 slots x VB bytes
  uint32_t norm;
  uint32_t zb;  // sketched K: the D / 8 sketch bits of the K chunk
};

// Dwords [off / 4, off / 4 + N) of a page through a buffer resource (zero-size for a missing page).
template <int N>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *w) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 t = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0));
      w[4 * i] = t.x;
      w[4 * i + 1] = t.y;
      w[4 * i + 2] = t.z;
      w[4 * i + 3] = t.w;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint2 t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off + 8 * i, 0, 0));
      w[2 * i] = t.x;
      w[2 * i + 1] = t.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, 0);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const PrefillArgs &a, int pg) {
  const bool ok = pg >= 0 && pg < a.num_pages32;
  return __builtin_amdgcn_make_buffer_rsrc((void *)(a.pages + (int64_t)(ok ? pg : 0) * a.page_bytes), (short)0,
                                           ok ? (int)a.page_bytes : 0, 0x00020000);
}

// NB bits at bit offset `bit` of a little-endian dword array (NB <= 8, the field may straddle two dwords).
template <int NB, int NW>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[NW], int bit) {
  const int i = bit >> 5, s = bit & 31;
  const uint32_t lo = w[i];
  const uint32_t hi = (i + 1 < NW) ? w[i + 1] : 0u;
  return __builtin_amdgcn_alignbit(hi, lo, s) & ((1u << NB) - 1u);
}

// Coordinate (inside its 8-coordinate group) of K-tile position p: 4-bit codes are looked up eight at a time
// in the MFMA order of lut_k4, the other widths are stored in coordinate order.
template <int KB>
__device__ __forceinline__ constexpr int kpos(int p) {
  return KB == 4 ? k_order<4>(p) : p;
}

template <int D, int KB, bool KPROD, int VB>
__global__ __launch_bounds__(kThreadsP, kBlocksPerCU) void prefill_kernel(PrefillArgs a) {
  constexpr int kNQ = col_blocks(KPROD);
  constexpr int KBLK = D / 32;  // 32-coordinate blocks of the score contraction
  constexpr int NB = D / 16;    // 16-coordinate blocks of the value contraction
  constexpr int KREC = D * KB / 8;
  constexpr int CPT = D / 32;   // V coordinates per thread and step
  constexpr int NH = 8 / CPT;   // threads per (piece, group) of one page
  using R = StepRegs<D, KB, VB>;

  __shared__ __align__(16) PrefillLds<D, KPROD> lds;
  __shared__ uint16_t s_lutk[1 << KB], s_lutv[1 << VB];
  __shared__ float s_sig[kWavesP][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15;
  const int g4 = lane >> 4;

  // work item: consecutive items (tiles of one KV head) go to one XCD when the grid divides evenly
  int item = blockIdx.x;
  {
    const int total = gridDim.x;
    if ((total & 7) == 0) item = (item & 7) * (total >> 3) + (item >> 3);
  }
  const int tile = item % a.tiles;
  const int kvh = (item / a.tiles) % a.Hkv;
  const int b = item / (a.tiles * a.Hkv);
  const int G = a.G;
  const int i0 = tile * a.TQ;
  const int ntok = min(a.TQ, a.C - i0);
  const int kmax = a.max_pages * TQ_PAGE_TOKENS;
  int P = a.prefix_lens[b];
  P = P < 0 ? 0 : P;
  const int kend = min(P + i0 + ntok, kmax);  // keys [0, kend) are visible to some column of this work-group
  const int nsteps = kend > 0 ? (kend + kStepKeys - 1) / kStepKeys : 0;
  const int32_t *ptab = a.page_table + (int64_t)b * a.max_pages;

  // level tables (code-indexed: code c -> ascending level c in the upper half, half - 1 - c in the lower)
  {
    const int nk = 1 << KB, nv = 1 << VB;
    for (int i = tid; i < nk; i += kThreadsP)
      s_lutk[i] = ((const uint16_t *)(a.kcb + a.ko.levels))[i >= nk / 2 ? i : nk / 2 - 1 - i];
    for (int i = tid; i < nv; i += kThreadsP)
      s_lutv[i] = ((const uint16_t *)(a.vcb + a.vo.levels))[i >= nv / 2 ? i : nv / 2 - 1 - i];
  }

  // ---- 1. query columns: column j = 16 kNQ wave + 16 nq + c is token i0 + j / G, head kvh * G + j % G
  half8_t qhi[kNQ][KBLK], qlo[kNQ][KBLK];
  // sketched K: q_s = S (R q) sqrt(pi/2) / m as a second operand, with its own range factor (skratio = the
  // ratio of the two factors)
  half8_t shi[KPROD ? kNQ : 1][KPROD ? KBLK : 1], slo[KPROD ? kNQ : 1][KPROD ? KBLK : 1];
  float skratio[kNQ];
  float colscale[kNQ];
  int lim[kNQ];  // last visible key of the lane's column (-1: a column with no query)
  {
    const uint32_t *ksw = (const uint32_t *)(a.kcb + a.ko.signs);
    const bool neg0 = (ksw[lane >> 5] >> (lane & 31)) & 1u;
    const bool neg1 = D == 128 ? ((ksw[(lane + 64) >> 5] >> (lane & 31)) & 1u) : false;
    float(*st)[D + 4] = lds.stage[wave];
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      // the 16 rows of this block, raw bits, into registers first (independent loads in flight; the dtype
      // is the same for every row, so one branch)
      uint32_t x0[16], x1[16];
      auto row_base = [&](int r, bool &real) {
        const int j = 16 * kNQ * wave + 16 * nq + r;
        const int i = i0 + j / G;
        real = j < a.TQ * G && i < a.C;
        return (((int64_t)b * a.C + (real ? i : 0)) * a.Hq + kvh * G + j % G) * D;
      };
      if (a.q_dtype == TQ_F32) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          bool real;
          const uint32_t *row = (const uint32_t *)a.q + row_base(r, real);
          x0[r] = real ? row[lane] : 0u;
          x1[r] = (real && D == 128) ? row[lane + 64] : 0u;
        }
      } else {
        const bool bf = a.q_dtype == TQ_BF16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          bool real;
          const uint16_t *row = (const uint16_t *)a.q + row_base(r, real);
          const uint32_t u0 = real ? row[lane] : 0u;
          const uint32_t u1 = (real && D == 128) ? row[lane + 64] : 0u;
          x0[r] = bf ? u0 << 16 : __float_as_uint(half_bits_to_float((uint16_t)u0));
          x1[r] = bf ? u1 << 16 : __float_as_uint(half_bits_to_float((uint16_t)u1));
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float y0 = __uint_as_float(x0[r] ^ (neg0 ? 0x80000000u : 0u));
        float y1 = __uint_as_float(x1[r] ^ (neg1 ? 0x80000000u : 0u));
        y0 = wht_stage<1>(y0, lane);
        y1 = wht_stage<1>(y1, lane);
        y0 = wht_stage<2>(y0, lane);
        y1 = wht_stage<2>(y1, lane);
        y0 = wht_stage<4>(y0, lane);
        y1 = wht_stage<4>(y1, lane);
        y0 = wht_stage<8>(y0, lane);
        y1 = wht_stage<8>(y1, lane);
        y0 = wht_stage<16>(y0, lane);
        y1 = wht_stage<16>(y1, lane);
        y0 = wht_stage<32>(y0, lane);
        y1 = wht_stage<32>(y1, lane);
        if (D == 128) {
          const float u = y0;
          y0 = u + y1;
          y1 = u - y1;
        }
        y0 *= (1.0f / D);
        y1 *= (1.0f / D);
        const float mx = wave_max(fmaxf(fabsf(y0), D == 128 ? fabsf(y1) : 0.f), lane);
        st[r][lane] = y0;
        if (D == 128) st[r][lane + 64] = y1;
        if (lane == 0) s_sig[wave][r] = range_factor(mx);
      }
      __syncthreads();
      {
        const int j = 16 * kNQ * wave + 16 * nq + c;
        const int i = i0 + j / G;
        const bool real = j < a.TQ * G && i < a.C;
        const float sig = s_sig[wave][c];
        // at least the smallest normal float: a masked score (-inf) times the factor stays -inf, never NaN; with a
        // softmax scale of 0 the factor times any score is far below an ulp of the weight reference
        colscale[nq] = fmaxf(real ? a.scale_log2 / sig : 0.f, 1.17549435e-38f);
        lim[nq] = real ? min(P + i, kmax - 1) : -1;
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) {
          const float4 u0 = *(const float4 *)&st[c][32 * kb + 8 * g4];
          const float4 u1 = *(const float4 *)&st[c][32 * kb + 8 * g4 + 4];
          const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
          half8_t lo8;
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            _Float16 h, l;
            split_hi_lo(real ? v[kpos<KB>(p)] * sig : 0.f, h, l);
            qhi[nq][kb][p] = h;
            lo8[p] = l;
          }
          qlo[nq][kb] = lo8;
        }
        skratio[nq] = 0.f;
        if constexpr (KPROD) {
          // the lane's 8 * KBLK coordinates j = 32 kb + 8 g4 + p of column c: rows j of S times the column
          const float *S = (const float *)(a.kcb + a.ko.proj);
          const float cq = 1.2533141373155003f / (float)a.ko.qjl_rows * (float)D *
                           (D == 128 ? 0.088388347648318440f : 0.125f);
          float qs[KBLK][8];
          float mx = 0.f;
#pragma unroll
          for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              const float4 *srow = (const float4 *)(S + (int64_t)(32 * kb + 8 * g4 + p) * D);
              float acc = 0.f;
#pragma unroll 8
              for (int k4 = 0; k4 < D / 4; ++k4) {
                const float4 sv = srow[k4];
                const float4 xv = *(const float4 *)&st[c][4 * k4];
                acc = fmaf(sv.x, xv.x, fmaf(sv.y, xv.y, fmaf(sv.z, xv.z, fmaf(sv.w, xv.w, acc))));
              }
              qs[kb][p] = acc * cq;
              mx = fmaxf(mx, fabsf(qs[kb][p]));
            }
          mx = max_xor32(max_xor16(mx));  // over the four lanes of column c
          const float sig2 = range_factor(mx);
          skratio[nq] = real ? sig / sig2 : 0.f;
#pragma unroll
          for (int kb = 0; kb < KBLK; ++kb) {
            half8_t h8, l8;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
              _Float16 h, l;
              split_hi_lo(real ? qs[kb][p] * sig2 : 0.f, h, l);
              h8[p] = h;
              l8[p] = l;
            }
            shi[nq][kb] = h8;
            slo[nq][kb] = l8;
          }
        }
      }
      __syncthreads();  // the staging block is rewritten by the next block (and then by the level tiles)
    }
  }
  // ---- 2. the key steps, in two wavefront groups half a step apart. Each group alternates between a matrix
  // phase M_j (the value sums of step j - 1, the scores of step j, and the group's share of the tile lookups) and
  // a vector phase V_j (the softmax of step j); group 1 runs one phase behind group 0, so on every SIMD one
  // wavefront issues MFMAs and table lookups while the other runs the softmax, and a barrier between phases keeps
  // the offset. In M_j group 0 builds the V tile of step j, group 1 the K tile and the norms of step j + 1; tile j
  // (K, V, norms) lives in buffer j & 1, which is rewritten only after both groups have read its previous content.
  // With a sketched K the lookups move to the vector phases (group 0: V tile j in V_j; group 1: K tile j + 2 in
  // V_j) and the norms to buffer j % 3 (the loops below).
  const int grp = wave >> 2;
  const int lw = wave & 3;
  const int t = tid & 255;
  Tab tk{0, 0, 0, 0}, tv{0, 0, 0, 0};
  if constexpr (KB == 4) tk = make_tab_k4(s_lutk);
  if constexpr (VB == 2) tv = make_tab_v2(s_lutv);
  // thread roles of the loads. Group 1: K codes of key kk (page kk / 16 = lw / 2), coordinate chunk kc;
  // norms (its wavefronts 0 and 2, lanes 0..31, 0..47 with a sketched K): K (lanes < 16), V (16..31) or
  // residual (32..47) norm of slot lane % 16 of page lw / 2. Group 0: V codes of piece vp, slot group vg,
  // coordinates CPT vh .. of page lw / 2.
  const int kk = t >> 3, kc = t & 7;
  const int pq = lw >> 1;
  const int vt = t & 127;
  const int vp = vt / (4 * NH), vg = (vt / NH) & 3, vh = vt % NH;
  const uint32_t k_off = (uint32_t)(a.k_codes + (int64_t)(kvh * TQ_PAGE_TOKENS + (kk & 15)) * KREC) +
                         (uint32_t)(kc * R::KBYTES);
  const uint32_t k_off_al = k_off & ~3u;
  const int k_bit0 = 8 * (int)(k_off & 3u);
  const uint32_t v_off = (uint32_t)(a.v_codes + ((int64_t)(kvh * (D / 8) + vp) * TQ_PAGE_TOKENS + 4 * vg) * VB);
  const bool norm_lane = (lw & 1) == 0 && lane < (KPROD ? 48 : 32);
  const uint32_t n_off = (uint32_t)((lane < 16 ? a.k_norms : (lane < 32 ? a.v_norms : a.k_gamma)) +
                                    (int64_t)(kvh * TQ_PAGE_TOKENS + (lane & 15)) * 2);
  const uint32_t z_off = (uint32_t)(a.k_qjl + (int64_t)(kvh * TQ_PAGE_TOKENS + (kk & 15)) * (D / 8)) +
                         (uint32_t)(kc * (D / 64));

  auto page_id = [&](int pi) { return pi < a.max_pages ? ptab[pi] : -1; };
  auto page_ok = [&](int pg) { return pg >= 0 && pg < a.num_pages32; };

  R rg;
  auto load_k = [&](int st) __attribute__((always_inline)) {  // group 1: step st's K codes, norms (and sketch bits)
    const __amdgpu_buffer_rsrc_t r = page_rsrc(a, page_id(2 * st + pq));
    load_dwords<R::KW>(r, k_off_al, rg.kw);
    rg.norm = norm_lane ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, n_off & ~1u, 0, 0) : 0u;
    rg.zb = 0u;
    if constexpr (KPROD) {
      if constexpr (D == 128) rg.zb = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, z_off, 0, 0);
      else rg.zb = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, z_off, 0, 0);
    }
  };
  auto load_v = [&](int st) __attribute__((always_inline)) {  // group 0: step st's V codes
    const __amdgpu_buffer_rsrc_t r = page_rsrc(a, page_id(2 * st + pq));
    load_dwords<VB>(r, v_off, rg.vw);
  };
  auto store_k = [&](int st) __attribute__((always_inline)) {  // step st's K tile and norms
    const int buf = st & 1, nbuf = KPROD ? st % 3 : st & 1;
    // D / 8 levels of key kk (4-bit codes: byte-table lookups, eight at a time; other widths: the codes
    // shifted down to bit 0, so every field offset is fixed, and one table read each)
    if constexpr (KB == 4) {
#pragma unroll
      for (int i = 0; i < D / 64; ++i) *(half8_t *)&lds.t.k[buf][kk][kc * (D / 8) + 8 * i] = lut_k4(rg.kw[i], tk);
    } else {
      uint32_t kw[R::KW];
#pragma unroll
      for (int i = 0; i < R::KW; ++i)
        kw[i] = __builtin_amdgcn_alignbit(i + 1 < R::KW ? rg.kw[i + 1] : 0u, rg.kw[i], k_bit0);
      _Float16 h[D / 8];
#pragma unroll
      for (int i = 0; i < D / 8; ++i) {
        const uint16_t bits = s_lutk[field<KB, R::KW>(kw, KB * i)];
        h[i] = __builtin_bit_cast(_Float16, bits);
      }
#pragma unroll
      for (int i = 0; i < D / 64; ++i) {
        half8_t t8;
#pragma unroll
        for (int p = 0; p < 8; ++p) t8[p] = h[8 * i + p];
        *(half8_t *)&lds.t.k[buf][kk][kc * (D / 8) + 8 * i] = t8;
      }
    }
    if (norm_lane) {
      const int key = 16 * pq + (lane & 15);
      const float nf = half_bits_to_float((uint16_t)rg.norm);
      if (lane < 16) lds.t.nk[nbuf][key] = nf;
      else if (lane < 32) lds.t.nv[nbuf][key] = nf;
      else lds.t.gm[nbuf][key] = nf;
    }
    if constexpr (KPROD) {
      // sketch bit set: +1 (0x3C00), clear: -1 (0xBC00), coordinate order
#pragma unroll
      for (int i = 0; i < D / 64; ++i) {
        half8_t t8;
#pragma unroll
        for (int p = 0; p < 8; ++p)
          t8[p] = __builtin_bit_cast(_Float16, (uint16_t)(((rg.zb >> (8 * i + p)) & 1u) ? 0x3C00u : 0xBC00u));
        *(half8_t *)&lds.t.z[buf][kk][kc * (D / 8) + 8 * i] = t8;
      }
    }
  };
  auto store_v = [&](int buf) __attribute__((always_inline)) {
    // CPT coordinates of piece vp for slots 4 vg .. 4 vg + 3 of page pq (2-bit codes: slots 0, 1 and 2, 3 of a
    // coordinate looked up as pairs)
    if constexpr (VB == 2) {
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        const int ci = CPT * vh + e;
        *(uint2 *)&lds.t.v[buf][8 * vp + ci][8 * vg + 4 * pq] =
            uint2{lut_v2_pair(rg.vw[0] >> (2 * ci), tv), lut_v2_pair(rg.vw[1] >> (2 * ci), tv)};
      }
    } else {
      uint32_t w[VB];
#pragma unroll
      for (int i = 0; i < VB; ++i) w[i] = rg.vw[i];
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        const int ci = CPT * vh + e;
        half4p_t t4;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const uint16_t bits = s_lutv[field<VB, VB>(w, 8 * VB * s4 + VB * ci)];
          t4[s4] = __builtin_bit_cast(_Float16, bits);
        }
        *(half4p_t *)&lds.t.v[buf][8 * vp + ci][8 * vg + 4 * pq] = t4;
      }
    }
  };

  float m_run[kNQ], l_part[kNQ];
  float ev[kNQ], wmax[kNQ];  // each column's weight shift and largest value weight (see weight_shift)
  floatx4_t O[kNQ][NB];
#pragma unroll
  for (int nq = 0; nq < kNQ; ++nq) {
    m_run[nq] = kNoMaxP;
    l_part[nq] = 0.f;
    ev[nq] = 0.f;
    wmax[nq] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) O[nq][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  // carried from M_j to V_j: the scores (and the sketch contraction); from V_j to M_{j+1}:
  // the value weights as fp16 hi + lo operands
  floatx4_t acc[2][kNQ], acc2[KPROD ? 2 : 1][kNQ];

  half8_t phi[kNQ], plo[kNQ];
  // the smallest position of the wavefront's columns: steps whose keys all precede it need no causal mask
  const int first_pos = P + i0 + (16 * kNQ * wave) / G;

  auto mphase = [&](int j) __attribute__((always_inline)) {
    if (j >= 1) {  // O^T += Vhat^T P'^T of step j - 1
      const int buf = (j - 1) & 1;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const half8_t Vop = *(const half8_t *)&lds.t.v[buf][16 * nb + c][8 * g4];
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) {
          O[nq][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Vop, phi[nq], O[nq][nb], 0, 0, 0);
          O[nq][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Vop, plo[nq], O[nq][nb], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the value operands' registers are free before the key operands load
    if (j < nsteps) {  // S^T = Khat Q of step j (hi and lo query parts), the step's norms into registers
      const int buf = j & 1;
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq) acc[q2][nq] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) {
          const half8_t A = *(const half8_t *)&lds.t.k[buf][16 * q2 + c][32 * kb + 8 * g4];
#pragma unroll
          for (int nq = 0; nq < kNQ; ++nq) {
            acc[q2][nq] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qhi[nq][kb], acc[q2][nq], 0, 0, 0);
            acc[q2][nq] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qlo[nq][kb], acc[q2][nq], 0, 0, 0);
          }
        }
      if constexpr (KPROD) {  // <q_s, z> for every key
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
#pragma unroll
          for (int nq = 0; nq < kNQ; ++nq) acc2[q2][nq] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KBLK; ++kb) {
            const half8_t Z = *(const half8_t *)&lds.t.z[buf][16 * q2 + c][32 * kb + 8 * g4];
#pragma unroll
            for (int nq = 0; nq < kNQ; ++nq) {
              acc2[q2][nq] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Z, shi[nq][kb], acc2[q2][nq], 0, 0, 0);
              acc2[q2][nq] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Z, slo[nq][kb], acc2[q2][nq], 0, 0, 0);
            }
          }
        }
      }
    }
  };

  // the online softmax of step j: running maximum, weights, value weights P' = p ||v|| as fp16 hi + lo. One body
  // for masked and unmasked steps (full: every key of the step is visible to every column of the wavefront and
  // lies in a valid page); a second copy raises the register pressure past the budget.
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const bool ok0 = page_ok(page_id(2 * j)), ok1 = page_ok(page_id(2 * j + 1));
    const bool full = ok0 && ok1 && kStepKeys * (j + 1) <= first_pos + 1;
    const int nbuf = KPROD ? j % 3 : j & 1;
    float4 nkr[2], nvr[2], gmr[KPROD ? 2 : 1];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      nkr[q2] = *(const float4 *)&lds.t.nk[nbuf][16 * q2 + 4 * g4];
      nvr[q2] = *(const float4 *)&lds.t.nv[nbuf][16 * q2 + 4 * g4];
      if constexpr (KPROD) gmr[q2] = *(const float4 *)&lds.t.gm[nbuf][16 * q2 + 4 * g4];
    }
    if constexpr (KPROD) {
      // the sketch term, times gamma and the ratio of the two range factors, joins the level term before the
      // key norm
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int nq = 0; nq < kNQ; ++nq)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[q2][nq][jj] = fmaf(f4at(gmr[q2], jj) * skratio[nq], acc2[q2][nq][jj], acc[q2][nq][jj]);
    }
#pragma unroll
    for (int nq = 0; nq < kNQ; ++nq) {
      float sc[2][4];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sc[q2][jj] = f4at(nkr[q2], jj) * acc[q2][nq][jj];  // score / (scale log2 e)
      if (!full) {  // keys past a column's position or in a missing page weigh exp2(-inf) = 0
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int key = kStepKeys * j + 16 * q2 + 4 * g4 + jj;
            if (!((q2 ? ok1 : ok0) && key <= lim[nq])) sc[q2][jj] = -INFINITY;
          }
      }
      // the lane's own maximum first; the column's (over its four lanes) only when some lane passes m_run
      const float mxl = max8(sc);
      if (__any(colscale[nq] * mxl > m_run[nq])) {
        const float m_new = colscale[nq] * max_xor32(max_xor16(mxl));
        const bool up = m_new > m_run[nq];
        const float m_ref = up ? m_new + kHeadroomP : m_run[nq];
        const float alpha = up ? fast_exp2(m_run[nq] - m_ref) : 1.f;
        l_part[nq] *= alpha;
        wmax[nq] *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nq][nb] *= alpha;
        m_run[nq] = m_ref;
      }
      // weights against the effective reference m_run - ev, value weights P' = p ||v|| kept in the fp16 range
      const float m_eff = m_run[nq] - ev[nq];
      float pv[2][4];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float p = fast_exp2(fmaf(sc[q2][jj], colscale[nq], -m_eff));
          l_part[nq] += p;
          pv[q2][jj] = f4at(nvr[q2], jj) * p;
        }
      const float pvl = max8(pv);
      wmax[nq] = fmaxf(wmax[nq], pvl);
      if (__any(pvl > kWeightHigh || (wmax[nq] < kWeightLow && pvl > 0.f))) {
        const float f = weight_shift(max_xor32(max_xor16(wmax[nq])), ev[nq], wmax[nq]);
        l_part[nq] *= f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nq][nb] *= f;
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) pv[q2][jj] *= f;
      }
      // hi = fp16(P'), lo = fp16(P' - hi) with the difference taken in fp32 from the fp16 hi (one mixed fma)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int jj = 0; jj < 4; jj += 2) {
          const float2_t pw = {pv[q2][jj], pv[q2][jj + 1]};
          const half2_t h = __builtin_convertvector(pw, half2_t);
          const float2_t r = {fmaf((float)h[0], -1.0f, pw[0]), fmaf((float)h[1], -1.0f, pw[1])};
          const half2_t l = __builtin_convertvector(r, half2_t);
          phi[nq][4 * q2 + jj] = h[0];
          phi[nq][4 * q2 + jj + 1] = h[1];
          plo[nq][4 * q2 + jj] = l[0];
          plo[nq][4 * q2 + jj + 1] = l[1];
        }
    }
  };

  if (nsteps > 0) {
    // Phases 0 .. 2 nsteps + 1, one barrier after each; each group runs its own loop (the two execute the
    // same sequence of barriers). Group 0: M_0, V_0, M_1, .., V_{nsteps-1}, M_nsteps, then one idle phase;
    // group 1 one phase later. The table lookups go where the phases balance: into the matrix phase, or with a
    // sketched K (whose matrix phase is bound by its three LDS operand tiles) into the vector phase. Codes are
    // loaded one phase pair ahead of their lookup. Either way each tile is written in the phase pair before the
    // first matrix phase that reads it, after the last read of its buffer's previous content.
    constexpr bool kLookupsInMatrix = !KPROD;
    if (grp == 0) {
      load_v(0);
      __syncthreads();  // step 0's K tile and norms
      for (int j = 0; j < nsteps; ++j) {
        mphase(j);
        if constexpr (kLookupsInMatrix) {  // V tile j, read from M_{j+1} on
          store_v(j & 1);
          if (j + 1 < nsteps) load_v(j + 1);
        }
        __syncthreads();
        if constexpr (!kLookupsInMatrix) {
          store_v(j & 1);
          if (j + 1 < nsteps) load_v(j + 1);
        }
        softmax(j);
        __syncthreads();
      }
      mphase(nsteps);
      __syncthreads();
      __syncthreads();
    } else {
      load_k(0);
      store_k(0);
      if (nsteps > 1) load_k(1);
      __syncthreads();
      if constexpr (!kLookupsInMatrix) {  // K tile 1 in group 1's first (idle) phase
        if (nsteps > 1) store_k(1);
        if (nsteps > 2) load_k(2);
      }
      __syncthreads();
      for (int j = 0; j < nsteps; ++j) {
        mphase(j);
        if constexpr (kLookupsInMatrix) {  // K tile j + 1, read from group 0's M_{j+1} on
          if (j + 1 < nsteps) store_k(j + 1);
          if (j + 2 < nsteps) load_k(j + 2);
        }
        __syncthreads();
        if constexpr (!kLookupsInMatrix) {  // K tile j + 2
          if (j + 2 < nsteps) store_k(j + 2);
          if (j + 3 < nsteps) load_k(j + 3);
        }
        softmax(j);
        __syncthreads();
      }
      mphase(nsteps);
      __syncthreads();
    }
  }

  // ---- 3. normalise, inverse rotation, fp32 rows
  const uint32_t *vsw = (const uint32_t *)(a.vcb + a.vo.signs);
  const bool vneg0 = (vsw[lane >> 5] >> (lane & 31)) & 1u;
  const bool vneg1 = D == 128 ? ((vsw[(lane + 64) >> 5] >> (lane & 31)) & 1u) : false;
  float(*st)[D + 4] = lds.stage[wave];
#pragma unroll
  for (int nq = 0; nq < kNQ; ++nq) {
    const float L = sum_xor16_32(l_part[nq]);
    const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *(float4 *)&st[c][16 * nb + 4 * g4] =
          float4{O[nq][nb][0] * inv, O[nq][nb][1] * inv, O[nq][nb][2] * inv, O[nq][nb][3] * inv};
    __syncthreads();
    for (int r = 0; r < 16; ++r) {
      const int j = 16 * kNQ * wave + 16 * nq + r;
      const int i = i0 + j / G;
      if (!(j < a.TQ * G && i < a.C)) continue;  // wavefront-uniform
      float y0 = st[r][lane];
      float y1 = D == 128 ? st[r][lane + 64] : 0.f;
      y0 = wht_stage<1>(y0, lane);
      y1 = wht_stage<1>(y1, lane);
      y0 = wht_stage<2>(y0, lane);
      y1 = wht_stage<2>(y1, lane);
      y0 = wht_stage<4>(y0, lane);
      y1 = wht_stage<4>(y1, lane);
      y0 = wht_stage<8>(y0, lane);
      y1 = wht_stage<8>(y1, lane);
      y0 = wht_stage<16>(y0, lane);
      y1 = wht_stage<16>(y1, lane);
      y0 = wht_stage<32>(y0, lane);
      y1 = wht_stage<32>(y1, lane);
      if (D == 128) {
        const float u = y0;
        y0 = u + y1;
        y1 = u - y1;
      }
      y0 *= (1.0f / D);
      y1 *= (1.0f / D);
      float *orow = a.out + (((int64_t)b * a.C + i) * a.Hq + kvh * G + j % G) * D;
      orow[lane] = vneg0 ? -y0 : y0;
      if (D == 128) orow[lane + 64] = vneg1 ? -y1 : y1;
    }
    __syncthreads();
  }
}

template <int D, int KB, bool KPROD>
bool prefill_dispatch_v(int vb, const PrefillArgs &a, dim3 grid, hipStream_t s) {
  switch (vb) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, KB, KPROD, 1>), grid, dim3(kThreadsP), 0, s, a); return true;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, KB, KPROD, 2>), grid, dim3(kThreadsP), 0, s, a); return true;
    case 3: hipLaunchKernelGGL((prefill_kernel<D, KB, KPROD, 3>), grid, dim3(kThreadsP), 0, s, a); return true;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, KB, KPROD, 4>), grid, dim3(kThreadsP), 0, s, a); return true;
    case 8: hipLaunchKernelGGL((prefill_kernel<D, KB, KPROD, 8>), grid, dim3(kThreadsP), 0, s, a); return true;
    default: return false;
  }
}

template <int D>
bool prefill_dispatch(int kb, bool kprod, int vb, const PrefillArgs &a, dim3 grid, hipStream_t s) {
  if (kprod) {  // MSE parts of a sketched K: 1 to 3 bits
    switch (kb) {
      case 1: return prefill_dispatch_v<D, 1, true>(vb, a, grid, s);
      case 2: return prefill_dispatch_v<D, 2, true>(vb, a, grid, s);
      case 3: return prefill_dispatch_v<D, 3, true>(vb, a, grid, s);
      default: return false;
    }
  }
  switch (kb) {
    case 1: return prefill_dispatch_v<D, 1, false>(vb, a, grid, s);
    case 2: return prefill_dispatch_v<D, 2, false>(vb, a, grid, s);
    case 3: return prefill_dispatch_v<D, 3, false>(vb, a, grid, s);
    case 4: return prefill_dispatch_v<D, 4, false>(vb, a, grid, s);
    case 8: return prefill_dispatch_v<D, 8, false>(vb, a, grid, s);
    default: return false;
  }
}

}  // namespace

int launch_prefill(const PageGeom &g, const void *pages, int64_t num_pages, const void *q, int q_dtype, int batch,
                   int chunk_len, int num_q_heads, const int32_t *page_table, int max_pages_per_seq,
                   const int32_t *prefix_lens, float softmax_scale, const void *k_cb, const void *v_cb, float *out,
                   hipStream_t stream) {
  if (g.v_mode != TQ_MSE) return TQ_ENOTSUP;
  const bool kprod = g.k_mode == TQ_PROD;
  PrefillArgs a;
  a.pages = (const unsigned char *)pages;
  a.num_pages32 = (int)std::min<int64_t>(num_pages, 0x7FFFFFFF);
  a.page_bytes = g.page_bytes;
  a.k_codes = g.k_codes;
  a.k_norms = g.k_norms;
  a.v_codes = g.v_codes;
  a.v_norms = g.v_norms;
  a.k_qjl = g.k_qjl;
  a.k_gamma = g.k_gamma;
  a.q = q;
  a.q_dtype = q_dtype;
  a.B = batch;
  a.C = chunk_len;
  a.Hq = num_q_heads;
  a.Hkv = g.num_kv_heads;
  a.G = num_q_heads / g.num_kv_heads;
  a.TQ = cols_per_group(kprod) / a.G;
  a.tiles = (chunk_len + a.TQ - 1) / a.TQ;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.prefix_lens = prefix_lens;
  a.scale_log2 = softmax_scale * kLog2eP;
  a.kcb = (const unsigned char *)k_cb;
  a.vcb = (const unsigned char *)v_cb;
  a.ko = g.kcb;
  a.vo = g.vcb;
  a.out = out;
  const int64_t items = (int64_t)a.tiles * a.Hkv * batch;
  if (items > 0x7FFFFFFF) return TQ_EINVAL;
  const dim3 grid((unsigned)items);
  const bool ok = g.head_dim == 128 ? prefill_dispatch<128>(g.k_mse_bits, kprod, g.v_mse_bits, a, grid, stream)
                                    : prefill_dispatch<64>(g.k_mse_bits, kprod, g.v_mse_bits, a, grid, stream);
  if (!ok) return TQ_ENOTSUP;
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EHIP;
}

}  // namespace tq
