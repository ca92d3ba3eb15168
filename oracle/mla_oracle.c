/*
 * mla_oracle.c -- plain float64 CPU oracle for Multi-head Latent Attention (MLA)
 * decoding over a paged latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file exists to check the GPU path.  Only the
 * test suite, the smoke check of the package entry point and the CPU-baseline leg
 * of the benchmark may load it.  The product path never links, imports or calls
 * anything here, and nothing here is shared with the GPU sources (no common
 * header, helper, table or constant generator).
 *
 * What it computes (sources are the FlashMLA pages):
 *   - "FlashMLA: DeepSeek's efficient MLA decoding kernel" (geoz.com.cn), usage
 *     example section: decode takes q, the paged KV cache, block_table and
 *     cache_seqlens and returns o and lse; the paged cache uses 64-token blocks
 *     (main features section).
 *   - "FlashMLA attention kernel source walk-through: the 656-byte KV cache"
 *     (bjdmk.com.cn):
 *       * data-loading section: a token is 576 dims; the first 512 are stored as
 *         e4m3 with 1x128 tile scales, the last 64 are RoPE dims kept in bf16; the
 *         kernel dequantises to bf16, concatenates, and multiplies in bf16 with
 *         fp32 accumulation (so the FP8 latent the attention sees is bf16);
 *       * scheduling section: long sequences are cut into splits computed
 *         separately;
 *       * combine section: each split leaves a partial o and lse, merged with lse.
 *   - gitgenius.co FlashMLA summary: the FP8 token holds 512 bytes of quantised
 *     values, 16 bytes of scale factors and 128 bytes of unquantised RoPE.
 *   - agentlenshq.com FlashMLA summary, technical details: sparse indices are
 *     3-D int32, and -1 entries are ignored.
 *
 * The definition, for one query row (request b, query token s, head h):
 *   T      = [0, seqlen_b) for the dense cache, else the multiset of
 *            indices[b, s, k] (k < topk) that are not -1;
 *   K_j    = the 576-dim latent of logical token j, found at
 *            page block_table[b, j / 64], row j % 64;
 *   s_j    = scale * <q, K_j>;
 *   lse    = log(sum_j exp(s_j))        (natural log; -inf when T is empty)
 *   o      = sum_j exp(s_j - lse) * K_j[0:512]   (0 when T is empty)
 * evaluated in float64 with inputs widened exactly from their stored bytes.
 *
 * Readings taken where the pages are silent (each stated once, here):
 *   - lse is the natural log-sum-exp of the scaled scores;
 *   - an empty attended set gives o = 0 and lse = -inf;
 *   - duplicate indices count with multiplicity;
 *   - decode is non-causal by default: every query token of a request sees all
 *     seqlen_b tokens (dense) or its own index list (sparse);
 *   - with the causal flag (the usage example passes causal=True for
 *     autoregressive decoding; geoz.com.cn, usage example section) the dense
 *     mask is aligned to the end of the cache: the s_q query tokens are the
 *     last s_q positions, so query token s sees positions
 *     j <= seqlen_b - s_q + s (an empty set when that is negative); the flag is
 *     not defined for sparse decoding, whose index lists already decide what
 *     each query token sees;
 *   - sparse indices are logical token positions translated through
 *     block_table;
 *   - FP8 byte layout: byte d (d < 512) holds dim d as OCP e4m3fn; bytes
 *     512..527 hold four little-endian fp32 scales, scale t covering dims
 *     [128 t, 128 t + 128); bytes 528..655 hold dims 512..575 as little-endian
 *     bf16.
 *
 * The split/tile schedule rule at the bottom is this project's own design (the
 * pages only say that work units are spread evenly ahead of time); it is
 * written out plainly here so the GPU scheduler can be compared with it
 * bit for bit.  Parity for it is pinned by coverage and balance properties only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_D_QK 576
#define ORACLE_D_V 512
#define ORACLE_PAGE_TOKENS 64
#define ORACLE_FP8_DIMS 512
#define ORACLE_FP8_TILE 128

/* ---- stored-format widening ------------------------------------------------ */

/* bf16 -> float64, exact: a bf16 is the top half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* little-endian binary32 at p -> float64, exact. */
static double le_f32_to_f64(const uint8_t* p) {
  uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * OCP FP8 E4M3 ("fn" flavour) -> float64.  Format definition: 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
 * subnormals m/8 * 2^-6; there is no infinity; S.1111.111 is NaN, so the
 * largest finite magnitude is 1.75 * 2^8 = 448.
 */
double oracle_e4m3fn_to_f64(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Bytes one token occupies in the cache: 576 bf16, or 512 + 16 + 128 for FP8. */
int64_t oracle_token_bytes(int is_fp8) {
  return is_fp8 ? (int64_t)ORACLE_FP8_DIMS + 4 * 4 + (ORACLE_D_QK - ORACLE_FP8_DIMS) * 2
                : (int64_t)ORACLE_D_QK * 2;
}

/* ---- FP8 element -> the bf16 value the matrix multiply uses ---------------- */

/*
 * Dequantisation of one FP8 element.  The source walk-through (data-loading
 * section) has the kernel turn the 512 FP8 values back into bfloat16 and run
 * the matrix multiplies in bf16, so the latent the attention sees is a bf16
 * value.  Reading of the rounding: widen e4m3 to binary32 (exact), multiply by
 * the binary32 scale with round-to-nearest-even, then round the binary32
 * product to bf16 with round-to-nearest-even.  NaN stays NaN (quiet).
 */
uint16_t oracle_fp8_dequant_bf16(uint8_t code, float scale) {
  float v = (float)oracle_e4m3fn_to_f64(code);
  volatile float p = v * scale; /* binary32 multiply, round to nearest even */
  float pf = p;
  uint32_t u;
  memcpy(&u, &pf, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) return (uint16_t)((u >> 16) | 0x0040u);
  {
    uint32_t lsb = (u >> 16) & 1u;
    uint32_t rounded = u + 0x7FFFu + lsb;
    return (uint16_t)(rounded >> 16);
  }
}

/*
 * The 576-dim latent of one stored token, widened to float64.
 * FP8: K[d] = bf16(fp32(e4m3(byte d) * scale[d / 128])) for d < 512 (the
 * dequantised value above), and the RoPE dims are the stored bf16 values.
 */
void oracle_token_latent(const uint8_t* token, int is_fp8, double* k) {
  int d;
  if (!is_fp8) {
    for (d = 0; d < ORACLE_D_QK; ++d) {
      uint16_t b = (uint16_t)(token[2 * d] | (token[2 * d + 1] << 8));
      k[d] = oracle_bf16_to_f64(b);
    }
    return;
  }
  for (d = 0; d < ORACLE_FP8_DIMS; ++d) {
    float scale = (float)le_f32_to_f64(token + ORACLE_FP8_DIMS + 4 * (d / ORACLE_FP8_TILE));
    k[d] = oracle_bf16_to_f64(oracle_fp8_dequant_bf16(token[d], scale));
  }
  for (d = ORACLE_FP8_DIMS; d < ORACLE_D_QK; ++d) {
    const uint8_t* r = token + ORACLE_FP8_DIMS + 16 + 2 * (d - ORACLE_FP8_DIMS);
    k[d] = oracle_bf16_to_f64((uint16_t)(r[0] | (r[1] << 8)));
  }
}

/* Where logical token j of a request lives: page block_table_row[j / 64], row j % 64. */
static const uint8_t* token_address(const uint8_t* kvcache, int is_fp8, const int32_t* block_table_row, int64_t j) {
  int64_t page = block_table_row[j / ORACLE_PAGE_TOKENS];
  int64_t row = j % ORACLE_PAGE_TOKENS;
  return kvcache + (page * ORACLE_PAGE_TOKENS + row) * oracle_token_bytes(is_fp8);
}

/* ---- attention for one query row over an explicit list of positions ------- */

/*
 * softmax(scale * q K^T) over the listed positions, then P V with V = K[:, :512];
 * returns lse = log sum exp(scores).  n == 0 gives o = 0, lse = -inf.
 */
void oracle_attend(const uint16_t* q_row, const uint8_t* kvcache, int is_fp8, const int32_t* block_table_row,
                   const int64_t* pos, int64_t n, double scale, double* o, double* lse) {
  double q[ORACLE_D_QK], k[ORACLE_D_QK];
  double* s;
  double mx, sum;
  int64_t j;
  int d;
  for (d = 0; d < ORACLE_D_V; ++d) o[d] = 0.0;
  if (n == 0) {
    *lse = -INFINITY;
    return;
  }
  for (d = 0; d < ORACLE_D_QK; ++d) q[d] = oracle_bf16_to_f64(q_row[d]);
  s = (double*)malloc(sizeof(double) * (size_t)n);
  for (j = 0; j < n; ++j) {
    double dot = 0.0;
    oracle_token_latent(token_address(kvcache, is_fp8, block_table_row, pos[j]), is_fp8, k);
    for (d = 0; d < ORACLE_D_QK; ++d) dot += q[d] * k[d];
    s[j] = scale * dot;
  }
  mx = -INFINITY;
  for (j = 0; j < n; ++j)
    if (s[j] > mx) mx = s[j];
  sum = 0.0;
  for (j = 0; j < n; ++j) sum += exp(s[j] - mx);
  *lse = mx + log(sum);
  for (j = 0; j < n; ++j) {
    double p = exp(s[j] - *lse);
    oracle_token_latent(token_address(kvcache, is_fp8, block_table_row, pos[j]), is_fp8, k);
    for (d = 0; d < ORACLE_D_V; ++d) o[d] += p * k[d];
  }
  free(s);
}

/*
 * Merge of per-split results by their lse (combine section of the source
 * walk-through): L = log sum_i exp(lse_i), o = sum_i exp(lse_i - L) o_i.
 * Parts with lse = -inf carry no weight; if every part is -inf the result is
 * o = 0, lse = -inf.
 */
void oracle_lse_combine(int64_t n_parts, const double* o_parts, const double* lse_parts, double* o, double* lse) {
  double mx = -INFINITY, sum = 0.0;
  int64_t i;
  int d;
  for (d = 0; d < ORACLE_D_V; ++d) o[d] = 0.0;
  for (i = 0; i < n_parts; ++i)
    if (lse_parts[i] > mx) mx = lse_parts[i];
  if (mx == -INFINITY) {
    *lse = -INFINITY;
    return;
  }
  for (i = 0; i < n_parts; ++i) sum += exp(lse_parts[i] - mx);
  *lse = mx + log(sum);
  for (i = 0; i < n_parts; ++i) {
    double w = exp(lse_parts[i] - *lse);
    if (lse_parts[i] == -INFINITY) continue;
    for (d = 0; d < ORACLE_D_V; ++d) o[d] += w * o_parts[i * ORACLE_D_V + d];
  }
}

/*
 * The attended positions of query row (b, s): all of [0, seqlen_b) when
 * indices is NULL (with causal != 0, only [0, seqlen_b - s_q + s + 1)), else the
 * non-(-1) entries of indices[b, s, :topk].
 * Returns the count; pos must hold max(seqlen_b, topk) entries.
 */
int64_t oracle_attended_positions(const int32_t* cache_seqlens, const int32_t* indices, int s_q, int topk, int b, int s,
                                  int causal, int64_t* pos) {
  int64_t n = 0, j;
  if (indices == NULL) {
    int64_t end = cache_seqlens[b];
    if (causal) {
      int64_t last = (int64_t)cache_seqlens[b] - s_q + s; /* the query token's own position */
      if (last + 1 < end) end = last + 1;
      if (end < 0) end = 0;
    }
    for (j = 0; j < end; ++j) pos[n++] = j;
    return n;
  }
  for (j = 0; j < topk; ++j) {
    int32_t v = indices[((int64_t)b * s_q + s) * topk + j];
    if (v != -1) pos[n++] = v;
  }
  return n;
}

/*
 * The decode call for a list of query rows.  A row id is the flat index
 * (b * s_q + s) * h_q + h of q[B, s_q, h_q, 576] / o[B, s_q, h_q, 512] /
 * lse[B, s_q, h_q].  rows == NULL means all B * s_q * h_q rows in order.
 * o is [n_rows, 512] and lse is [n_rows], in the order of the list.
 */
void oracle_mla_decode(const uint16_t* q, int B, int s_q, int h_q, const uint8_t* kvcache, int is_fp8,
                       const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens, const int32_t* indices,
                       int topk, int causal, double scale, const int64_t* rows, int64_t n_rows, double* o,
                       double* lse) {
  int64_t r;
  int64_t cap = topk;
  int b;
  (void)B;
  for (b = 0; b < B; ++b)
    if (cache_seqlens[b] > cap) cap = cache_seqlens[b];
#pragma omp parallel for schedule(dynamic, 1)
  for (r = 0; r < n_rows; ++r) {
    int64_t row = rows ? rows[r] : r;
    int s = (int)((row / h_q) % s_q);
    int bb = (int)(row / ((int64_t)h_q * s_q));
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
    int64_t n = oracle_attended_positions(cache_seqlens, indices, s_q, topk, bb, s, causal, pos);
    oracle_attend(q + row * ORACLE_D_QK, kvcache, is_fp8, block_table + (int64_t)bb * max_blocks, pos, n, scale,
                  o + r * ORACLE_D_V, lse + r);
    free(pos);
  }
}

/* ---- the split/tile schedule rule ------------------------------------------ */

/*
 * Streams: dense -> one per request b with ceil(seqlen_b / 64) tiles;
 *          sparse (topk > 0) -> one per (b, s) with ceil(topk / 64) tiles.
 * N = total tiles; q = max(ceil(N / W), min_tiles) (q >= 1).
 * Worker w owns global tiles [w q, min((w + 1) q, N)) of the streams laid end
 * to end.  A stream's splits are the workers that touch it, in worker order.
 *
 * Output (int32):
 *   sched[w * 8 + 0..4] = begin_stream, begin_tile, end_stream, end_tile,
 *                         first_split  (end exclusive; begin == end when idle)
 *   sched[w * 8 + 5, 6] = the end tile of the worker's first piece (in its first
 *                         stream) and that stream's number of splits: derived
 *                         from the words above and split_offset, stored so that
 *                         a worker learns its first piece from one read (0 when
 *                         idle)
 *   split_offset[i]     = first split id of stream i, i = 0..n_streams
 *                         (split_offset[n_streams] = total splits)
 * Returns the number of streams.
 */
int oracle_schedule(const int32_t* cache_seqlens, int B, int s_q, int topk, int num_workers, int min_tiles,
                    int32_t* sched, int32_t* split_offset) {
  int n_streams = topk > 0 ? B * s_q : B;
  int64_t* tiles = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_streams + 1));
  int64_t* first = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_streams + 1));
  int64_t N = 0, q;
  int i, w;
  for (i = 0; i < n_streams; ++i) {
    int64_t len = topk > 0 ? topk : cache_seqlens[i];
    tiles[i] = len > 0 ? (len + ORACLE_PAGE_TOKENS - 1) / ORACLE_PAGE_TOKENS : 0;
    first[i] = N;
    N += tiles[i];
  }
  first[n_streams] = N;
  q = (N + num_workers - 1) / num_workers;
  if (q < min_tiles) q = min_tiles;
  if (q < 1) q = 1;
  /* splits per stream: the number of workers whose range meets the stream */
  split_offset[0] = 0;
  for (i = 0; i < n_streams; ++i) {
    int64_t n = tiles[i] == 0 ? 0 : (first[i] + tiles[i] - 1) / q - first[i] / q + 1;
    split_offset[i + 1] = (int32_t)(split_offset[i] + n);
  }
  for (w = 0; w < num_workers; ++w) {
    int64_t lo = (int64_t)w * q, hi = (int64_t)(w + 1) * q;
    int32_t* e = sched + (int64_t)w * 8;
    int bs, es;
    if (hi > N) hi = N;
    memset(e, 0, 8 * sizeof(int32_t));
    if (lo >= N) { /* idle */
      e[0] = e[2] = n_streams;
      continue;
    }
    /* the stream holding tile lo (skip empty streams), and the position of hi */
    bs = 0;
    while (!(first[bs] <= lo && lo < first[bs] + tiles[bs])) ++bs;
    es = bs;
    while (es < n_streams && first[es] + tiles[es] <= hi) ++es;
    e[0] = bs;
    e[1] = (int32_t)(lo - first[bs]);
    e[2] = es;
    e[3] = es < n_streams ? (int32_t)(hi - first[es]) : 0;
    e[4] = (int32_t)(split_offset[bs] + (w - first[bs] / q));
    e[5] = es == bs ? e[3] : (int32_t)tiles[bs];
    e[6] = split_offset[bs + 1] - split_offset[bs];
  }
  free(tiles);
  free(first);
  return n_streams;
}
