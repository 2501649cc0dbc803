/*
 * CSA2 oracle: a plain, slow, CPU implementation of what the CSA2 hot path
 * computes, in double precision.  TEST INFRASTRUCTURE ONLY: it exists to check
 * the GPU library, is never linked into it, and shares no code with it.
 *
 * Citations name the source pages by site and section:
 *   [summary]  picx.dev whiteboard summary "DeepSeek-V4.1-Flash: Pushing the Limits
 *              of KV Cache Compression"
 *   [blog]     cyber-feed.org repost of the blog article of the same title
 *   [abstract] unarxived.com abstract page of the same title
 *   [card]     wesearch.press story card of the same title
 * and the OCP Microscaling Formats (MX) v1.0 specification for the MXFP4 element
 * and scale encodings that [summary] names.
 *
 * Every decision the pages leave open is taken as listed in the design notes
 * (scale format E8M0 per 32, OCP shared-exponent rule, indexer form, tie-break,
 * visibility, SWA window, output dtypes).
 *
 * Parity-unpinned parts: the decomposition of the pages' 890 bytes/token figure
 * into per-layer pieces (the footprint function is pinned only on its structural
 * values); the block-pooling formula of the KV append path (csa2o_kv_pool: the
 * pages name C and Z but print no pooling rule; pinned only on the mathematics of
 * the reading); the whole path against the pages (they print no worked example).
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define LAT 512      /* latent channels, MXFP4 */
#define ROPE 64      /* rope channels, bf16 */
#define DQ (LAT + ROPE)
#define BLK 32       /* channels per shared scale (E8M0) */
#define NBLK (LAT / BLK)
#define DIDX 64      /* indexer dim */
#define DSWA 128     /* SWA head dim */
#define PAGE 64      /* entries per page */

/* ------------------------------------------------------------------------- */
/* Storage types                                                              */
/* ------------------------------------------------------------------------- */

/* bf16 bit pattern -> exact value. */
static double bf16_val(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* E2M1 (OCP MX v1.0, FP4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit;
 * exponent field 0 encodes the subnormals 0 and 0.5.  [summary] Architecture
 * Components, item 5 (FP4 main KV cache, E2M1 elements). */
double csa2o_e2m1_decode(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* E8M0 scale byte -> 2^(byte - 127) (byte 255 is NaN in OCP MX and is never
 * produced by the quantizer below). */
double csa2o_e8m0_decode(int byte) { return ldexp(1.0, byte - 127); }

/* Round a non-negative y (already divided by the block scale) to the E2M1
 * magnitude grid {0, .5, 1, 1.5, 2, 3, 4, 6}: nearest value, ties to the value
 * whose mantissa bit is 0 (round-half-to-even on the format), and values beyond
 * the largest magnitude saturate to 6 (OCP MX conversion with saturation).
 * Returns the 3-bit magnitude code. */
static int e2m1_round_mag(double y) {
  if (y >= 6.0) return 7;
  /* binade step: 0.5 below 2, 1 in [2, 4), 2 in [4, 6) */
  double step = (y < 2.0) ? 0.5 : (y < 4.0 ? 1.0 : 2.0);
  double base = (y < 2.0) ? 0.0 : (y < 4.0 ? 2.0 : 4.0);
  int base_code = (y < 2.0) ? 0 : (y < 4.0 ? 4 : 6);
  double k = (y - base) / step;         /* exact: step is a power of two */
  double fl = floor(k);
  double frac = k - fl;
  int q = (int)fl;
  if (frac > 0.5) q += 1;
  else if (frac == 0.5) q += ((base_code + q) & 1);   /* tie: go to the even code */
  return base_code + q;
}

/* MXFP4 quantization of one 32-channel block following the OCP MX conversion:
 * shared exponent X = floor(log2(max|x|)) - emax(E2M1) with emax = 2, clamped to
 * the E8M0 range; each element x / 2^X rounded to E2M1 (ties to even code,
 * saturating); the sign bit is the sign of x, also where the magnitude rounds to
 * zero.  An all-zero block takes X = -127.  Returns -1 on NaN/Inf input.
 * [summary] Architecture Components, item 5; the per-32 E8M0 scale is the OCP
 * MXFP4 layout that item names. */
static int quant_block(const float* x, uint8_t* scale_byte, uint8_t codes[BLK]) {
  double amax = 0.0;
  for (int i = 0; i < BLK; ++i) {
    if (!isfinite(x[i])) return -1;
    double a = fabs((double)x[i]);
    if (a > amax) amax = a;
  }
  int X;
  if (amax == 0.0) {
    X = -127;
  } else {
    int ex;
    frexp(amax, &ex);        /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
    X = (ex - 1) - 2;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
  }
  *scale_byte = (uint8_t)(X + 127);
  for (int i = 0; i < BLK; ++i) {
    double y = ldexp(fabs((double)x[i]), -X);
    int mag = e2m1_round_mag(y);
    int sign = signbit(x[i]) ? 1 : 0;
    codes[i] = (uint8_t)((sign << 3) | mag);
  }
  return 0;
}

/* Quantize `rows` fp32 latent rows [rows, 512] into the cache planes:
 * lat [rows, 256] (byte k = code(2k) | code(2k+1) << 4, even channel in the low
 * nibble) and scl [rows, 16] (one E8M0 byte per 32 channels).  Returns 0, or -1
 * if any input is NaN/Inf (nothing is defined for those). */
int csa2o_mxfp4_quantize(const float* x, int64_t rows, uint8_t* lat, uint8_t* scl) {
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < NBLK; ++b) {
      uint8_t codes[BLK];
      if (quant_block(x + r * LAT + b * BLK, &scl[r * NBLK + b], codes)) {
        bad = 1;
        continue;
      }
      for (int k = 0; k < BLK / 2; ++k)
        lat[r * (LAT / 2) + b * (BLK / 2) + k] =
            (uint8_t)(codes[2 * k] | (codes[2 * k + 1] << 4));
    }
  }
  return bad ? -1 : 0;
}

/* v[c] = e2m1(code c) * 2^(scale_byte(c / 32) - 127), exact in double. */
void csa2o_mxfp4_dequantize(const uint8_t* lat, const uint8_t* scl, int64_t rows,
                            double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < LAT; ++c) {
      uint8_t byte = lat[r * (LAT / 2) + c / 2];
      int code = (c & 1) ? (byte >> 4) : (byte & 15);
      out[r * LAT + c] = csa2o_e2m1_decode(code) * csa2o_e8m0_decode(scl[r * NBLK + c / BLK]);
    }
}

/* ------------------------------------------------------------------------- */
/* FP4 with E4M3 scales per 16 channels                                       */
/* ------------------------------------------------------------------------- */

/* E4M3 (OCP 8-bit floating point, E4M3 variant): 1 sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent field 0 encodes subnormals m 2^-9; no
 * infinities; S.1111.111 is NaN, so the largest magnitude is 1.75 * 2^8 = 448.
 * The literal format of [summary] Architecture Components, item 5 (one E4M3 scale
 * per 16 channels; its range 2688 = 6 * 448). */
double csa2o_e4m3_decode(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Non-negative v -> the nearest E4M3 value (ties to the even mantissa), saturating
 * at 448.  Returns the byte. */
int csa2o_e4m3_round(double v) {
  if (v >= 448.0) return 0x7e;
  if (v < ldexp(1.0, -6)) {                     /* subnormal range: steps of 2^-9 */
    double k = v * 512.0, fl = floor(k), frac = k - fl;
    int q = (int)fl;
    if (frac > 0.5 || (frac == 0.5 && (q & 1))) q += 1;
    return q;                                   /* q = 8 is the smallest normal, 0x08 */
  }
  int ex;
  frexp(v, &ex);                                /* v in [2^(ex-1), 2^ex) */
  int e = ex - 1;                               /* floor(log2 v) >= -6 */
  double k = ldexp(v, 3 - e), fl = floor(k), frac = k - fl;   /* k in [8, 16) */
  int q = (int)fl;
  if (frac > 0.5 || (frac == 0.5 && (q & 1))) q += 1;
  if (q == 16) { q = 8; e += 1; }
  if (e > 8) return 0x7e;
  return ((e + 7) << 3) | (q - 8);
}

/* One 16-channel block: scale s = E4M3(max|x| / 6) (nearest, ties to even); each
 * element |x| / s rounded to E2M1 (ties to the even code, saturating at 6), sign
 * bit from x.  A scale that rounds to 0 encodes the block as (signed) zeros.
 * Returns -1 on NaN/Inf. */
static int quant_block16_e4m3(const float* x, uint8_t* scale_byte, uint8_t codes[16]) {
  double amax = 0.0;
  for (int i = 0; i < 16; ++i) {
    if (!isfinite(x[i])) return -1;
    double a = fabs((double)x[i]);
    if (a > amax) amax = a;
  }
  int sb = csa2o_e4m3_round(amax / 6.0);
  *scale_byte = (uint8_t)sb;
  double sv = csa2o_e4m3_decode(sb);
  for (int i = 0; i < 16; ++i) {
    int mag = (sv > 0.0) ? e2m1_round_mag(fabs((double)x[i]) / sv) : 0;
    codes[i] = (uint8_t)(((signbit(x[i]) ? 1 : 0) << 3) | mag);
  }
  return 0;
}

/* Rows [rows, 512] -> lat [rows, 256] (as the MXFP4 layout) and scl [rows, 32]
 * (one E4M3 byte per 16 channels).  Returns -1 if any input is NaN/Inf. */
int csa2o_fp4e4m3_quantize(const float* x, int64_t rows, uint8_t* lat, uint8_t* scl) {
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < LAT / 16; ++b) {
      uint8_t codes[16];
      if (quant_block16_e4m3(x + r * LAT + b * 16, &scl[r * (LAT / 16) + b], codes)) {
        bad = 1;
        continue;
      }
      for (int k = 0; k < 8; ++k)
        lat[r * (LAT / 2) + b * 8 + k] = (uint8_t)(codes[2 * k] | (codes[2 * k + 1] << 4));
    }
  }
  return bad ? -1 : 0;
}

/* v[c] = e2m1(code c) * e4m3(scale byte c / 16), exact in double. */
void csa2o_fp4e4m3_dequantize(const uint8_t* lat, const uint8_t* scl, int64_t rows,
                              double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < LAT; ++c) {
      uint8_t byte = lat[r * (LAT / 2) + c / 2];
      int code = (c & 1) ? (byte >> 4) : (byte & 15);
      out[r * LAT + c] =
          csa2o_e2m1_decode(code) * csa2o_e4m3_decode(scl[r * (LAT / 16) + c / 16]);
    }
}

/* ------------------------------------------------------------------------- */
/* KV append: block pooling                                                   */
/* ------------------------------------------------------------------------- */

/* One compressed entry from a block of R raw tokens ([summary] Architecture
 * Components, item 1, Eq. 1: the decoder's global KV entries come from the
 * projections C = H W^KV and Z = H W^Z; [card] block-based sequence compression;
 * compression ratio 4).  The pooling formula is not on the pages (parity unpinned
 * against them).  Reading: Z holds one pooling logit per token and channel, and
 * the entry is the softmax-over-the-block weighted sum of the tokens' C:
 *   y[ch] = sum_i w_i[ch] c_i[ch],  w_i[ch] = exp(z_i[ch]) / sum_k exp(z_k[ch]).
 * c, z: [n, R, D] fp32; out: [n, D] double. */
void csa2o_kv_pool(const float* c, const float* z, int64_t n, int R, int D, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) {
    for (int ch = 0; ch < D; ++ch) {
      double m = -INFINITY;
      for (int i = 0; i < R; ++i) {
        double zi = z[(e * R + i) * D + ch];
        if (zi > m) m = zi;
      }
      double num = 0.0, den = 0.0;
      for (int i = 0; i < R; ++i) {
        double w = exp((double)z[(e * R + i) * D + ch] - m);
        num += w * (double)c[(e * R + i) * D + ch];
        den += w;
      }
      out[e * D + ch] = num / den;
    }
  }
}

/* Round to bfloat16 (8 significant bits), to nearest with ties to the even
 * significand; finite inputs whose result is a normal bf16 or zero. */
uint16_t csa2o_round_bf16(double x) {
  if (x == 0.0) return signbit(x) ? 0x8000u : 0u;
  int ex;
  double m = frexp(fabs(x), &ex);              /* |x| = m 2^ex, m in [0.5, 1) */
  double q = m * 256.0;                         /* 8 significant bits */
  double r = floor(q);
  double frac = q - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  double v = ldexp(r, ex - 8);
  float f = (float)v;                           /* exact: v has 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  u >>= 16;
  if (x < 0) u |= 0x8000u;
  return (uint16_t)u;
}

void csa2o_round_bf16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = csa2o_round_bf16(x[i]);
}

/* ------------------------------------------------------------------------- */
/* Paging                                                                     */
/* ------------------------------------------------------------------------- */

/* Physical cache row of logical entry j of sequence b (64 entries per page). */
static int64_t phys_row(const int32_t* page_table, int max_pages, int b, int64_t j) {
  return (int64_t)page_table[(int64_t)b * max_pages + j / PAGE] * PAGE + j % PAGE;
}

/* ------------------------------------------------------------------------- */
/* Indexer scoring and Top-K                                                  */
/* ------------------------------------------------------------------------- */

/* Score of every visible entry of one query row:
 *   s[j] = sum_h w[h] * max(0, q_idx[h, :] . k_idx[j, :]),  j < n_vis.
 * The pages name the indexer key and the fresh Top-K of Full and Reindex layers
 * ([summary] Architecture Components, item 2) but print no scoring formula; this
 * is the ReLU-gated multi-head form of the DeepSeek sparse-attention indexer that
 * the CSA2 design extends, with one 64-d key per entry shared by the indexer
 * heads. */
static void index_scores_row(const uint16_t* q_idx_t, const float* w_t, int H_I,
                             const uint16_t* k_idx, const int32_t* page_table,
                             int max_pages, int b, int64_t n_vis, double* s) {
  double q[16][DIDX];
  for (int h = 0; h < H_I; ++h)
    for (int c = 0; c < DIDX; ++c) q[h][c] = bf16_val(q_idx_t[h * DIDX + c]);
  for (int64_t j = 0; j < n_vis; ++j) {
    const uint16_t* k = k_idx + phys_row(page_table, max_pages, b, j) * DIDX;
    double kv[DIDX];
    for (int c = 0; c < DIDX; ++c) kv[c] = bf16_val(k[c]);
    double acc = 0.0;
    for (int h = 0; h < H_I; ++h) {
      double d = 0.0;
      for (int c = 0; c < DIDX; ++c) d += q[h][c] * kv[c];
      acc += (double)w_t[h] * (d > 0.0 ? d : 0.0);
    }
    s[j] = acc;
  }
}

typedef struct {
  double s;
  int64_t j;
} scored;

/* Descending score, then ascending index (the lowest index wins a tie). */
static int cmp_scored(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Top-K selection over one row's scores: order all (score, index) pairs by
 * descending score and ascending index (+0 and -0 compare equal), keep the first
 * min(K, n), emit them in ascending index order, pad with -1.
 * [summary] Architecture Components, item 2 (Top-K indices of Full and Reindex
 * layers, borrowed by Reuse layers). */
void csa2o_topk_from_scores(const double* s, int64_t n, int K, int32_t* out) {
  scored* v = (scored*)malloc(sizeof(scored) * (size_t)(n > 0 ? n : 1));
  for (int64_t j = 0; j < n; ++j) {
    v[j].s = s[j];
    v[j].j = j;
  }
  qsort(v, (size_t)n, sizeof(scored), cmp_scored);
  int64_t m = n < K ? n : K;
  for (int64_t i = 0; i < m; ++i) out[i] = (int32_t)v[i].j;
  qsort(out, (size_t)m, sizeof(int32_t), cmp_i32);
  for (int64_t i = m; i < K; ++i) out[i] = -1;
  free(v);
}

/* Indexer scoring + Top-K for the listed query rows (rows[r] in [0, T)).
 * idx_out: [n_rows, K]; scores_out (optional): [n_rows, max_pages * 64], entries
 * at or beyond n_vis are left untouched. */
void csa2o_index_topk(int T, int H_I, int K, int max_pages, const uint16_t* q_idx,
                      const float* w_idx, const uint16_t* k_idx,
                      const int32_t* page_table, const int32_t* seq_id,
                      const int32_t* n_vis, const int32_t* rows, int n_rows,
                      int32_t* idx_out, double* scores_out) {
  (void)T;
  const int64_t E = (int64_t)max_pages * PAGE;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    int t = rows[r];
    int64_t nv = n_vis[t];
    double* s = scores_out ? scores_out + (int64_t)r * E
                           : (double*)malloc(sizeof(double) * (size_t)(nv > 0 ? nv : 1));
    index_scores_row(q_idx + (int64_t)t * H_I * DIDX, w_idx + (int64_t)t * H_I, H_I, k_idx,
                     page_table, max_pages, seq_id[t], nv, s);
    csa2o_topk_from_scores(s, nv, K, idx_out + (int64_t)r * K);
    if (!scores_out) free(s);
  }
}

/* Candidate pool of the hierarchical sparse indexer ([summary] Architecture
 * Components, item 3: the first Full layer builds a pool of up to 2,048 blocks of 8
 * positions that bounds the search of the later Reindex layers).  Reading: a block is
 * an aligned run of 8 compressed-entry positions, block b = {8b, ..., 8b + 7}; every
 * entry the Full layer selected contributes its block, and the pool is the union of
 * those blocks cut to the visible entries, in ascending order.  sel holds the Full
 * layer's K_sel selected entries of the row (-1 = unused slot).  pool must hold
 * 8 * K_sel positions; returns the pool size. */
int64_t csa2o_pool_positions(const int32_t* sel, int K_sel, int64_t n_vis, int32_t* pool) {
  const int64_t nb = (n_vis + 7) / 8;
  unsigned char* in = (unsigned char*)calloc((size_t)(nb > 0 ? nb : 1), 1);
  for (int i = 0; i < K_sel; ++i)
    if (sel[i] >= 0 && sel[i] < n_vis) in[sel[i] / 8] = 1;
  int64_t m = 0;
  for (int64_t b = 0; b < nb; ++b) {
    if (!in[b]) continue;
    for (int64_t j = 8 * b; j < 8 * b + 8 && j < n_vis; ++j) pool[m++] = (int32_t)j;
  }
  free(in);
  return m;
}

/* Reindex layer searching the pool: the layer's own indexer scores every pool
 * position (the same score as csa2o_index_topk), and the Top-K runs over the pool
 * alone: order the (score, position) pairs by descending score and ascending
 * position, keep the first min(K, pool size), emit ascending, pad with -1.
 * sel: [T, K_sel] selected entries of the Full layer that builds the pool.
 * scores_out (optional): [n_rows, max_pages * 64], pool positions written, the
 * rest left untouched. */
void csa2o_index_topk_pool(int T, int H_I, int K, int max_pages, const uint16_t* q_idx,
                           const float* w_idx, const uint16_t* k_idx,
                           const int32_t* page_table, const int32_t* seq_id,
                           const int32_t* n_vis, const int32_t* sel, int K_sel,
                           const int32_t* rows, int n_rows, int32_t* idx_out,
                           double* scores_out) {
  (void)T;
  const int64_t E = (int64_t)max_pages * PAGE;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    int t = rows[r];
    int64_t nv = n_vis[t];
    int32_t* pool = (int32_t*)malloc(sizeof(int32_t) * (size_t)(8 * K_sel > 0 ? 8 * K_sel : 1));
    int64_t m = csa2o_pool_positions(sel + (int64_t)t * K_sel, K_sel, nv, pool);
    double* s = (double*)malloc(sizeof(double) * (size_t)(nv > 0 ? nv : 1));
    index_scores_row(q_idx + (int64_t)t * H_I * DIDX, w_idx + (int64_t)t * H_I, H_I, k_idx,
                     page_table, max_pages, seq_id[t], nv, s);
    scored* v = (scored*)malloc(sizeof(scored) * (size_t)(m > 0 ? m : 1));
    for (int64_t i = 0; i < m; ++i) {
      v[i].s = s[pool[i]];
      v[i].j = pool[i];
      if (scores_out) scores_out[(int64_t)r * E + pool[i]] = s[pool[i]];
    }
    qsort(v, (size_t)m, sizeof(scored), cmp_scored);
    int32_t* out = idx_out + (int64_t)r * K;
    int64_t keep = m < K ? m : K;
    for (int64_t i = 0; i < keep; ++i) out[i] = (int32_t)v[i].j;
    qsort(out, (size_t)keep, sizeof(int32_t), cmp_i32);
    for (int64_t i = keep; i < K; ++i) out[i] = -1;
    free(v);
    free(s);
    free(pool);
  }
}

/* ------------------------------------------------------------------------- */
/* Attention                                                                  */
/* ------------------------------------------------------------------------- */

/* Softmax attention of one query over n keys given their logits l[] and values
 * v[j * dv ...]: o = sum_j exp(l_j - lse) v_j, lse = log sum_j exp(l_j).
 * No keys: o = 0, lse = -inf. */
static void softmax_combine(const double* l, const double* v, int64_t n, int dv, double* o,
                            double* lse) {
  for (int c = 0; c < dv; ++c) o[c] = 0.0;
  if (n == 0) {
    *lse = -INFINITY;
    return;
  }
  double m = l[0];
  for (int64_t j = 1; j < n; ++j)
    if (l[j] > m) m = l[j];
  double z = 0.0;
  for (int64_t j = 0; j < n; ++j) z += exp(l[j] - m);
  *lse = m + log(z);
  for (int64_t j = 0; j < n; ++j) {
    double p = exp(l[j] - *lse);
    for (int c = 0; c < dv; ++c) o[c] += p * v[j * dv + c];
  }
}

/* Global sparse branch for the listed rows: every head of row t attends over the
 * selected entries idx[t, :] (-1 = no entry), all heads sharing each entry:
 *   key = [dequant(latent) ; rope] (576-d), value = dequant(latent) (512-d),
 *   logit = sm_scale * q . key.
 * [summary] Architecture Components, item 2 (CSA2) and item 5 (FP4 main KV);
 * [blog] introduction (sparse attention covering the whole context).
 * fmt 0: MXFP4 planes (E8M0 scale per 32 channels, kv_scl [*, 16]); fmt 1: FP4 with
 * an E4M3 scale per 16 channels (kv_scl [*, 32]).
 * o_out: [n_rows, H, 512]; lse_out: [n_rows, H]. */
void csa2o_sparse_attn_fmt(int H, int K, int max_pages, const uint16_t* q,
                           const uint8_t* kv_lat, const uint8_t* kv_scl, int fmt,
                           const uint16_t* kv_rope, const int32_t* page_table,
                           const int32_t* seq_id, const int32_t* idx, double sm_scale,
                           const int32_t* rows, int n_rows, double* o_out, double* lse_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    int t = rows[r];
    int b = seq_id[t];
    const int32_t* sel = idx + (int64_t)t * K;
    int64_t n = 0;
    for (int i = 0; i < K; ++i) n += (sel[i] >= 0);
    double* v = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * LAT);
    double* rope = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * ROPE);
    double* l = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    int64_t k = 0;
    for (int i = 0; i < K; ++i) {
      if (sel[i] < 0) continue;
      int64_t pr = phys_row(page_table, max_pages, b, sel[i]);
      if (fmt == 1)
        csa2o_fp4e4m3_dequantize(kv_lat + pr * (LAT / 2), kv_scl + pr * (LAT / 16), 1,
                                 v + k * LAT);
      else
        csa2o_mxfp4_dequantize(kv_lat + pr * (LAT / 2), kv_scl + pr * NBLK, 1, v + k * LAT);
      for (int c = 0; c < ROPE; ++c) rope[k * ROPE + c] = bf16_val(kv_rope[pr * ROPE + c]);
      ++k;
    }
    for (int h = 0; h < H; ++h) {
      const uint16_t* qh = q + ((int64_t)t * H + h) * DQ;
      double qd[DQ];
      for (int c = 0; c < DQ; ++c) qd[c] = bf16_val(qh[c]);
      for (int64_t j = 0; j < n; ++j) {
        double d = 0.0;
        for (int c = 0; c < LAT; ++c) d += qd[c] * v[j * LAT + c];
        for (int c = 0; c < ROPE; ++c) d += qd[LAT + c] * rope[j * ROPE + c];
        l[j] = sm_scale * d;
      }
      softmax_combine(l, v, n, LAT, o_out + ((int64_t)r * H + h) * LAT,
                      lse_out + (int64_t)r * H + h);
    }
    free(v);
    free(rope);
    free(l);
  }
}

void csa2o_sparse_attn(int H, int K, int max_pages, const uint16_t* q, const uint8_t* kv_lat,
                       const uint8_t* kv_scl, const uint16_t* kv_rope,
                       const int32_t* page_table, const int32_t* seq_id, const int32_t* idx,
                       double sm_scale, const int32_t* rows, int n_rows, double* o_out,
                       double* lse_out) {
  csa2o_sparse_attn_fmt(H, K, max_pages, q, kv_lat, kv_scl, 0, kv_rope, page_table, seq_id,
                        idx, sm_scale, rows, n_rows, o_out, lse_out);
}

/* Sliding-window branch for the listed rows: head h of row t attends over the
 * bf16 keys/values at positions [swa_start[t], swa_start[t] + swa_len[t]) of its
 * sequence's window buffer, using KV head h * H_kv / H.
 * [summary] Introduction (global branch combined with local sliding-window
 * attention); [blog] introduction (SWA covering the local window).
 * swa_k, swa_v: [B, L_swa, H_kv, 128]; o_out: [n_rows, H, 128]; lse_out [n_rows, H]. */
void csa2o_swa_attn(int H, int H_kv, int L_swa, const uint16_t* q_swa, const uint16_t* swa_k,
                    const uint16_t* swa_v, const int32_t* seq_id, const int32_t* swa_start,
                    const int32_t* swa_len, double sm_scale, const int32_t* rows, int n_rows,
                    double* o_out, double* lse_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    int t = rows[r];
    int b = seq_id[t];
    int64_t n = swa_len[t];
    double* l = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* v = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * DSWA);
    for (int h = 0; h < H; ++h) {
      int kh = (int)((int64_t)h * H_kv / H);
      double qd[DSWA];
      for (int c = 0; c < DSWA; ++c) qd[c] = bf16_val(q_swa[((int64_t)t * H + h) * DSWA + c]);
      for (int64_t j = 0; j < n; ++j) {
        int64_t pos = (int64_t)swa_start[t] + j;
        int64_t base = (((int64_t)b * L_swa + pos) * H_kv + kh) * DSWA;
        double d = 0.0;
        for (int c = 0; c < DSWA; ++c) {
          d += qd[c] * bf16_val(swa_k[base + c]);
          v[j * DSWA + c] = bf16_val(swa_v[base + c]);
        }
        l[j] = sm_scale * d;
      }
      softmax_combine(l, v, n, DSWA, o_out + ((int64_t)r * H + h) * DSWA,
                      lse_out + (int64_t)r * H + h);
    }
    free(l);
    free(v);
  }
}

/* Threads the oracle's parallel loops use (1 without OpenMP). */
int csa2o_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Footprint                                                                  */
/* ------------------------------------------------------------------------- */

/* Bytes of global cache per raw context token for a layer schedule: every layer
 * that computes its own main KV stores one entry (lat_bytes + scale_bytes +
 * rope_bytes) per compressed position, every layer that computes its own indexer
 * key stores idx_bytes; `ratio` raw tokens share one compressed position.
 * modes: 0 Full (own KV and indexer key), 1 Reindex (own indexer key), 2 Reuse
 * (nothing).  [summary] Architecture Components, item 2 (what each mode computes);
 * Results, KV cache compression (bytes per token). */
double csa2o_footprint_bytes_per_token(const int32_t* modes, int n_layers, int lat_bytes,
                                       int scale_bytes, int rope_bytes, int idx_bytes,
                                       int ratio) {
  double total = 0.0;
  for (int i = 0; i < n_layers; ++i) {
    if (modes[i] == 0) total += lat_bytes + scale_bytes + rope_bytes + idx_bytes;
    else if (modes[i] == 1) total += idx_bytes;
  }
  return total / ratio;
}
