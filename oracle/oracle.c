/*
 * CPU oracle for the lightning-indexer scan: TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this library.  The product path (the HIP library under
 * sparse_attention_token_lightning_amd/) never calls, links or imports it,
 * and this file shares no code, header, table or constant with it.
 *
 * What it computes is the plain definition of the method, written as direct
 * loops in double precision, with a full sort for top-k:
 *
 *   score[s] = sum_h w[h] * ReLU(q[h] . k[s])
 *
 * over every visible cached position s, then the k highest scores, the lower
 * position winning ties.  Sources (page title, section):
 *   - "IndexCache: Cross-Layer Index Reuse for Sparse Attention", Symbol Map:
 *     a score for each position the query may attend, then a selection of
 *     k = 2,048 positions per query.
 *   - same page, Deep Dive: a Full layer turns its scores into the index
 *     tensor by top-k.
 *   - "Multi-layer Indexer: Overlapping Selection and Attention in DeepSeek
 *     Sparse Attention", The abstract: the selection ranges over the entire
 *     cache, 2048 tokens per query.
 *   - "LatentIndex: Cross-Layer Sharing with Layer-Specific Selection for
 *     Sparse Attention", Abstract and Figure 1: one latent cache per layer
 *     group; per-layer key decoders folded into the queries, so nothing is
 *     decoded per token; in hierarchical selection (HS) the anchor layer's
 *     selection bounds what the follower layers may pick.
 *   - same page, Table 5: 64 indexer heads of 128 dims (64 rotary + 64 not).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - per-token scales dequantize first: k = sigma_s * dec(k_hat);
 *   - prefill row t sees positions s <= qpos0 + t (diagonal included);
 *   - ties: (score descending, position ascending); -0 equals +0;
 *   - output: the kept positions in ascending order, padded with -1 when
 *     fewer than k positions are visible;
 *   - fp8 is OCP E4M3FN (bias 7, no infinities, S.1111.111 is NaN);
 *   - the latent decoder W_l is stored [Dc][H*Dh]; head h's key is
 *     k[j] = sum_c W_l[c][h*Dh + j] * c_s[c], so the absorbed query is
 *     qt[c] = sum_j W_l[c][h*Dh + j] * q[j];
 *   - latent-cache append: the page builds the group's shared latent from
 *     the first layer's hidden state without giving the encoder; read as a
 *     linear down-projection c = W_enc h (W_enc stored [Dc][d_model]), the
 *     sum taken exactly and stored once as bfloat16, nearest, ties to even;
 *   - latent scales: c_scale holds c_nblk entries per row: one scale for the
 *     whole row (c_nblk = 1), or one per 128-value block of an fp8 latent
 *     counted from the row's start, a width that is not a multiple of 128
 *     ending in a shorter block (Dc = 192: 128 + 64; c_nblk = ceil(Dc / 128));
 *   - sparse-attention consumer: the selected rows of a latent KV cache
 *     shared by all heads (keys = the whole row, values = its first Dv
 *     values), softmax with a caller-given scale, -1 entries skipped.
 *
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BF16 0
#define OR_FP8_E4M3 1
#define OR_FP16 2
#define OR_FP32 3

/* ---- element decoders, written from the format definitions ---------------- */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
static double dec_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
 * is subnormal (m * 2^-9); S.1111.111 is NaN; there are no infinities. */
static double dec_e4m3fn(uint8_t b) {
  int sgn = (b >> 7) & 1;
  int e = (b >> 3) & 0xF;
  int m = b & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return sgn ? -v : v;
}

/* IEEE-754 binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
static double dec_f16(uint16_t b) {
  int sgn = (b >> 15) & 1;
  int e = (b >> 10) & 0x1F;
  int m = b & 0x3FF;
  double v;
  if (e == 0x1F) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);
  else v = ldexp((double)(1024 + m), e - 25);
  return sgn ? -v : v;
}

static int dt_ok(int dt) { return dt >= OR_BF16 && dt <= OR_FP32; }

static double dec_at(const void* base, int dt, int64_t i) {
  switch (dt) {
    case OR_BF16: return dec_bf16(((const uint16_t*)base)[i]);
    case OR_FP8_E4M3: return dec_e4m3fn(((const uint8_t*)base)[i]);
    case OR_FP16: return dec_f16(((const uint16_t*)base)[i]);
    default: return (double)((const float*)base)[i];
  }
}

/* Exported so that tests can pin the decoders against the format tables. */
double oracle_decode_element(const void* base, int dt, int64_t i) { return dec_at(base, dt, i); }

/* ---- top-k by full sort ----------------------------------------------------- */

typedef struct {
  double s;
  int64_t i;
} pair_t;

/* (score descending, position ascending).  Doubles compare -0 == +0, which
 * is the canonicalisation the reading asks for. */
static int cmp_pair(const void* a, const void* b) {
  const pair_t* x = (const pair_t*)a;
  const pair_t* y = (const pair_t*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->i < y->i) ? -1 : (x->i > y->i) ? 1 : 0;
}

static int cmp_i64(const void* a, const void* b) {
  int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x < y) ? -1 : (x > y) ? 1 : 0;
}

/* Keep the min(k, n) best of scores[0..n) and write their positions, mapped
 * through idx_map when it is not NULL, in ascending order; pad with -1. */
static int topk_row(const double* scores, int64_t n, int k, const int32_t* idx_map, int32_t* out) {
  int64_t kk = n < k ? n : k;
  pair_t* p = (pair_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(pair_t));
  int64_t* sel = (int64_t*)malloc((size_t)(kk > 0 ? kk : 1) * sizeof(int64_t));
  if (!p || !sel) {
    free(p);
    free(sel);
    return -2;
  }
  for (int64_t i = 0; i < n; ++i) {
    p[i].s = scores[i];
    p[i].i = i;
  }
  qsort(p, (size_t)n, sizeof(pair_t), cmp_pair);
  for (int64_t j = 0; j < kk; ++j) sel[j] = p[j].i;
  qsort(sel, (size_t)kk, sizeof(int64_t), cmp_i64);
  for (int64_t j = 0; j < k; ++j)
    out[j] = (j < kk) ? (idx_map ? idx_map[sel[j]] : (int32_t)sel[j]) : -1;
  free(p);
  free(sel);
  return 0;
}

/* Standalone top-k over `rows` rows of doubles, row r holding lens[r] values
 * at scores + r*stride.  out is [rows][k]. */
int oracle_topk(const double* scores, int64_t stride, const int64_t* lens, int rows, int k,
                int32_t* out) {
  if (!scores || !lens || !out || rows < 0 || k <= 0) return -1;
  int rc = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int r = 0; r < rows; ++r) {
    int e = topk_row(scores + (int64_t)r * stride, lens[r], k, NULL, out + (int64_t)r * k);
    if (e < rc) rc = e;
  }
  return rc;
}

/* ---- decode: one query token per request over a ragged key cache ------------ */

/* q [B][H][D] (q_dt), w [B][H] fp32, kc [n_tok][D] (k_dt), k_scale [n_tok] or
 * NULL (= 1), kv_off [B+1].  Request b owns cache rows [kv_off[b], kv_off[b+1]).
 * Outputs: out_idx [B][k] positions in [0, L_b); out_scores and out_abs are
 * [n_tok] (either may be NULL).  out_abs[s] = sum_h |w_h| * |x_h| is the
 * magnitude against which a floating-point score is judged. */
int oracle_index_decode(const void* q, int q_dt, const float* w, const void* kc, int k_dt,
                        const float* k_scale, const int64_t* kv_off, int B, int H, int D, int k,
                        int32_t* out_idx, double* out_scores, double* out_abs) {
  if (!q || !w || !kc || !kv_off || !out_idx || B < 0 || H <= 0 || D <= 0 || k <= 0) return -1;
  if (!dt_ok(q_dt) || !dt_ok(k_dt)) return -1;
  int rc = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int b = 0; b < B; ++b) {
    int64_t off = kv_off[b];
    int64_t L = kv_off[b + 1] - off;
    double* qd = (double*)malloc((size_t)H * D * sizeof(double));
    double* kd = (double*)malloc((size_t)D * sizeof(double));
    double* S = (double*)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    if (!qd || !kd || !S) {
      rc = -2;
    } else {
      for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d) qd[h * D + d] = dec_at(q, q_dt, ((int64_t)b * H + h) * D + d);
      for (int64_t s = 0; s < L; ++s) {
        int64_t row = off + s;
        double sig = k_scale ? (double)k_scale[row] : 1.0;
        for (int d = 0; d < D; ++d) kd[d] = sig * dec_at(kc, k_dt, row * D + d);
        double acc = 0.0, mag = 0.0;
        for (int h = 0; h < H; ++h) {
          double x = 0.0;
          for (int d = 0; d < D; ++d) x += qd[h * D + d] * kd[d];
          double wh = (double)w[(int64_t)b * H + h];
          acc += wh * (x > 0.0 ? x : 0.0);
          mag += fabs(wh) * fabs(x);
        }
        S[s] = acc;
        if (out_scores) out_scores[row] = acc;
        if (out_abs) out_abs[row] = mag;
      }
      int e = topk_row(S, L, k, NULL, out_idx + (int64_t)b * k);
      if (e < rc) rc = e;
    }
    free(qd);
    free(kd);
    free(S);
  }
  return rc;
}

/* ---- prefill: T new query tokens of one sequence, causal ------------------- */

/* q [T][H][D] (q_dt) with q_scale [T] or NULL, w [T][H], kc [L][D] with
 * k_scale [L] or NULL.  Row t sees s <= qpos0 + t.  out_idx [T][k];
 * out_scores / out_abs [T][L] (may be NULL); masked entries are -inf / 0. */
int oracle_index_prefill(const void* q, int q_dt, const float* q_scale, const float* w,
                         const void* kc, int k_dt, const float* k_scale, int T, int L, int qpos0,
                         int H, int D, int k, int32_t* out_idx, double* out_scores,
                         double* out_abs) {
  if (!q || !w || !kc || !out_idx || T < 0 || L < 0 || H <= 0 || D <= 0 || k <= 0) return -1;
  if (qpos0 < 0 || (int64_t)qpos0 + T > L) return -1;
  if (!dt_ok(q_dt) || !dt_ok(k_dt)) return -1;
  int rc = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int t = 0; t < T; ++t) {
    int64_t vis = (int64_t)qpos0 + t + 1;
    double* qd = (double*)malloc((size_t)H * D * sizeof(double));
    double* kd = (double*)malloc((size_t)D * sizeof(double));
    double* S = (double*)malloc((size_t)vis * sizeof(double));
    if (!qd || !kd || !S) {
      rc = -2;
    } else {
      double sq = q_scale ? (double)q_scale[t] : 1.0;
      for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d)
          qd[h * D + d] = sq * dec_at(q, q_dt, ((int64_t)t * H + h) * D + d);
      for (int64_t s = 0; s < L; ++s) {
        int64_t o = (int64_t)t * L + s;
        if (s >= vis) {
          if (out_scores) out_scores[o] = -INFINITY;
          if (out_abs) out_abs[o] = 0.0;
          continue;
        }
        double sig = k_scale ? (double)k_scale[s] : 1.0;
        for (int d = 0; d < D; ++d) kd[d] = sig * dec_at(kc, k_dt, s * D + d);
        double acc = 0.0, mag = 0.0;
        for (int h = 0; h < H; ++h) {
          double x = 0.0;
          for (int d = 0; d < D; ++d) x += qd[h * D + d] * kd[d];
          double wh = (double)w[(int64_t)t * H + h];
          acc += wh * (x > 0.0 ? x : 0.0);
          mag += fabs(wh) * fabs(x);
        }
        S[s] = acc;
        if (out_scores) out_scores[o] = acc;
        if (out_abs) out_abs[o] = mag;
      }
      int e = topk_row(S, vis, k, NULL, out_idx + (int64_t)t * k);
      if (e < rc) rc = e;
    }
    free(qd);
    free(kd);
    free(S);
  }
  return rc;
}

/* ---- LatentIndex: absorbed queries over a shared latent cache ---------------- */

/* Absorb layer l's key decoder into the query (LatentIndex, Abstract and
 * Figure 1: decoders are absorbed into queries).  q [B][G][H][Dh] (q_dt),
 * w_dec [G][Dc][H*Dh] (w_dt).  out_qt [B][G][H][Dc] in double:
 *   qt[b][l][h][c] = sum_j w_dec[l][c][h*Dh + j] * q[b][l][h][j]. */
int oracle_latent_absorb(const void* q, int q_dt, const void* w_dec, int w_dt, int B, int G,
                         int H, int Dh, int Dc, double* out_qt) {
  if (!q || !w_dec || !out_qt || B < 0 || G <= 0 || H <= 0 || Dh <= 0 || Dc <= 0) return -1;
  if (!dt_ok(q_dt) || !dt_ok(w_dt)) return -1;
#pragma omp parallel for schedule(dynamic)
  for (int bl = 0; bl < B * G; ++bl) {
    int l = bl % G;
    for (int h = 0; h < H; ++h) {
      for (int c = 0; c < Dc; ++c) {
        double acc = 0.0;
        for (int j = 0; j < Dh; ++j)
          acc += dec_at(w_dec, w_dt, ((int64_t)l * Dc + c) * H * Dh + (int64_t)h * Dh + j) *
                 dec_at(q, q_dt, (((int64_t)bl) * H + h) * Dh + j);
        out_qt[(((int64_t)bl) * H + h) * Dc + c] = acc;
      }
    }
  }
  return 0;
}

/* The scale of value c of latent row `row` (1 when there are none): the
 * row's one scale (c_nblk = 1) or its entry c / 128 (128-value blocks). */
static double row_scale(const float* c_scale, int c_nblk, int64_t row, int c) {
  if (!c_scale) return 1.0;
  return (double)c_scale[row * c_nblk + (c_nblk == 1 ? 0 : c / 128)];
}

/* c_nblk is 1 or the number of 128-value blocks of a Dc-value row. */
static int nblk_ok(int c_nblk, int Dc) { return c_nblk == 1 || c_nblk == (Dc + 127) / 128; }

/* Score the shared latent cache for all G layers of each request, then take
 * each layer's own top-k (layer-specific selection).
 * latent [n_tok][Dc] (c_dt) with c_scale [n_tok][c_nblk] or NULL: scale entry j of a
 * row multiplies its values 128 j .. min(128 j + 127, Dc - 1) (c_nblk = 1: one scale
 * per row; ceil(Dc / 128): one per 128-value block); w [B][G][H].
 * out_idx [B][G][k]; out_scores / out_abs [G][n_tok] (may be NULL). */
int oracle_latent_score_group(const void* q, int q_dt, const float* w, const void* w_dec,
                              int w_dt, const void* latent, int c_dt, const float* c_scale, int c_nblk,
                              const int64_t* kv_off, int B, int G, int H, int Dh, int Dc, int k,
                              int32_t* out_idx, double* out_scores, double* out_abs) {
  if (!q || !w || !w_dec || !latent || !kv_off || !out_idx || B < 0 || G <= 0 || H <= 0 ||
      Dh <= 0 || Dc <= 0 || k <= 0)
    return -1;
  if (!dt_ok(c_dt) || !nblk_ok(c_nblk, Dc)) return -1;
  double* qt = (double*)malloc((size_t)(B > 0 ? B : 1) * G * H * Dc * sizeof(double));
  if (!qt) return -2;
  int rc = oracle_latent_absorb(q, q_dt, w_dec, w_dt, B, G, H, Dh, Dc, qt);
  if (rc) {
    free(qt);
    return rc;
  }
  int64_t n_tok = kv_off[B];
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int bl = 0; bl < B * G; ++bl) {
    int b = bl / G, l = bl % G;
    int64_t off = kv_off[b];
    int64_t L = kv_off[b + 1] - off;
    double* cd = (double*)malloc((size_t)Dc * sizeof(double));
    double* S = (double*)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    if (!cd || !S) {
      rc = -2;
    } else {
      for (int64_t s = 0; s < L; ++s) {
        int64_t row = off + s;
        for (int c = 0; c < Dc; ++c) cd[c] = row_scale(c_scale, c_nblk, row, c) * dec_at(latent, c_dt, row * Dc + c);
        double acc = 0.0, mag = 0.0;
        for (int h = 0; h < H; ++h) {
          const double* qh = qt + ((int64_t)bl * H + h) * Dc;
          double x = 0.0;
          for (int c = 0; c < Dc; ++c) x += qh[c] * cd[c];
          double wh = (double)w[(int64_t)bl * H + h];
          acc += wh * (x > 0.0 ? x : 0.0);
          mag += fabs(wh) * fabs(x);
        }
        S[s] = acc;
        if (out_scores) out_scores[(int64_t)l * n_tok + row] = acc;
        if (out_abs) out_abs[(int64_t)l * n_tok + row] = mag;
      }
      int e = topk_row(S, L, k, NULL, out_idx + (int64_t)bl * k);
      if (e < rc) rc = e;
    }
    free(cd);
    free(S);
  }
  free(qt);
  return rc;
}

/* The same scores computed the long way: reconstruct every layer-specific
 * historical key k_{l,h,s}[j] = sum_c w_dec[l][c][h*Dh + j] * c_s[c] and score
 * it with the un-absorbed query (what LatentIndex's absorption avoids doing).
 * Used only to check that absorption changes nothing.  out_scores [G][n_tok]. */
int oracle_latent_reconstruct_scores(const void* q, int q_dt, const float* w, const void* w_dec,
                                     int w_dt, const void* latent, int c_dt,
                                     const float* c_scale, int c_nblk, const int64_t* kv_off, int B, int G,
                                     int H, int Dh, int Dc, double* out_scores) {
  if (!q || !w || !w_dec || !latent || !kv_off || !out_scores || B < 0 || G <= 0 || H <= 0 ||
      Dh <= 0 || Dc <= 0)
    return -1;
  if (!dt_ok(q_dt) || !dt_ok(w_dt) || !dt_ok(c_dt) || !nblk_ok(c_nblk, Dc)) return -1;
  int64_t n_tok = kv_off[B];
  int rc = 0;
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int bl = 0; bl < B * G; ++bl) {
    int b = bl / G, l = bl % G;
    double* cd = (double*)malloc((size_t)Dc * sizeof(double));
    double* kk = (double*)malloc((size_t)Dh * sizeof(double));
    if (!cd || !kk) {
      rc = -2;
    } else {
      for (int64_t row = kv_off[b]; row < kv_off[b + 1]; ++row) {
        for (int c = 0; c < Dc; ++c) cd[c] = row_scale(c_scale, c_nblk, row, c) * dec_at(latent, c_dt, row * Dc + c);
        double acc = 0.0;
        for (int h = 0; h < H; ++h) {
          for (int j = 0; j < Dh; ++j) {
            double v = 0.0;
            for (int c = 0; c < Dc; ++c)
              v += dec_at(w_dec, w_dt, ((int64_t)l * Dc + c) * H * Dh + (int64_t)h * Dh + j) *
                   cd[c];
            kk[j] = v;
          }
          double x = 0.0;
          for (int j = 0; j < Dh; ++j)
            x += dec_at(q, q_dt, ((int64_t)bl * H + h) * Dh + j) * kk[j];
          acc += (double)w[(int64_t)bl * H + h] * (x > 0.0 ? x : 0.0);
        }
        out_scores[(int64_t)l * n_tok + row] = acc;
      }
    }
    free(cd);
    free(kk);
  }
  return rc;
}

/* ---- HS: followers rescore only the anchor's candidate set ------------------- */

/* cand_idx [B][C]: the anchor's kept positions, ascending, -1 padded (the
 * output of the anchor's own top-C).  Each follower f < Gf scores the latent
 * rows of those candidates with its absorbed query and keeps its own top-k
 * among them (LatentIndex, Abstract: the anchor's selection is the pool each
 * follower picks from, on its own scores).  Ties go to the lower position.
 * out_idx [B][Gf][k] token positions; out_scores / out_abs [B][Gf][C] indexed by
 * candidate slot (slots past the valid candidates are left untouched). */
int oracle_hs_refine(const int32_t* cand_idx, int C, const void* q, int q_dt, const float* w,
                     const void* w_dec, int w_dt, const void* latent, int c_dt,
                     const float* c_scale, int c_nblk, const int64_t* kv_off, int B, int Gf, int H, int Dh,
                     int Dc, int k, int32_t* out_idx, double* out_scores, double* out_abs) {
  if (!cand_idx || !q || !w || !w_dec || !latent || !kv_off || !out_idx || C < 0 || B < 0 ||
      Gf <= 0 || H <= 0 || Dh <= 0 || Dc <= 0 || k <= 0)
    return -1;
  if (!dt_ok(c_dt) || !nblk_ok(c_nblk, Dc)) return -1;
  double* qt = (double*)malloc((size_t)(B > 0 ? B : 1) * Gf * H * Dc * sizeof(double));
  if (!qt) return -2;
  int rc = oracle_latent_absorb(q, q_dt, w_dec, w_dt, B, Gf, H, Dh, Dc, qt);
  if (rc) {
    free(qt);
    return rc;
  }
#pragma omp parallel for schedule(dynamic) reduction(min : rc)
  for (int bf = 0; bf < B * Gf; ++bf) {
    int b = bf / Gf;
    const int32_t* cand = cand_idx + (int64_t)b * C;
    int64_t nv = 0;
    while (nv < C && cand[nv] >= 0) ++nv;
    double* cd = (double*)malloc((size_t)Dc * sizeof(double));
    double* S = (double*)malloc((size_t)(nv > 0 ? nv : 1) * sizeof(double));
    if (!cd || !S) {
      rc = -2;
    } else {
      for (int64_t j = 0; j < nv; ++j) {
        int64_t row = kv_off[b] + cand[j];
        for (int c = 0; c < Dc; ++c) cd[c] = row_scale(c_scale, c_nblk, row, c) * dec_at(latent, c_dt, row * Dc + c);
        double acc = 0.0, mag = 0.0;
        for (int h = 0; h < H; ++h) {
          const double* qh = qt + ((int64_t)bf * H + h) * Dc;
          double x = 0.0;
          for (int c = 0; c < Dc; ++c) x += qh[c] * cd[c];
          double wh = (double)w[(int64_t)bf * H + h];
          acc += wh * (x > 0.0 ? x : 0.0);
          mag += fabs(wh) * fabs(x);
        }
        S[j] = acc;
        if (out_scores) out_scores[(int64_t)bf * C + j] = acc;
        if (out_abs) out_abs[(int64_t)bf * C + j] = mag;
      }
      int e = topk_row(S, nv, k, cand, out_idx + (int64_t)bf * k);
      if (e < rc) rc = e;
    }
    free(cd);
    free(S);
  }
  free(qt);
  return rc;
}

/* ---- latent-cache append ---------------------------------------------------- */
/*
 * "LatentIndex: Cross-Layer Sharing with Layer-Specific Selection for Sparse
 * Attention", Abstract and Figure 1: a layer group builds its shared latent
 * cache from the group's first layer's hidden states.  The pages do not give
 * the encoder; the reading here is a linear down-projection (the latent of
 * Multi-head Latent Attention, whose principle the page extends):
 *     c[b][d] = sum_i h[b][i] * w_enc[d][i]
 * stored as bfloat16 (nearest, ties to even) at latent row dst_row[b].
 */

/* bfloat16 code nearest to a finite real value, ties to the even code.
 * bfloat16 keeps 8 significant bits (exponent range of binary32): a normal
 * value is s * 2^(e-7) with s an integer in [128, 256); below 2^-126 the
 * spacing is fixed at 2^-133. */
static uint16_t enc_bf16_rne(double v) {
  uint16_t sgn = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return sgn;
  if (a < ldexp(1.0, -126)) {                  /* subnormal range */
    double q = rint(ldexp(a, 133));            /* rint: nearest, ties to even */
    return (uint16_t)(sgn | (uint16_t)q);      /* q == 128 is the smallest normal */
  }
  int e;
  double m = frexp(a, &e);                     /* a = m * 2^e, m in [0.5, 1) */
  double s = rint(ldexp(m, 8));                /* significand, 8 bits: [128, 256] */
  if (s == 256.0) {                            /* rounded up to the next binade */
    s = 128.0;
    e += 1;
  }
  int biased = (e - 1) + 127;                  /* a ~ (s/128) * 2^(e-1) */
  if (biased >= 255) return (uint16_t)(sgn | 0x7F80u); /* beyond range: infinity */
  return (uint16_t)(sgn | (uint16_t)(biased << 7) | (uint16_t)((int)s - 128));
}

/* OCP E4M3FN code nearest to a finite value, ties to the even code, values
 * beyond the largest finite (448 = 1.75 * 2^8) saturated to it.  A normal
 * value is (8 + m)/8 * 2^e with e in [-6, 8] and m in 0..7 (the code
 * S.1111.111 is NaN, so m <= 6 at e = 8); below 2^-6 the spacing is 2^-9. */
static uint8_t enc_e4m3_rne(double v) {
  uint8_t sgn = signbit(v) ? 0x80u : 0u;
  double a = fabs(v);
  if (a >= 464.0) return (uint8_t)(sgn | 0x7Eu); /* 464 is the tie 448|480: even is 448 */
  if (a < ldexp(1.0, -6)) return (uint8_t)(sgn | (uint8_t)rint(ldexp(a, 9))); /* 8 -> 2^-6, code 0x08 */
  int e;
  double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  double s = rint(ldexp(m, 4)); /* 4 significant bits: [8, 16] */
  if (s == 16.0) {
    s = 8.0;
    e += 1;
  }
  int biased = (e - 1) + 7;
  return (uint8_t)(sgn | (uint8_t)(biased << 3) | (uint8_t)((int)s - 8));
}

/* Latent-cache append.  c_dt OR_BF16: latent [n_tok][Dc] bf16 codes (uint16).
 * c_dt OR_FP8_E4M3: latent [n_tok][Dc] E4M3 codes (uint8) and c_scale
 * [n_tok][ceil(Dc/128)]: each 128-value block of a row (the last one shorter when Dc
 * is not a multiple of 128) is the exact sum rounded to
 * fp32, its scale the block's largest magnitude / 448 in fp32 (1 for an
 * all-zero block) and its codes E4M3 of (value / scale) taken in fp32, nearest
 * even, saturating: the quantisation steps in the precision of the kernel that
 * takes them (fp32 sums, divisions and maxima). */
int oracle_latent_append(const void* h, int h_dt, const void* w_enc, int w_dt, const int64_t* dst_row, int B,
                         int d_model, int Dc, void* latent, int c_dt, float* c_scale, int64_t n_tok, double* exact) {
  if (!dt_ok(h_dt) || !dt_ok(w_dt) || B < 0 || d_model <= 0 || Dc <= 0) return -1;
  if (c_dt != OR_BF16 && !(c_dt == OR_FP8_E4M3 && c_scale)) return -1;
  for (int b = 0; b < B; ++b)
    if (dst_row[b] < 0 || dst_row[b] >= n_tok) return -1;
  double* row = (double*)malloc(sizeof(double) * (size_t)Dc);
  if (!row) return -2;
  for (int b = 0; b < B; ++b) {
    for (int d = 0; d < Dc; ++d) {
      double acc = 0.0;
      for (int i = 0; i < d_model; ++i)
        acc += dec_at(h, h_dt, (int64_t)b * d_model + i) * dec_at(w_enc, w_dt, (int64_t)d * d_model + i);
      if (exact) exact[(int64_t)b * Dc + d] = acc;
      row[d] = acc;
    }
    if (c_dt == OR_BF16) {
      for (int d = 0; d < Dc; ++d) ((uint16_t*)latent)[dst_row[b] * Dc + d] = enc_bf16_rne(row[d]);
      continue;
    }
    const int nblk = (Dc + 127) / 128;
    for (int blk = 0; blk < nblk; ++blk) {
      const int d1 = 128 * blk + 128 < Dc ? 128 * blk + 128 : Dc;
      float amax = 0.0f;
      for (int d = 128 * blk; d < d1; ++d) {
        const float f = fabsf((float)row[d]);
        if (f > amax) amax = f;
      }
      const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      c_scale[dst_row[b] * nblk + blk] = sc;
      for (int d = 128 * blk; d < d1; ++d)
        ((uint8_t*)latent)[dst_row[b] * Dc + d] = enc_e4m3_rne((double)((float)row[d] / sc));
    }
  }
  free(row);
  return 0;
}

/* Exported so that tests can pin the E4M3 encoder on its own. */
uint8_t oracle_encode_e4m3(double v) { return enc_e4m3_rne(v); }

/* Exported so that tests can pin the bfloat16 encoder on its own. */
uint16_t oracle_encode_bf16(double v) { return enc_bf16_rne(v); }

/* ---- sparse-attention consumer -------------------------------------------------- */
/*
 * The attention that consumes the indexer's selection ("IndexCache: Cross-Layer
 * Index Reuse for Sparse Attention", Symbol Map: the selected set holds the k
 * positions sent to core sparse attention; "Multi-layer Indexer ...", The
 * abstract: each layer attends the tokens its indexer kept).  The pages do not
 * give the attention's form; the reading here is the decode attention of the
 * pages' model in its latent form: every selected token contributes one cached
 * row kv[r] of Dk values shared by all heads, its first Dv values are the value
 *     o[b][h] = sum_j p_j kv[r_j][0:Dv] / sum_j p_j,
 *     p_j = exp(s_j - max s),  s_j = scale * (q[b][h] . kv[r_j]),
 * over the valid entries j of idx[b] (r_j = kv_off[b] + idx[b][j]; -1 entries
 * are skipped).  A request with no valid entry gets o = 0.  `mag` receives
 * sum_j p_j |kv[r_j][d]| / sum_j p_j, the scale of each output's error.
 */
int oracle_sparse_attention(const void* q, int q_dt, const void* kv, int kv_dt, const int32_t* idx,
                            const int64_t* kv_off, int B, int H, int K, int Dk, int Dv, double scale, double* out,
                            double* mag) {
  if (!dt_ok(q_dt) || !dt_ok(kv_dt) || B < 0 || H <= 0 || K <= 0 || Dk <= 0 || Dv <= 0 || Dv > Dk) return -1;
  double* s = (double*)malloc(sizeof(double) * (size_t)K);
  if (!s) return -2;
  for (int b = 0; b < B; ++b) {
    const int64_t len = kv_off[b + 1] - kv_off[b];
    for (int j = 0; j < K; ++j)
      if (idx[(int64_t)b * K + j] < -1 || idx[(int64_t)b * K + j] >= len) {
        free(s);
        return -1;
      }
    for (int h = 0; h < H; ++h) {
      const int64_t qo = ((int64_t)b * H + h) * Dk;
      double m = -INFINITY;
      for (int j = 0; j < K; ++j) {
        const int32_t t = idx[(int64_t)b * K + j];
        if (t < 0) continue;
        const int64_t r = (kv_off[b] + t) * Dk;
        double acc = 0.0;
        for (int d = 0; d < Dk; ++d) acc += dec_at(q, q_dt, qo + d) * dec_at(kv, kv_dt, r + d);
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
      }
      double l = 0.0;
      double* o = out + ((int64_t)b * H + h) * Dv;
      double* g = mag + ((int64_t)b * H + h) * Dv;
      for (int d = 0; d < Dv; ++d) o[d] = g[d] = 0.0;
      for (int j = 0; j < K; ++j) {
        const int32_t t = idx[(int64_t)b * K + j];
        if (t < 0) continue;
        const int64_t r = (kv_off[b] + t) * Dk;
        const double p = exp(s[j] - m);
        l += p;
        for (int d = 0; d < Dv; ++d) {
          const double v = dec_at(kv, kv_dt, r + d);
          o[d] += p * v;
          g[d] += p * fabs(v);
        }
      }
      if (l > 0.0)
        for (int d = 0; d < Dv; ++d) {
          o[d] /= l;
          g[d] /= l;
        }
    }
  }
  free(s);
  return 0;
}
