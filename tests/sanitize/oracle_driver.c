/* Host sanitizer driver for the CPU oracle (test infrastructure).
 *
 * Built together with oracle/oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py) and run on small
 * ragged inputs through every exported function, including empty requests,
 * rows shorter than k, ties, -1 padded candidate rows and every decoder code,
 * so that an out-of-bounds access, a leak or undefined behaviour anywhere in
 * the oracle fails the CPU suite.  It checks only shapes and orderings; the
 * values are pinned elsewhere. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_topk(const double*, int64_t, const int64_t*, int, int, int32_t*);
int oracle_index_decode(const void*, int, const float*, const void*, int, const float*, const int64_t*, int, int,
                        int, int, int32_t*, double*, double*);
int oracle_index_prefill(const void*, int, const float*, const float*, const void*, int, const float*, int, int,
                         int, int, int, int, int32_t*, double*, double*);
int oracle_latent_absorb(const void*, int, const void*, int, int, int, int, int, int, double*);
int oracle_latent_score_group(const void*, int, const float*, const void*, int, const void*, int, const float*,
                              int, const int64_t*, int, int, int, int, int, int, int32_t*, double*, double*);
int oracle_latent_reconstruct_scores(const void*, int, const float*, const void*, int, const void*, int,
                                     const float*, int, const int64_t*, int, int, int, int, int, double*);
int oracle_hs_refine(const int32_t*, int, const void*, int, const float*, const void*, int, const void*, int,
                     const float*, int, const int64_t*, int, int, int, int, int, int, int32_t*, double*, double*);
int oracle_latent_append(const void*, int, const void*, int, const int64_t*, int, int, int, void*, int, float*,
                         int64_t, double*);
int oracle_sparse_attention(const void*, int, const void*, int, const int32_t*, const int64_t*, int, int, int, int,
                            int, double, double*, double*);
double oracle_decode_element(const void*, int, int64_t);
uint8_t oracle_encode_e4m3(double);
uint16_t oracle_encode_bf16(double);

enum { BF16 = 0, FP8 = 1, FP16 = 2, FP32 = 3 };

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 33);
}
/* bf16 bits of a small integer in [-3, 3] (exact in bf16) */
static uint16_t bf16_int(void) {
  float f = (float)((int)(rnd() % 7) - 3);
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static uint8_t fp8_code(void) {
  uint8_t c;
  do c = (uint8_t)rnd(); while ((c & 0x7F) == 0x7F);
  return c;
}
static float unit(void) { return 0.5f + (float)(rnd() % 1000) / 1000.0f; }

static int fails = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      ++fails;                                                    \
    }                                                             \
  } while (0)

/* a row of k output slots: ascending valid positions < n, then -1 */
static void check_row(const int32_t* r, int k, int64_t n) {
  int64_t kk = n < k ? n : k;
  for (int j = 0; j < k; ++j) {
    if (j < kk) {
      CHECK(r[j] >= 0 && r[j] < n);
      if (j) CHECK(r[j] > r[j - 1]);
    } else {
      CHECK(r[j] == -1);
    }
  }
}

int main(void) {
  enum { H = 4, D = 128, K = 8 };
  /* ---- decode: ragged requests, one empty, one shorter than k ---- */
  {
    const int B = 3;
    int64_t off[4] = {0, 40, 40, 45};
    uint16_t* q = malloc(sizeof(uint16_t) * B * H * D);
    float w[B * H];
    uint8_t* kc = malloc((size_t)45 * D);
    float ks[45];
    for (int i = 0; i < B * H * D; ++i) q[i] = bf16_int();
    for (int i = 0; i < B * H; ++i) w[i] = (float)((int)(rnd() % 5) - 2);
    for (int i = 0; i < 45 * D; ++i) kc[i] = fp8_code();
    for (int i = 0; i < 45; ++i) ks[i] = unit();
    int32_t idx[B * K];
    double sc[45], ab[45];
    CHECK(oracle_index_decode(q, BF16, w, kc, FP8, ks, off, B, H, D, K, idx, sc, ab) == 0);
    for (int b = 0; b < B; ++b) check_row(idx + b * K, K, off[b + 1] - off[b]);
    CHECK(oracle_index_decode(q, BF16, w, kc, FP8, NULL, off, B, H, D, K, idx, NULL, NULL) == 0);
    CHECK(oracle_index_decode(NULL, BF16, w, kc, FP8, ks, off, B, H, D, K, idx, sc, ab) < 0);
    /* top-k with ties, signed zeros and rows of every length */
    double s[3 * 10] = {1, 1, 1, -0.0, 0.0, 2, 2, -1, 5, 5};
    for (int i = 10; i < 30; ++i) s[i] = (double)(i % 3);
    int64_t lens[3] = {10, 0, 7};
    int32_t out[3 * 4];
    CHECK(oracle_topk(s, 10, lens, 3, 4, out) == 0);
    for (int r = 0; r < 3; ++r) check_row(out + r * 4, 4, lens[r]);
    free(q);
    free(kc);
  }
  /* ---- prefill: causal rows, some shorter than k ---- */
  {
    const int T = 5, L = 12, q0 = 7;
    uint8_t* q = malloc((size_t)T * H * D);
    uint8_t* kc = malloc((size_t)L * D);
    float qs[5], ks[12], w[5 * H];
    for (int i = 0; i < T * H * D; ++i) q[i] = fp8_code();
    for (int i = 0; i < L * D; ++i) kc[i] = fp8_code();
    for (int i = 0; i < T; ++i) qs[i] = unit();
    for (int i = 0; i < L; ++i) ks[i] = unit();
    for (int i = 0; i < T * H; ++i) w[i] = unit() - 1.0f;
    int32_t idx[5 * K];
    double* sc = malloc(sizeof(double) * T * L);
    double* ab = malloc(sizeof(double) * T * L);
    CHECK(oracle_index_prefill(q, FP8, qs, w, kc, FP8, ks, T, L, q0, H, D, K, idx, sc, ab) == 0);
    for (int t = 0; t < T; ++t) {
      check_row(idx + t * K, K, q0 + t + 1);
      for (int s2 = q0 + t + 1; s2 < L; ++s2) CHECK(isinf(sc[t * L + s2]) && sc[t * L + s2] < 0);
    }
    CHECK(oracle_index_prefill(q, FP8, qs, w, kc, FP8, ks, T, L, L - T + 1, H, D, K, idx, sc, ab) < 0);
    free(q);
    free(kc);
    free(sc);
    free(ab);
  }
  /* ---- latent group, reconstruction, HS (bf16 and fp8 block-scaled latents) ---- */
  for (int fp8 = 0; fp8 < 2; ++fp8) {
    const int B = 3, G = 2, Hh = 3, Dh = 16, Dc = fp8 ? 256 : 24, nblk = fp8 ? 2 : 1;
    int64_t off[4] = {0, 30, 30, 39};
    const int n = 39;
    uint16_t* q = malloc(sizeof(uint16_t) * B * G * Hh * Dh);
    uint16_t* wd = malloc(sizeof(uint16_t) * G * Dc * Hh * Dh);
    void* lat = malloc((size_t)n * Dc * (fp8 ? 1 : 2));
    float* cs = malloc(sizeof(float) * n * nblk);
    float w[3 * 2 * 3];
    for (int i = 0; i < B * G * Hh * Dh; ++i) q[i] = bf16_int();
    for (int i = 0; i < G * Dc * Hh * Dh; ++i) wd[i] = bf16_int();
    for (int i = 0; i < n * Dc; ++i) {
      if (fp8) ((uint8_t*)lat)[i] = fp8_code();
      else ((uint16_t*)lat)[i] = bf16_int();
    }
    for (int i = 0; i < n * nblk; ++i) cs[i] = unit();
    for (int i = 0; i < B * G * Hh; ++i) w[i] = unit() - 1.0f;
    int32_t idx[3 * 2 * 6];
    double* sc = malloc(sizeof(double) * G * n);
    double* ab = malloc(sizeof(double) * G * n);
    double* rec = malloc(sizeof(double) * G * n);
    double* qt = malloc(sizeof(double) * B * G * Hh * Dc);
    const int cdt = fp8 ? FP8 : BF16;
    CHECK(oracle_latent_absorb(q, BF16, wd, BF16, B, G, Hh, Dh, Dc, qt) == 0);
    CHECK(oracle_latent_score_group(q, BF16, w, wd, BF16, lat, cdt, cs, nblk, off, B, G, Hh, Dh, Dc, 6, idx, sc,
                                    ab) == 0);
    for (int r = 0; r < B * G; ++r) check_row(idx + r * 6, 6, off[r / G + 1] - off[r / G]);
    CHECK(oracle_latent_reconstruct_scores(q, BF16, w, wd, BF16, lat, cdt, cs, nblk, off, B, G, Hh, Dh, Dc, rec) ==
          0);
    int32_t cand[3 * 8];
    for (int b = 0; b < B; ++b)
      for (int j = 0; j < 8; ++j) {
        const int64_t len = off[b + 1] - off[b];
        cand[b * 8 + j] = j < len ? (int32_t)(j * len / 8) : -1;
      }
    double* hsc = malloc(sizeof(double) * B * G * 8);
    double* hab = malloc(sizeof(double) * B * G * 8);
    int32_t hidx[3 * 2 * 5];
    CHECK(oracle_hs_refine(cand, 8, q, BF16, w, wd, BF16, lat, cdt, cs, nblk, off, B, G, Hh, Dh, Dc, 5, hidx, hsc,
                           hab) == 0);
    free(q);
    free(wd);
    free(lat);
    free(cs);
    free(sc);
    free(ab);
    free(rec);
    free(qt);
    free(hsc);
    free(hab);
  }
  /* ---- latent append (bf16 and fp8 output) ---- */
  {
    const int M = 3, dm = 64, Dc = 128;
    const int64_t n = 6;
    int64_t dst[3] = {4, 0, 5};
    uint16_t* h = malloc(sizeof(uint16_t) * M * dm);
    uint16_t* we = malloc(sizeof(uint16_t) * Dc * dm);
    for (int i = 0; i < M * dm; ++i) h[i] = bf16_int();
    for (int i = 0; i < Dc * dm; ++i) we[i] = bf16_int();
    uint16_t* lat = calloc((size_t)n * Dc, 2);
    uint8_t* lat8 = calloc((size_t)n * Dc, 1);
    float cs[6];
    double* ex = malloc(sizeof(double) * M * Dc);
    CHECK(oracle_latent_append(h, BF16, we, BF16, dst, M, dm, Dc, lat, BF16, NULL, n, ex) == 0);
    CHECK(oracle_latent_append(h, BF16, we, BF16, dst, M, dm, Dc, lat8, FP8, cs, n, NULL) == 0);
    int64_t bad[3] = {4, 0, 6};
    CHECK(oracle_latent_append(h, BF16, we, BF16, bad, M, dm, Dc, lat, BF16, NULL, n, NULL) < 0);
    free(h);
    free(we);
    free(lat);
    free(lat8);
    free(ex);
  }
  /* ---- sparse attention: padded selections, one empty request ---- */
  {
    const int B = 2, Hh = 2, Kk = 4, Dk = 8, Dv = 6;
    int64_t off[3] = {0, 5, 5};
    uint16_t q[2 * 2 * 8], kv[5 * 8];
    for (int i = 0; i < 32; ++i) q[i] = bf16_int();
    for (int i = 0; i < 40; ++i) kv[i] = bf16_int();
    int32_t idx[2 * 4] = {0, 2, 4, -1, -1, -1, -1, -1};
    double out[2 * 2 * 6], mag[2 * 2 * 6];
    CHECK(oracle_sparse_attention(q, BF16, kv, BF16, idx, off, B, Hh, Kk, Dk, Dv, 0.25, out, mag) == 0);
    for (int i = 12; i < 24; ++i) CHECK(out[i] == 0.0);
  }
  /* ---- decoders over every code, encoders over a sweep ---- */
  {
    uint8_t c8[256];
    uint16_t c16[65536];
    for (int i = 0; i < 256; ++i) c8[i] = (uint8_t)i;
    for (int i = 0; i < 65536; ++i) c16[i] = (uint16_t)i;
    double acc = 0.0;
    for (int i = 0; i < 256; ++i)
      if ((i & 0x7F) != 0x7F) acc += oracle_decode_element(c8, FP8, i);
    for (int i = 0; i < 65536; ++i) {
      double a = oracle_decode_element(c16, BF16, i), b = oracle_decode_element(c16, FP16, i);
      if (isfinite(a)) acc += a * 0.0;
      if (isfinite(b)) acc += b * 0.0;
    }
    CHECK(isfinite(acc));
    for (int e = -140; e <= 140; ++e)
      for (int m = 0; m < 8; ++m) {
        const double v = ldexp(1.0 + m / 8.0, e);
        (void)oracle_encode_bf16(v);
        (void)oracle_encode_bf16(-v);
        (void)oracle_encode_e4m3(v);
        (void)oracle_encode_e4m3(-v);
      }
  }
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("oracle driver ok\n");
  return 0;
}
