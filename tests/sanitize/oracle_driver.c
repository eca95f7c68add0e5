/* The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Built by tests/test_sanitize.py with the C compiler, together with oracle/kvq_oracle.c, and run as a
 * program: every oracle entry point is called on small inputs whose buffers are sized exactly as the
 * oracle's comments state (heap blocks, so an access past one is reported), including the edge sizes
 * (one key, lengths of zero and of one, a key of zeros).  The checks here are only sanity checks (finite
 * values, rows of probabilities summing to one, codes in range); the oracle's numerical pins are the
 * Python tests.  Exit status 0 when every check holds; the sanitizers abort the program on the first
 * memory or undefined-behaviour error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ora_lloyd_max_unit(int b, double* c, double* t);
int ora_codebook(int d, int b, double* levels, double* thresholds);
double ora_quantizer_mse_unit(int b, const double* c, const double* t);
void ora_hadamard(int d, double* H);
void ora_rotate_query(int d, const int8_t* signs, const double* q, double* qrot);
void ora_encode_keys(int d, int b, const double* thresholds, const int8_t* signs, const double* keys, int64_t n,
                     uint8_t* codes, double* norms, double* y_out, uint8_t* tie, double tie_eps);
void ora_unpack_codes(int d, int b, const uint8_t* codes, int64_t n, int32_t* idx);
void ora_build_lut(int d, int b, const double* levels, const double* qrot, double* lut);
void ora_scores(int d, int b, const double* levels, const int8_t* signs, const double* q, const uint8_t* codes,
                const double* norms, int B, int Hq, int Hkv, int64_t Tcap, const int32_t* seq_lens, double* scores);
void ora_softmax_row(const double* s, int64_t len, double scale, double* p);
void ora_decode_attn(int d, int b, const double* levels, const int8_t* signs, const double* q, const uint8_t* codes,
                     const double* norms, const double* v, int B, int Hq, int Hkv, int64_t Tcap,
                     const int32_t* seq_lens, double scale, double* out);
void ora_dequant_rows(int d, int b, const double* levels, const int8_t* signs, const uint8_t* codes,
                      const double* norms, int64_t n, double* out);
void ora_decode_attn_qv(int d, int b, const double* levels, const int8_t* signs, const double* q, const uint8_t* codes,
                        const double* norms, const uint8_t* vcodes, const double* vnorms, int B, int Hq, int Hkv,
                        int64_t Tcap, const int32_t* seq_lens, double scale, double* out);
void ora_exact_attn(int d, const double* q, const double* keys, const double* v, int n, int Hq, int Hkv, int64_t T,
                    double scale, double* out);
int ora_sign_errors(int d, int b, const double* levels, const double* thresholds, const int8_t* cands, int C,
                    const double* q, const double* keys, const double* v, int n, int Hq, int Hkv, int64_t T,
                    double scale, double* errors);
void ora_kmeans(const double* train, int64_t n, int ds, int K, int iters, const int64_t* init_rows, double* cent,
                double* objective);
void ora_pq_encode(int d, int m, int K, int cbits, const double* cent, const double* keys, int64_t n, uint8_t* codes,
                   double* gap);
void ora_pq_scores(int d, int m, int K, int cbits, const double* cent, const double* q, const uint8_t* codes, int B,
                   int Hq, int Hkv, int64_t Tcap, const int32_t* seq_lens, double* scores);
void ora_pq_decode_attn(int d, int m, int K, int cbits, const double* cent, const double* q, const uint8_t* codes,
                        const double* v, int B, int Hq, int Hkv, int64_t Tcap, const int32_t* seq_lens, double scale,
                        double* out);
void ora_pot_levels(int b, int mant, double* mags, double* thresholds);
void ora_pot_encode(int d, int b, int mant, const double* keys, int64_t n, uint8_t* codes, double* scales,
                    uint8_t* tie, double tie_eps);
void ora_pot_dequant(int d, int b, int mant, const uint8_t* codes, const double* scales, int64_t n, double* out);
void ora_pot_scores(int d, int b, int mant, const double* q, const uint8_t* codes, const double* scales, int B,
                    int Hq, int Hkv, int64_t Tcap, const int32_t* seq_lens, double* scores);
void ora_pot_decode_attn(int d, int b, int mant, const double* q, const uint8_t* codes, const double* scales,
                         const double* v, int B, int Hq, int Hkv, int64_t Tcap, const int32_t* seq_lens, double scale,
                         double* out);

static int n_fail = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);       \
      ++n_fail;                                                      \
    }                                                                \
  } while (0)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}
static double* dalloc(size_t n) {
  double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = urand();
  return p;
}
static int all_finite(const double* x, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

static void scalar_codec(int d, int b) {
  const int L = 1 << b, bpk = d * b / 8, B = 2, Hq = 4, Hkv = 2;
  const int64_t T = 37;
  double* levels = dalloc((size_t)L);
  double* thr = dalloc((size_t)L - 1);
  CHECK(ora_codebook(d, b, levels, thr) > 0); /* iterations to converge */
  for (int j = 0; j + 1 < L; ++j) CHECK(levels[j] < thr[j] && thr[j] < levels[j + 1]);
  int8_t* signs = (int8_t*)malloc((size_t)d);
  for (int i = 0; i < d; ++i) signs[i] = urand() < 0 ? -1 : 1;
  const int64_t nk = (int64_t)B * Hkv * T;
  double* keys = dalloc((size_t)nk * d);
  for (int i = 0; i < d; ++i) keys[i] = 0.0; /* a key of zeros */
  uint8_t* codes = (uint8_t*)malloc((size_t)nk * bpk);
  double* norms = dalloc((size_t)nk);
  double* y = dalloc((size_t)nk * d);
  uint8_t* tie = (uint8_t*)malloc((size_t)nk * d);
  ora_encode_keys(d, b, thr, signs, keys, nk, codes, norms, y, tie, 1e-6);
  CHECK(norms[0] == 0.0 && all_finite(norms, (size_t)nk));
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)nk * d);
  ora_unpack_codes(d, b, codes, nk, idx);
  for (int64_t i = 0; i < nk * d; ++i) CHECK(idx[i] >= 0 && idx[i] < L);
  double* q = dalloc((size_t)B * Hq * d);
  double* qrot = dalloc((size_t)d);
  ora_rotate_query(d, signs, q, qrot);
  double* lut = dalloc((size_t)d * L);
  ora_build_lut(d, b, levels, qrot, lut);
  CHECK(all_finite(lut, (size_t)d * L));
  int32_t lens[2] = {(int32_t)T, 1};
  double* scores = dalloc((size_t)B * Hq * T);
  ora_scores(d, b, levels, signs, q, codes, norms, B, Hq, Hkv, T, lens, scores);
  CHECK(isinf(scores[(size_t)1 * Hq * T + 5]) && scores[(size_t)1 * Hq * T + 5] < 0); /* past the length */
  double* v = dalloc((size_t)nk * d);
  double* out = dalloc((size_t)B * Hq * d);
  ora_decode_attn(d, b, levels, signs, q, codes, norms, v, B, Hq, Hkv, T, lens, 0.125, out);
  CHECK(all_finite(out, (size_t)B * Hq * d));
  ora_decode_attn(d, b, levels, signs, q, codes, norms, v, B, Hq, Hkv, T, NULL, 0.125, out);
  CHECK(all_finite(out, (size_t)B * Hq * d));
  double* deq = dalloc((size_t)nk * d);
  ora_dequant_rows(d, b, levels, signs, codes, norms, nk, deq);
  CHECK(all_finite(deq, (size_t)nk * d));
  uint8_t* vcodes = (uint8_t*)malloc((size_t)nk * bpk);
  double* vnorms = dalloc((size_t)nk);
  ora_encode_keys(d, b, thr, signs, v, nk, vcodes, vnorms, NULL, NULL, 0.0);
  ora_decode_attn_qv(d, b, levels, signs, q, codes, norms, vcodes, vnorms, B, Hq, Hkv, T, lens, 0.125, out);
  CHECK(all_finite(out, (size_t)B * Hq * d));
  /* sign-pattern selection on the same keys */
  const int C = 3;
  int8_t* cands = (int8_t*)malloc((size_t)C * d);
  for (int i = 0; i < C * d; ++i) cands[i] = urand() < 0 ? -1 : 1;
  double* errors = dalloc((size_t)C);
  const int best = ora_sign_errors(d, b, levels, thr, cands, C, q, keys, v, B, Hq, Hkv, T, 0.125, errors);
  CHECK(best >= 0 && best < C);
  for (int c = 0; c < C; ++c) CHECK(errors[c] >= 0.0 && errors[best] <= errors[c]);
  double* eout = dalloc((size_t)B * Hq * d);
  ora_exact_attn(d, q, keys, v, B, Hq, Hkv, T, 0.125, eout);
  CHECK(all_finite(eout, (size_t)B * Hq * d));
  free(levels); free(thr); free(signs); free(keys); free(codes); free(norms); free(y); free(tie); free(idx);
  free(q); free(qrot); free(lut); free(scores); free(v); free(out); free(deq); free(vcodes); free(vnorms);
  free(cands); free(errors); free(eout);
}

static void pq_codec(int cbits, int K) {
  const int d = 32, m = 8, ds = d / m, B = 2, Hq = 4, Hkv = 2, bpk = m * cbits / 8;
  const int64_t T = 29, n = 64;
  double* cent = dalloc((size_t)Hkv * m * K * ds);
  /* k-means of one subspace of one head, with its objective trace */
  double* train = dalloc((size_t)n * ds);
  int64_t* init = (int64_t*)malloc(sizeof(int64_t) * (size_t)K);
  for (int c = 0; c < K; ++c) init[c] = (c * 7) % n;
  double obj[4];
  ora_kmeans(train, n, ds, K, 3, init, cent, obj);
  for (int it = 0; it + 1 < 4; ++it) CHECK(obj[it + 1] <= obj[it] + 1e-12);
  for (size_t i = 0; i < (size_t)Hkv * m * K * ds; ++i) cent[i] = urand();
  const int64_t nk = (int64_t)B * Hkv * T;
  double* keys = dalloc((size_t)nk * d);
  uint8_t* codes = (uint8_t*)malloc((size_t)nk * bpk);
  double* gap = dalloc((size_t)T * m);
  for (int64_t r = 0; r < (int64_t)B * Hkv; ++r) /* each row of T keys with its own head's centroids */
    ora_pq_encode(d, m, K, cbits, cent + (size_t)(r % Hkv) * m * K * ds, keys + (size_t)r * T * d, T,
                  codes + (size_t)r * T * bpk, gap);
  for (int64_t i = 0; i < T * m; ++i) CHECK(gap[i] >= 0.0);
  double* q = dalloc((size_t)B * Hq * d);
  int32_t lens[2] = {(int32_t)T, 0};
  double* scores = dalloc((size_t)B * Hq * T);
  ora_pq_scores(d, m, K, cbits, cent, q, codes, B, Hq, Hkv, T, lens, scores);
  double* v = dalloc((size_t)nk * d);
  double* out = dalloc((size_t)B * Hq * d);
  ora_pq_decode_attn(d, m, K, cbits, cent, q, codes, v, B, Hq, Hkv, T, lens, 0.125, out);
  CHECK(all_finite(out, (size_t)Hq * d)); /* batch 0; batch 1 has no keys */
  free(cent); free(train); free(init); free(keys); free(codes); free(gap); free(q); free(scores); free(v);
  free(out);
}

static void pot_codec(int b, int mant) {
  const int d = 64, bpk = d * b / 8, B = 2, Hq = 4, Hkv = 2;
  const int64_t T = 21;
  const int NM = 1 << (b - 1);
  double* mags = dalloc((size_t)NM);
  double* thr = dalloc((size_t)NM - 1);
  ora_pot_levels(b, mant, mags, thr);
  for (int j = 0; j + 1 < NM; ++j) CHECK(mags[j] > thr[j] && thr[j] > mags[j + 1]);
  const int64_t nk = (int64_t)B * Hkv * T;
  double* keys = dalloc((size_t)nk * d);
  uint8_t* codes = (uint8_t*)malloc((size_t)nk * bpk);
  double* scales = dalloc((size_t)nk);
  uint8_t* tie = (uint8_t*)malloc((size_t)nk * d);
  ora_pot_encode(d, b, mant, keys, nk, codes, scales, tie, 1e-9);
  double* deq = dalloc((size_t)nk * d);
  ora_pot_dequant(d, b, mant, codes, scales, nk, deq);
  CHECK(all_finite(deq, (size_t)nk * d));
  double* q = dalloc((size_t)B * Hq * d);
  double* scores = dalloc((size_t)B * Hq * T);
  ora_pot_scores(d, b, mant, q, codes, scales, B, Hq, Hkv, T, NULL, scores);
  CHECK(all_finite(scores, (size_t)B * Hq * T));
  double* v = dalloc((size_t)nk * d);
  double* out = dalloc((size_t)B * Hq * d);
  ora_pot_decode_attn(d, b, mant, q, codes, scales, v, B, Hq, Hkv, T, NULL, 0.125, out);
  CHECK(all_finite(out, (size_t)B * Hq * d));
  free(mags); free(thr); free(keys); free(codes); free(scales); free(tie); free(deq); free(q); free(scores);
  free(v); free(out);
}

int main(void) {
  for (int b = 1; b <= 4; ++b) {
    double c[16], t[15];
    CHECK(ora_lloyd_max_unit(b, c, t) > 0);
    CHECK(ora_quantizer_mse_unit(b, c, t) > 0.0);
  }
  double* H = dalloc(64 * 64);
  ora_hadamard(64, H);
  for (int i = 0; i < 64; ++i) /* rows orthonormal */
    for (int j = 0; j < 64; ++j) {
      double s = 0.0;
      for (int k = 0; k < 64; ++k) s += H[i * 64 + k] * H[j * 64 + k];
      CHECK(fabs(s - (i == j ? 1.0 : 0.0)) < 1e-12);
    }
  free(H);
  double s[5] = {0.3, -1.0, 2.0, -INFINITY, 0.0}, p[5];
  ora_softmax_row(s, 5, 0.7, p);
  CHECK(fabs(p[0] + p[1] + p[2] + p[3] + p[4] - 1.0) < 1e-12 && p[3] == 0.0);
  ora_softmax_row(s, 1, 1.0, p);
  CHECK(p[0] == 1.0);
  for (int d = 16; d <= 128; d *= 2)
    for (int b = 1; b <= 4; ++b) scalar_codec(d, b);
  pq_codec(8, 256);
  pq_codec(4, 16);
  for (int b = 2; b <= 4; ++b) {
    pot_codec(b, 0);
    if (b >= 3) pot_codec(b, 1);
  }
  printf("%s: %d failed check(s)\n", n_fail ? "FAIL" : "OK", n_fail);
  return n_fail ? 1 : 0;
}
