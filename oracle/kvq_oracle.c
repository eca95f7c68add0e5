/*
 * kvq_oracle.c -- plain, slow, fp64 CPU oracle for attention computed from
 * quantized key-cache codes.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the GPU library is
 * compared against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code, header, table or constant with
 * the HIP library and must never be linked into it.
 *
 * Sources (web pages, cited by title and section):
 *   [AX]  "AXELRAM: Quantize Once, Never Dequantize" -- Key Points and Abstract.
 *         Keys are rotated by an orthogonal transform on write, which makes every
 *         coordinate of the rotated unit vector close to N(0, 1/d); a codebook fixed
 *         at design time, depending only on d and the bit width b, quantizes each
 *         coordinate; on read the query is rotated once and scores come from table
 *         lookups over the stored indices, with no inverse transform.  A +-1 sign
 *         pattern is part of the transform.
 *   [LK]  "LOOKAT: Lookup-Optimized Key-Attention" summary page -- AI Summary and
 *         Abstract.  Product quantization: keys split into m subspaces, a learned
 *         codebook per subspace, scores by asymmetric distance computation
 *         (inner products of query sub-vectors with centroids, read from a table).
 *   [SA]  Shift-accumulate attention page (arxivdaily 2609.09208) -- English
 *         abstract: online softmax in a fused decode-attention kernel.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   - transform = normalised Sylvester Walsh-Hadamard matrix H (entries
 *     (-1)^popcount(i&j)/sqrt(d)) applied after the diagonal sign pattern D;
 *   - codebook = Lloyd-Max quantizer of N(0,1) divided by sqrt(d);
 *     thresholds = midpoints of adjacent levels;
 *   - code_i = number of thresholds t_j with t_j <= y_i (a value exactly on a
 *     threshold takes the upper code);
 *   - codes are packed LSB-first: code i occupies bits [i*b, i*b+b) of the key's
 *     byte row, bit 0 of byte 0 first;
 *   - a zero key has norm 0 and codes of the zero vector;
 *   - a key with an infinite or NaN element has no unit vector: it gets the
 *     codes of the zero vector too, and its norm is what its sum of squares
 *     gives (+inf when an element is infinite and none is NaN, NaN when an
 *     element is NaN).  Every finite key is encoded from its exact unit vector,
 *     however large or small its elements;
 *   - scores are raw estimates of q.k; softmax uses scale 1/sqrt(d) passed in;
 *   - grouped-query mapping: query head h reads kv head h / (Hq/Hkv);
 *   - an empty sequence (length 0) gives an all-zero attention output;
 *   - quantized values: a value row is encoded exactly as a key is, and the
 *     attention output uses the dequantized rows ||v|| D H^T c_hat;
 *   - sign-pattern selection ranks a candidate by the attention-output error
 *     sum ||o_hat - o||^2 / sum ||o||^2 over all calibration rows (the pages
 *     rank by perplexity, which needs a model); ties go to the lowest index.
 *   - power-of-two key codec ([SA] English abstract): a key element is stored
 *     as a sign and the index j of a magnitude in a fixed descending set, times
 *     a per-key scale alpha = max_i |k_i| (so every shift index is >= 0);
 *     b bits = 1 sign bit (the top bit of the field) + b-1 index bits.  Plain
 *     set: 2^-j.  With the one-term mantissa extension: 2^-(j/2) for even j and
 *     2^-(j+1)/2 + 2^-(j+3)/2 = (3/4) 2^-(j-1)/2 for odd j.  The index is the
 *     magnitude nearest to |k_i| / alpha in value (ties to the larger); there is
 *     no zero magnitude; a zero key has alpha 0 and all codes 0.  No rotation.
 *
 * Everything is fp64.  Inputs arrive as double arrays (fp16/fp32 convert
 * exactly).  No blocking, no fusion, no reordering beyond the definitions.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif
#ifndef M_SQRT2
#define M_SQRT2 1.41421356237309504880
#endif

/* ------------------------------------------------------------------------- */
/* Lloyd-Max quantizer for the standard normal.                              */
/* [AX] Abstract: the optimal quantizer depends only on d and b because the  */
/* rotated coordinates follow N(0, 1/d).  The Lloyd-Max conditions: every    */
/* level is the conditional mean of its cell, every threshold the midpoint   */
/* of its two neighbouring levels.                                           */
/* ------------------------------------------------------------------------- */

static double std_normal_pdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }

/* P(a <= X < b) for X ~ N(0,1), each tail taken from erfc so that cells far
 * out in a tail do not lose their mass to cancellation. */
static double std_normal_mass(double a, double b) {
  if (a >= 0.0) return 0.5 * (erfc(a / M_SQRT2) - erfc(b / M_SQRT2));
  if (b <= 0.0) return 0.5 * (erfc(-b / M_SQRT2) - erfc(-a / M_SQRT2));
  return 1.0 - 0.5 * erfc(b / M_SQRT2) - 0.5 * erfc(-a / M_SQRT2);
}

/* Levels c[L] (ascending) and thresholds t[L-1] of the Lloyd-Max quantizer for
 * N(0,1), L = 2^b.  Returns the number of iterations used (negative if the
 * iteration cap was hit). */
int ora_lloyd_max_unit(int b, double* c, double* t) {
  const int L = 1 << b;
  /* Start from evenly spaced levels on [-3, 3]; the normal density is
   * log-concave, so the fixed point does not depend on the start. */
  for (int j = 0; j < L; ++j) c[j] = -3.0 + 6.0 * (j + 0.5) / L;
  int it;
  const int max_it = 2000000;
  for (it = 1; it <= max_it; ++it) {
    for (int j = 1; j < L; ++j) t[j - 1] = 0.5 * (c[j - 1] + c[j]);
    double delta = 0.0;
    for (int j = 0; j < L; ++j) {
      double lo = (j == 0) ? -INFINITY : t[j - 1];
      double hi = (j == L - 1) ? INFINITY : t[j];
      double num = std_normal_pdf(lo) - std_normal_pdf(hi); /* integral of x*phi(x) over the cell */
      double den = std_normal_mass(lo, hi);
      double cj = num / den;
      double dj = fabs(cj - c[j]);
      if (dj > delta) delta = dj;
      c[j] = cj;
    }
    if (delta < 1e-15) break;
  }
  /* The density is symmetric, so the exact quantizer is too; remove the last
   * rounding asymmetry so that the middle threshold is exactly 0. */
  for (int j = 0; j < L / 2; ++j) {
    double s = 0.5 * (c[L - 1 - j] - c[j]);
    c[L - 1 - j] = s;
    c[j] = -s;
  }
  for (int j = 1; j < L; ++j) t[j - 1] = 0.5 * (c[j - 1] + c[j]);
  return it > max_it ? -max_it : it;
}

/* Codebook for N(0, 1/d): the unit quantizer scaled by 1/sqrt(d). */
int ora_codebook(int d, int b, double* levels, double* thresholds) {
  const int L = 1 << b;
  int it = ora_lloyd_max_unit(b, levels, thresholds);
  const double s = 1.0 / sqrt((double)d);
  for (int j = 0; j < L; ++j) levels[j] *= s;
  for (int j = 0; j < L - 1; ++j) thresholds[j] *= s;
  return it;
}

/* Mean squared error of a quantizer (levels c, thresholds t) for N(0,1),
 * from the closed-form cell integrals:
 *   int_a^b (x-c)^2 phi = [P + a phi(a) - b phi(b)] - 2c[phi(a)-phi(b)] + c^2 P. */
double ora_quantizer_mse_unit(int b, const double* c, const double* t) {
  const int L = 1 << b;
  double mse = 0.0;
  for (int j = 0; j < L; ++j) {
    double lo = (j == 0) ? -INFINITY : t[j - 1];
    double hi = (j == L - 1) ? INFINITY : t[j];
    double P = std_normal_mass(lo, hi);
    double plo = std_normal_pdf(lo), phi_ = std_normal_pdf(hi);
    double alo = isinf(lo) ? 0.0 : lo * plo;
    double ahi = isinf(hi) ? 0.0 : hi * phi_;
    double second = P + alo - ahi;
    double first = plo - phi_;
    mse += second - 2.0 * c[j] * first + c[j] * c[j] * P;
  }
  return mse;
}

/* ------------------------------------------------------------------------- */
/* The orthogonal transform: H (normalised Walsh-Hadamard) times D (signs).  */
/* [AX] Key Points / Abstract: orthogonal-transform quantization with a sign */
/* pattern.  Written as an explicit d x d matrix product, no fast transform. */
/* ------------------------------------------------------------------------- */

static int popcount_u32(uint32_t x) {
  int n = 0;
  while (x) { n += (int)(x & 1u); x >>= 1; }
  return n;
}

/* H[i*d + j] = (-1)^popcount(i & j) / sqrt(d). */
void ora_hadamard(int d, double* H) {
  const double s = 1.0 / sqrt((double)d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j)
      H[(size_t)i * d + j] = (popcount_u32((uint32_t)(i & j)) & 1) ? -s : s;
}

/* out = H * (D .* x), with D = diag(signs). */
static void rotate(int d, const double* H, const int8_t* signs, const double* x, double* out) {
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc += H[(size_t)i * d + j] * ((double)signs[j] * x[j]);
    out[i] = acc;
  }
}

/* q' = H D q for one query of length d.  [AX] Abstract: the query is
 * transformed once; the keys are never transformed back. */
void ora_rotate_query(int d, const int8_t* signs, const double* q, double* qrot) {
  double* H = (double*)malloc(sizeof(double) * (size_t)d * d);
  ora_hadamard(d, H);
  rotate(d, H, signs, q, qrot);
  free(H);
}

/* ------------------------------------------------------------------------- */
/* Write path.  [AX] Abstract "transform on write": store the key's norm and  */
/* the b-bit indices of its rotated unit vector.                             */
/* ------------------------------------------------------------------------- */

/* Index of y in the codebook: the number of thresholds that are <= y. */
static int quantize_index(int L, const double* t, double y) {
  int code = 0;
  for (int j = 0; j < L - 1; ++j)
    if (t[j] <= y) code += 1;
  return code;
}

/* Write code (b bits) for coordinate i into a zeroed LSB-first bit row. */
static void put_code(uint8_t* row, int i, int b, int code) {
  for (int k = 0; k < b; ++k) {
    int bit = i * b + k;
    if ((code >> k) & 1) row[bit >> 3] |= (uint8_t)(1u << (bit & 7));
  }
}

static int get_code(const uint8_t* row, int i, int b) {
  int code = 0;
  for (int k = 0; k < b; ++k) {
    int bit = i * b + k;
    code |= ((row[bit >> 3] >> (bit & 7)) & 1) << k;
  }
  return code;
}

/* Encode n keys [n][d].  codes: [n][d*b/8] bytes, norms: [n].
 * Optional outputs (may be NULL): y_out [n][d] rotated unit coordinates;
 * tie [n][d] = 1 where |y_i - t_j| < tie_eps for some threshold t_j.
 * thresholds: the L-1 codebook thresholds for N(0,1/d). */
void ora_encode_keys(int d, int b, const double* thresholds, const int8_t* signs,
                     const double* keys, int64_t n, uint8_t* codes, double* norms,
                     double* y_out, uint8_t* tie, double tie_eps) {
  const int L = 1 << b;
  const int bpk = d * b / 8;
  double* H = (double*)malloc(sizeof(double) * (size_t)d * d);
  double* u = (double*)malloc(sizeof(double) * (size_t)d);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  ora_hadamard(d, H);
  for (int64_t r = 0; r < n; ++r) {
    const double* k = keys + (size_t)r * d;
    double ss = 0.0;
    int finite = 1;
    for (int i = 0; i < d; ++i) {
      ss += k[i] * k[i];
      if (!isfinite(k[i])) finite = 0;
    }
    double nrm = sqrt(ss);
    norms[r] = nrm;
    /* no unit vector for a zero key or one with an infinite or NaN element: y = 0 */
    for (int i = 0; i < d; ++i) u[i] = (finite && nrm > 0.0) ? k[i] / nrm : 0.0;
    rotate(d, H, signs, u, y);
    uint8_t* row = codes + (size_t)r * bpk;
    memset(row, 0, (size_t)bpk);
    for (int i = 0; i < d; ++i) {
      put_code(row, i, b, quantize_index(L, thresholds, y[i]));
      if (y_out) y_out[(size_t)r * d + i] = y[i];
      if (tie) {
        uint8_t f = 0;
        for (int j = 0; j < L - 1; ++j)
          if (fabs(y[i] - thresholds[j]) < tie_eps) f = 1;
        tie[(size_t)r * d + i] = f;
      }
    }
  }
  free(y);
  free(u);
  free(H);
}

/* Unpack rows of codes into integer indices [n][d]. */
void ora_unpack_codes(int d, int b, const uint8_t* codes, int64_t n, int32_t* idx) {
  const int bpk = d * b / 8;
  for (int64_t r = 0; r < n; ++r)
    for (int i = 0; i < d; ++i) idx[(size_t)r * d + i] = get_code(codes + (size_t)r * bpk, i, b);
}

/* ------------------------------------------------------------------------- */
/* Read path.  [AX] Abstract "table-lookup on read with no inverse           */
/* transform": LUT[i][j] = q'_i * c_j, score = ||k|| * sum_i LUT[i][code_i]. */
/* ------------------------------------------------------------------------- */

/* LUT [d][L] for one rotated query. */
void ora_build_lut(int d, int b, const double* levels, const double* qrot, double* lut) {
  const int L = 1 << b;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < L; ++j) lut[(size_t)i * L + j] = qrot[i] * levels[j];
}

/* Score of one key row from a LUT. */
static double lut_score(int d, int b, const double* lut, const uint8_t* row, double nrm) {
  const int L = 1 << b;
  double acc = 0.0;
  for (int i = 0; i < d; ++i) acc += lut[(size_t)i * L + get_code(row, i, b)];
  return nrm * acc;
}

static int64_t seq_len_of(const int32_t* seq_lens, int bi, int64_t T) {
  return seq_lens ? (int64_t)seq_lens[bi] : T;
}

/* Raw scores [B][Hq][Tcap] from codes [B][Hkv][Tcap][d*b/8] and norms
 * [B][Hkv][Tcap].  Positions t >= seq_len[b] are set to -inf. */
void ora_scores(int d, int b, const double* levels, const int8_t* signs, const double* q,
                const uint8_t* codes, const double* norms, int B, int Hq, int Hkv, int64_t Tcap,
                const int32_t* seq_lens, double* scores) {
  const int L = 1 << b;
  const int bpk = d * b / 8;
  const int G = Hq / Hkv;
  double* qrot = (double*)malloc(sizeof(double) * (size_t)d);
  double* lut = (double*)malloc(sizeof(double) * (size_t)d * L);
  for (int bi = 0; bi < B; ++bi) {
    const int64_t len = seq_len_of(seq_lens, bi, Tcap);
    for (int h = 0; h < Hq; ++h) {
      const int kvh = h / G;
      ora_rotate_query(d, signs, q + ((size_t)bi * Hq + h) * d, qrot);
      ora_build_lut(d, b, levels, qrot, lut);
      double* srow = scores + ((size_t)bi * Hq + h) * Tcap;
      for (int64_t t = 0; t < Tcap; ++t) {
        if (t >= len) { srow[t] = -INFINITY; continue; }
        size_t key = ((size_t)bi * Hkv + kvh) * Tcap + t;
        srow[t] = lut_score(d, b, lut, codes + key * bpk, norms[key]);
      }
    }
  }
  free(lut);
  free(qrot);
}

/* Softmax of scale*s over the first len entries followed by the weighted sum of
 * value rows v[t][d]: two passes (maximum, then exponentials), fp64.
 * [SA] English abstract: fused decode attention with softmax and the AV
 * product.  len == 0 gives zeros. */
static void softmax_av(int d, const double* s, int64_t len, double scale, const double* v, double* out) {
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  if (len <= 0) return;
  double m = -INFINITY;
  for (int64_t t = 0; t < len; ++t)
    if (scale * s[t] > m) m = scale * s[t];
  double l = 0.0;
  for (int64_t t = 0; t < len; ++t) {
    double p = exp(scale * s[t] - m);
    l += p;
    for (int c = 0; c < d; ++c) out[c] += p * v[(size_t)t * d + c];
  }
  for (int c = 0; c < d; ++c) out[c] /= l;
}

/* Softmax probabilities of scale*s over one row (for row-sum checks). */
void ora_softmax_row(const double* s, int64_t len, double scale, double* p) {
  double m = -INFINITY;
  for (int64_t t = 0; t < len; ++t)
    if (scale * s[t] > m) m = scale * s[t];
  double l = 0.0;
  for (int64_t t = 0; t < len; ++t) { p[t] = exp(scale * s[t] - m); l += p[t]; }
  for (int64_t t = 0; t < len; ++t) p[t] /= l;
}

/* Decode attention: out [B][Hq][d] = softmax(scale * scores) . V, with V
 * [B][Hkv][Tcap][d] and the scores of ora_scores. */
void ora_decode_attn(int d, int b, const double* levels, const int8_t* signs, const double* q,
                     const uint8_t* codes, const double* norms, const double* v, int B, int Hq,
                     int Hkv, int64_t Tcap, const int32_t* seq_lens, double scale, double* out) {
  const int G = Hq / Hkv;
  double* s = (double*)malloc(sizeof(double) * (size_t)B * Hq * (Tcap > 0 ? Tcap : 1));
  ora_scores(d, b, levels, signs, q, codes, norms, B, Hq, Hkv, Tcap, seq_lens, s);
  for (int bi = 0; bi < B; ++bi) {
    const int64_t len = seq_len_of(seq_lens, bi, Tcap);
    for (int h = 0; h < Hq; ++h) {
      const int kvh = h / G;
      softmax_av(d, s + ((size_t)bi * Hq + h) * Tcap, len, scale,
                 v + ((size_t)bi * Hkv + kvh) * Tcap * d, out + ((size_t)bi * Hq + h) * d);
    }
  }
  free(s);
}

/* ------------------------------------------------------------------------- */
/* Values quantized with the key codec.  [AX] Abstract quantizes keys only;  */
/* [SA] English abstract quantizes values too, in its own codec.  Reading:   */
/* a value row is encoded exactly as a key is (its norm and the b-bit codes  */
/* of H D v / ||v||, ora_encode_keys), and attention uses the dequantized    */
/* rows v_hat = ||v|| (H D)^T c_hat = ||v|| D H^T c_hat.                     */
/* ------------------------------------------------------------------------- */

/* Dequantize n rows: out[r] = norms[r] * D * H^T * c_hat(row r), with
 * c_hat_i = levels[code_i], as an explicit matrix product. */
void ora_dequant_rows(int d, int b, const double* levels, const int8_t* signs, const uint8_t* codes,
                      const double* norms, int64_t n, double* out) {
  const int bpk = d * b / 8;
  double* H = (double*)malloc(sizeof(double) * (size_t)d * d);
  double* c = (double*)malloc(sizeof(double) * (size_t)d);
  ora_hadamard(d, H);
  for (int64_t r = 0; r < n; ++r) {
    const uint8_t* row = codes + (size_t)r * bpk;
    for (int i = 0; i < d; ++i) c[i] = levels[get_code(row, i, b)];
    for (int j = 0; j < d; ++j) {
      double acc = 0.0; /* (H^T c)_j = sum_i H[i][j] c_i */
      for (int i = 0; i < d; ++i) acc += H[(size_t)i * d + j] * c[i];
      out[(size_t)r * d + j] = norms[r] * (double)signs[j] * acc;
    }
  }
  free(c);
  free(H);
}

/* Decode attention with quantized values: the keys score as in
 * ora_decode_attn, and V is the dequantized cache of (vcodes, vnorms). */
void ora_decode_attn_qv(int d, int b, const double* levels, const int8_t* signs, const double* q,
                        const uint8_t* codes, const double* norms, const uint8_t* vcodes,
                        const double* vnorms, int B, int Hq, int Hkv, int64_t Tcap,
                        const int32_t* seq_lens, double scale, double* out) {
  const int64_t rows = (int64_t)B * Hkv * Tcap;
  double* v = (double*)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * d);
  ora_dequant_rows(d, b, levels, signs, vcodes, vnorms, rows, v);
  ora_decode_attn(d, b, levels, signs, q, codes, norms, v, B, Hq, Hkv, Tcap, seq_lens, scale, out);
  free(v);
}

/* ------------------------------------------------------------------------- */
/* Sign-pattern selection.  [AX] Key Points / Abstract: the sign pattern D   */
/* is chosen once, without gradients, among candidate patterns evaluated on  */
/* a few calibration samples (the pages use 200 candidates and 8 samples).  */
/* The pages rank candidates by perplexity, which needs a model; here each   */
/* candidate is ranked by the error it causes in the attention output.       */
/* ------------------------------------------------------------------------- */

/* Exact attention, no quantization: out [n][Hq][d] = softmax(scale * q.k_t)
 * V over all T keys, q [n][Hq][d], keys and v [n][Hkv][T][d]. */
void ora_exact_attn(int d, const double* q, const double* keys, const double* v, int n, int Hq, int Hkv,
                    int64_t T, double scale, double* out) {
  const int G = Hq / Hkv;
  double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  for (int bi = 0; bi < n; ++bi)
    for (int h = 0; h < Hq; ++h) {
      const int kvh = h / G;
      const double* qh = q + ((size_t)bi * Hq + h) * d;
      const double* kk = keys + ((size_t)bi * Hkv + kvh) * T * d;
      for (int64_t t = 0; t < T; ++t) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += qh[i] * kk[(size_t)t * d + i];
        s[t] = acc;
      }
      softmax_av(d, s, T, scale, v + ((size_t)bi * Hkv + kvh) * T * d, out + ((size_t)bi * Hq + h) * d);
    }
  free(s);
}

/* For every candidate pattern c (cands [C][d], each entry +-1): encode the
 * calibration keys with it, store the norms as fp32 (as the cache does), run
 * decode attention from the codes, and set
 *   errors[c] = sum over rows ||o_hat - o||^2 / sum over rows ||o||^2,
 * rows = every (sample, query head), o = exact attention.  Returns the index
 * of the smallest error; ties go to the lowest index. */
int ora_sign_errors(int d, int b, const double* levels, const double* thresholds, const int8_t* cands, int C,
                    const double* q, const double* keys, const double* v, int n, int Hq, int Hkv, int64_t T,
                    double scale, double* errors) {
  const size_t nkeys = (size_t)n * Hkv * T;
  const size_t nout = (size_t)n * Hq * d;
  uint8_t* codes = (uint8_t*)malloc((size_t)d * b / 8 * (nkeys > 0 ? nkeys : 1));
  double* norms = (double*)malloc(sizeof(double) * (nkeys > 0 ? nkeys : 1));
  double* o = (double*)malloc(sizeof(double) * nout);
  double* oh = (double*)malloc(sizeof(double) * nout);
  ora_exact_attn(d, q, keys, v, n, Hq, Hkv, T, scale, o);
  double den = 0.0;
  for (size_t i = 0; i < nout; ++i) den += o[i] * o[i];
  int best = 0;
  for (int c = 0; c < C; ++c) {
    const int8_t* sg = cands + (size_t)c * d;
    ora_encode_keys(d, b, thresholds, sg, keys, (int64_t)nkeys, codes, norms, NULL, NULL, 0.0);
    for (size_t r = 0; r < nkeys; ++r) norms[r] = (double)(float)norms[r];
    ora_decode_attn(d, b, levels, sg, q, codes, norms, v, n, Hq, Hkv, T, NULL, scale, oh);
    double num = 0.0;
    for (size_t i = 0; i < nout; ++i) num += (oh[i] - o[i]) * (oh[i] - o[i]);
    errors[c] = den > 0.0 ? num / den : 0.0;
    if (errors[c] < errors[best]) best = c;
  }
  free(oh);
  free(o);
  free(norms);
  free(codes);
  return best;
}

/* ------------------------------------------------------------------------- */
/* Product quantization with asymmetric distance computation.                */
/* [LK] AI Summary / Abstract: split keys into m subspaces, learn a codebook */
/* per subspace, score through lookup tables of query-centroid products.     */
/* ------------------------------------------------------------------------- */

/* Nearest centroid by squared L2 distance; ties go to the lowest index.
 * gap (may be NULL) = second-smallest minus smallest distance. */
static int nearest(const double* x, const double* cent, int K, int ds, double* gap) {
  int best = 0;
  double bd = INFINITY, second = INFINITY;
  for (int c = 0; c < K; ++c) {
    double dist = 0.0;
    for (int k = 0; k < ds; ++k) {
      double e = x[k] - cent[(size_t)c * ds + k];
      dist += e * e;
    }
    if (dist < bd) { second = bd; bd = dist; best = c; }
    else if (dist < second) second = dist;
  }
  if (gap) *gap = second - bd;
  return best;
}

/* Lloyd's k-means on n training vectors [n][ds] (one head, one subspace).
 * init_rows[K]: rows of the training set used as the starting centroids
 * (drawn by the caller).  Each iteration assigns every vector to its nearest
 * centroid, then moves every centroid to the mean of its members; a centroid
 * with no members stays where it is.  objective (may be NULL, [iters+1]) gets
 * the mean squared distance before each iteration and after the last. */
void ora_kmeans(const double* train, int64_t n, int ds, int K, int iters, const int64_t* init_rows,
                double* cent, double* objective) {
  int32_t* assign = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  double* sum = (double*)malloc(sizeof(double) * (size_t)K * ds);
  int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * (size_t)K);
  for (int c = 0; c < K; ++c)
    for (int k = 0; k < ds; ++k) cent[(size_t)c * ds + k] = train[(size_t)init_rows[c] * ds + k];
  for (int it = 0; it <= iters; ++it) {
    double obj = 0.0;
    for (int64_t r = 0; r < n; ++r) {
      double gap;
      int c = nearest(train + (size_t)r * ds, cent, K, ds, &gap);
      assign[r] = c;
      double dist = 0.0;
      for (int k = 0; k < ds; ++k) {
        double e = train[(size_t)r * ds + k] - cent[(size_t)c * ds + k];
        dist += e * e;
      }
      obj += dist;
    }
    if (objective) objective[it] = n > 0 ? obj / (double)n : 0.0;
    if (it == iters) break;
    for (size_t x = 0; x < (size_t)K * ds; ++x) sum[x] = 0.0;
    for (int c = 0; c < K; ++c) cnt[c] = 0;
    for (int64_t r = 0; r < n; ++r) {
      cnt[assign[r]] += 1;
      for (int k = 0; k < ds; ++k) sum[(size_t)assign[r] * ds + k] += train[(size_t)r * ds + k];
    }
    for (int c = 0; c < K; ++c)
      if (cnt[c] > 0)
        for (int k = 0; k < ds; ++k) cent[(size_t)c * ds + k] = sum[(size_t)c * ds + k] / (double)cnt[c];
  }
  free(cnt);
  free(sum);
  free(assign);
}

/* PQ encode of n keys [n][d] for one head: code_s = nearest centroid of
 * sub-vector s.  cent [m][K][d/m]; codes [n][m*cbits/8]: code s in bits
 * [s*cbits, s*cbits+cbits) of the key's row, LSB first (cbits = 8: one byte
 * per subspace; cbits = 4, for K <= 16: two subspaces per byte, the even one
 * in the low nibble); gap (may be NULL) [n][m]. */
void ora_pq_encode(int d, int m, int K, int cbits, const double* cent, const double* keys, int64_t n,
                   uint8_t* codes, double* gap) {
  const int ds = d / m;
  const int bpk = m * cbits / 8;
  for (int64_t r = 0; r < n; ++r) {
    uint8_t* row = codes + (size_t)r * bpk;
    memset(row, 0, (size_t)bpk);
    for (int s = 0; s < m; ++s) {
      double g;
      int c = nearest(keys + (size_t)r * d + (size_t)s * ds, cent + (size_t)s * K * ds, K, ds, &g);
      put_code(row, s, cbits, c);
      if (gap) gap[(size_t)r * m + s] = g;
    }
  }
}

/* PQ scores [B][Hq][Tcap]: LUT[s][c] = q_s . C_{s,c}, score = sum_s LUT[s][code_s].
 * cent [Hkv][m][K][d/m]; codes [B][Hkv][Tcap][m*cbits/8] as ora_pq_encode
 * writes them.  No rotation, no norm. */
void ora_pq_scores(int d, int m, int K, int cbits, const double* cent, const double* q, const uint8_t* codes,
                   int B, int Hq, int Hkv, int64_t Tcap, const int32_t* seq_lens, double* scores) {
  const int ds = d / m;
  const int bpk = m * cbits / 8;
  const int G = Hq / Hkv;
  double* lut = (double*)malloc(sizeof(double) * (size_t)m * K);
  for (int bi = 0; bi < B; ++bi) {
    const int64_t len = seq_len_of(seq_lens, bi, Tcap);
    for (int h = 0; h < Hq; ++h) {
      const int kvh = h / G;
      const double* qh = q + ((size_t)bi * Hq + h) * d;
      const double* ch = cent + (size_t)kvh * m * K * ds;
      for (int s = 0; s < m; ++s)
        for (int c = 0; c < K; ++c) {
          double acc = 0.0;
          for (int k = 0; k < ds; ++k) acc += qh[s * ds + k] * ch[((size_t)s * K + c) * ds + k];
          lut[(size_t)s * K + c] = acc;
        }
      double* srow = scores + ((size_t)bi * Hq + h) * Tcap;
      for (int64_t t = 0; t < Tcap; ++t) {
        if (t >= len) { srow[t] = -INFINITY; continue; }
        const uint8_t* row = codes + (((size_t)bi * Hkv + kvh) * Tcap + t) * bpk;
        double acc = 0.0;
        for (int s = 0; s < m; ++s) acc += lut[(size_t)s * K + get_code(row, s, cbits)];
        srow[t] = acc;
      }
    }
  }
  free(lut);
}

/* PQ decode attention: softmax(scale * PQ scores) . V. */
void ora_pq_decode_attn(int d, int m, int K, int cbits, const double* cent, const double* q, const uint8_t* codes,
                        const double* v, int B, int Hq, int Hkv, int64_t Tcap, const int32_t* seq_lens,
                        double scale, double* out) {
  const int G = Hq / Hkv;
  double* s = (double*)malloc(sizeof(double) * (size_t)B * Hq * (Tcap > 0 ? Tcap : 1));
  ora_pq_scores(d, m, K, cbits, cent, q, codes, B, Hq, Hkv, Tcap, seq_lens, s);
  for (int bi = 0; bi < B; ++bi) {
    const int64_t len = seq_len_of(seq_lens, bi, Tcap);
    for (int h = 0; h < Hq; ++h) {
      const int kvh = h / G;
      softmax_av(d, s + ((size_t)bi * Hq + h) * Tcap, len, scale,
                 v + ((size_t)bi * Hkv + kvh) * Tcap * d, out + ((size_t)bi * Hq + h) * d);
    }
  }
  free(s);
}

/* ------------------------------------------------------------------------- */
/* Power-of-two key codec.  [SA] English abstract: the key cache holds a     */
/* signed power-of-two code per element, so that each product in q.k is a    */
/* sign flip and a shift; a sub-power mantissa term adds one more shift for   */
/* half the error.  Readings: see the header.                                 */
/* ------------------------------------------------------------------------- */

/* Shift amounts that make up magnitude j: returns their count (1 or 2). */
static int pot_shifts(int mant, int j, int* r) {
  if (!mant) { r[0] = j; return 1; }
  if (j % 2 == 0) { r[0] = j / 2; return 1; }
  r[0] = (j + 1) / 2;
  r[1] = (j + 3) / 2;
  return 2;
}

/* Magnitudes [2^(b-1)] (descending) and the midpoints between neighbours
 * [2^(b-1) - 1]. */
void ora_pot_levels(int b, int mant, double* mags, double* thresholds) {
  const int n = 1 << (b - 1);
  for (int j = 0; j < n; ++j) {
    int r[2];
    const int c = pot_shifts(mant, j, r);
    mags[j] = 0.0;
    for (int k = 0; k < c; ++k) mags[j] += ldexp(1.0, -r[k]);
  }
  for (int j = 0; j + 1 < n; ++j) thresholds[j] = 0.5 * (mags[j] + mags[j + 1]);
}

/* Encode n keys [n][d] into codes [n][d*b/8] (LSB-first b-bit fields: index
 * in the low b-1 bits, sign in the top bit) and scales [n] = max_i |k_i|.
 * tie [n][d] (may be NULL) = 1 where |k_i| lies within tie_eps * alpha of a
 * midpoint times alpha. */
void ora_pot_encode(int d, int b, int mant, const double* keys, int64_t n, uint8_t* codes, double* scales,
                    uint8_t* tie, double tie_eps) {
  const int nm = 1 << (b - 1);
  const int bpk = d * b / 8;
  double mags[8], thr[7];
  ora_pot_levels(b, mant, mags, thr);
  for (int64_t r = 0; r < n; ++r) {
    const double* k = keys + (size_t)r * d;
    double alpha = 0.0;
    for (int i = 0; i < d; ++i)
      if (fabs(k[i]) > alpha) alpha = fabs(k[i]);
    scales[r] = alpha;
    uint8_t* row = codes + (size_t)r * bpk;
    memset(row, 0, (size_t)bpk);
    for (int i = 0; i < d; ++i) {
      int j = 0, sgn = 0;
      uint8_t f = 0;
      if (alpha > 0.0) {
        const double x = fabs(k[i]);
        for (int m = 0; m + 1 < nm; ++m) {
          if (x < thr[m] * alpha) j += 1;  /* below the midpoint: a smaller magnitude is nearer */
          if (fabs(x - thr[m] * alpha) < tie_eps * alpha) f = 1;
        }
        sgn = k[i] < 0.0 ? 1 : 0;
      }
      put_code(row, i, b, j | (sgn << (b - 1)));
      if (tie) tie[(size_t)r * d + i] = f;
    }
  }
}

/* Dequantized rows [n][d]: alpha * (-1)^sign * magnitude(j). */
void ora_pot_dequant(int d, int b, int mant, const uint8_t* codes, const double* scales, int64_t n, double* out) {
  const int bpk = d * b / 8;
  double mags[8], thr[7];
  ora_pot_levels(b, mant, mags, thr);
  for (int64_t r = 0; r < n; ++r)
    for (int i = 0; i < d; ++i) {
      const int c = get_code(codes + (size_t)r * bpk, i, b);
      const int j = c & ((1 << (b - 1)) - 1), sgn = c >> (b - 1);
      out[(size_t)r * d + i] = scales[r] * (sgn ? -mags[j] : mags[j]);
    }
}

/* Score of one key: alpha * sum_i of the query element, sign-flipped and
 * shifted right by each shift amount of the element's magnitude. */
static double pot_score(int d, int b, int mant, const double* q, const uint8_t* row, double alpha) {
  double acc = 0.0;
  for (int i = 0; i < d; ++i) {
    const int c = get_code(row, i, b);
    const int j = c & ((1 << (b - 1)) - 1);
    const double x = (c >> (b - 1)) ? -q[i] : q[i];
    int r[2];
    const int cnt = pot_shifts(mant, j, r);
    for (int k = 0; k < cnt; ++k) acc += ldexp(x, -r[k]);
  }
  return alpha * acc;
}

/* Raw scores [B][Hq][Tcap] from codes [B][Hkv][Tcap][d*b/8] and scales
 * [B][Hkv][Tcap]; positions t >= seq_len[b] are -inf. */
void ora_pot_scores(int d, int b, int mant, const double* q, const uint8_t* codes, const double* scales, int B,
                    int Hq, int Hkv, int64_t Tcap, const int32_t* seq_lens, double* scores) {
  const int bpk = d * b / 8;
  const int G = Hq / Hkv;
  for (int bi = 0; bi < B; ++bi) {
    const int64_t len = seq_len_of(seq_lens, bi, Tcap);
    for (int h = 0; h < Hq; ++h) {
      const double* qh = q + ((size_t)bi * Hq + h) * d;
      double* srow = scores + ((size_t)bi * Hq + h) * Tcap;
      for (int64_t t = 0; t < Tcap; ++t) {
        if (t >= len) { srow[t] = -INFINITY; continue; }
        const size_t key = ((size_t)bi * Hkv + h / G) * Tcap + t;
        srow[t] = pot_score(d, b, mant, qh, codes + key * bpk, scales[key]);
      }
    }
  }
}

/* Decode attention with power-of-two key codes: softmax(scale * scores) . V. */
void ora_pot_decode_attn(int d, int b, int mant, const double* q, const uint8_t* codes, const double* scales,
                         const double* v, int B, int Hq, int Hkv, int64_t Tcap, const int32_t* seq_lens,
                         double scale, double* out) {
  const int G = Hq / Hkv;
  double* s = (double*)malloc(sizeof(double) * (size_t)B * Hq * (Tcap > 0 ? Tcap : 1));
  ora_pot_scores(d, b, mant, q, codes, scales, B, Hq, Hkv, Tcap, seq_lens, s);
  for (int bi = 0; bi < B; ++bi) {
    const int64_t len = seq_len_of(seq_lens, bi, Tcap);
    for (int h = 0; h < Hq; ++h) {
      const double* vh = v + ((size_t)bi * Hkv + h / G) * Tcap * d;
      softmax_av(d, s + ((size_t)bi * Hq + h) * Tcap, len, scale, vh, out + ((size_t)bi * Hq + h) * d);
    }
  }
  free(s);
}
