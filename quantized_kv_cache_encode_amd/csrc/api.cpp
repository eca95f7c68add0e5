// Host side of the libkvq C ABI (include/kvq.h): argument validation, codebook
// construction, launch geometry and kernel dispatch.  No device memory is
// allocated here; every buffer belongs to the caller.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvq_status ok() {
  g_last_error.clear();
  return KVQ_OK;
}

kvq_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  if (e == hipErrorNotSupported) return fail(KVQ_ERR_UNSUPPORTED, "%s: this shape/dtype combination is not built", what);
  return fail(KVQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// The power-of-two codebook for (d, b, mantissa), arguments already checked: magnitudes 2^-j (or, with the
// mantissa term, 2^-(j/2) and (3/4) 2^-((j-1)/2) alternately), the signed level of every code value (sign in
// the top bit) and the midpoints of consecutive magnitudes.
void pot_codebook(int d, int b, int mantissa, kvq_codebook* out) {
  std::memset(out, 0, sizeof *out);
  const int nm = 1 << (b - 1);
  double mag[8];
  for (int j = 0; j < nm; ++j) mag[j] = mantissa ? std::ldexp(j % 2 ? 0.75 : 1.0, -(j / 2)) : std::ldexp(1.0, -j);
  for (int c = 0; c < 2 * nm; ++c) out->levels[c] = (float)(c >= nm ? -mag[c - nm] : mag[c]);
  for (int j = 0; j + 1 < nm; ++j) out->thresholds[j] = (float)(0.5 * (mag[j] + mag[j + 1]));
  out->kind = KVQ_POT;
  out->d = d;
  out->b = b;
  out->m = mantissa;
}

kvq_status check_codebook(const kvq_codebook* cb) {
  if (!cb) return fail(KVQ_ERR_INVALID_ARG, "codebook is NULL");
  if (cb->kind == KVQ_HADAMARD_LM) {
    if (!pow2(cb->d) || cb->d < 16 || cb->d > 256)
      return fail(KVQ_ERR_INVALID_ARG, "d=%d: must be a power of two in [16, 256]", cb->d);
    if (cb->b < 1 || cb->b > 4) return fail(KVQ_ERR_INVALID_ARG, "b=%d: must be 1..4", cb->b);
    return KVQ_OK;
  }
  if (cb->kind == KVQ_POT) {
    if (!pow2(cb->d) || cb->d < 16 || cb->d > 256)
      return fail(KVQ_ERR_INVALID_ARG, "d=%d: must be a power of two in [16, 256]", cb->d);
    if (cb->b < 2 || cb->b > 4) return fail(KVQ_ERR_INVALID_ARG, "power-of-two b=%d: must be 2..4", cb->b);
    if (cb->m != 0 && cb->m != 1) return fail(KVQ_ERR_INVALID_ARG, "power-of-two mantissa flag %d: must be 0 or 1", cb->m);
    // the kernels rely on the canonical levels and midpoints (powers of two, and 3/4 of them with the
    // mantissa term); anything else is rejected
    kvq_codebook ref;
    pot_codebook(cb->d, cb->b, cb->m, &ref);
    for (int c = 0; c < (2 << (cb->b - 1)); ++c)
      if (cb->levels[c] != ref.levels[c]) return fail(KVQ_ERR_INVALID_ARG, "power-of-two level %d is not canonical", c);
    for (int j = 0; j + 1 < (1 << (cb->b - 1)); ++j)
      if (cb->thresholds[j] != ref.thresholds[j])
        return fail(KVQ_ERR_INVALID_ARG, "power-of-two midpoint %d is not canonical", j);
    return KVQ_OK;
  }
  if (cb->kind == KVQ_PQ) {
    if (cb->d <= 0 || cb->m <= 0 || cb->d % cb->m != 0)
      return fail(KVQ_ERR_INVALID_ARG, "PQ d=%d, m=%d: m must divide d", cb->d, cb->m);
    if (cb->K < 2 || cb->K > 256) return fail(KVQ_ERR_INVALID_ARG, "PQ K=%d: must be 2..256", cb->K);
    if (cb->b != 8 && !(cb->b == 4 && cb->K <= 16 && cb->m % 2 == 0))
      return fail(KVQ_ERR_INVALID_ARG, "PQ code width b=%d: must be 8, or 4 with K <= 16 and an even m", cb->b);
    if (!cb->pq_centroids) return fail(KVQ_ERR_INVALID_ARG, "PQ centroids pointer is NULL");
    if (!aligned16(cb->pq_centroids)) return fail(KVQ_ERR_INVALID_ARG, "PQ centroids not 16-byte aligned");
    if (cb->n_heads <= 0) return fail(KVQ_ERR_INVALID_ARG, "PQ n_heads=%d", cb->n_heads);
    return KVQ_OK;
  }
  return fail(KVQ_ERR_INVALID_ARG, "unknown codebook kind %d", cb->kind);
}

int bytes_per_key(const kvq_codebook* cb) { return cb->kind == KVQ_PQ ? cb->m * cb->b / 8 : cb->d * cb->b / 8; }

kvq_status pack_signs(const int8_t* signs, int d, uint32_t out[8]) {
  for (int k = 0; k < 8; ++k) out[k] = 0;
  if (!signs) return fail(KVQ_ERR_INVALID_ARG, "signs is NULL");
  for (int i = 0; i < d; ++i) {
    if (signs[i] == -1) out[i >> 5] |= 1u << (i & 31);
    else if (signs[i] != 1) return fail(KVQ_ERR_INVALID_ARG, "signs[%d]=%d: must be +1 or -1", i, (int)signs[i]);
  }
  return KVQ_OK;
}

bool valid_dtype(int t) { return t == KVQ_F32 || t == KVQ_F16; }

// Largest power of two <= 8 dividing G: query heads served by one workgroup.
int heads_per_wg(int G) {
  for (int gg = 8; gg > 1; gg >>= 1)
    if (G % gg == 0) return gg;
  return 1;
}

// Compute units of the current device (256 on MI355X; also the fallback when
// no device can be queried, so that workspace sizes stay well defined).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

// Split of the token axis: every split is a multiple of 64 tokens.  With no
// request, aim for per_cu workgroups per compute unit (one round of the grid) but
// keep at least one 64-token chunk per wave in a split.  A launch that would
// then fill less than half the compute units with two or more splits per unit
// is all latency: there a split may hold half that, which halves each
// workgroup's serial part, up to about half the compute units (beyond that,
// and from one split to two, the merge costs more than the shorter splits
// save).  PQ decode (pq): every workgroup builds its head's whole table from the
// K centroids of every subspace, so a split repeats that work; there a split keeps
// at least four chunks per wave and the grid is not filled further (measured at
// the GPT-2-like shape, 48 units: unsplit fastest for 1024 and 2048 tokens, two
// splits for 4096).
void choose_splits(int64_t units, int64_t T_cap, int requested, int* n_splits, int64_t* split_len, int per_cu = 1,
                   bool pq = false) {
  const int64_t max_splits = (T_cap + 63) / 64;
  int64_t s;
  if (requested > 0) {
    s = requested < max_splits ? requested : max_splits;
  } else {
    const int64_t target = (int64_t)device_cus() * per_cu;
    s = (target + units - 1) / units;
    const int64_t min_tokens = (pq ? 4 : 1) * kvq::kReadThreads;  // 64 tokens (pq: 256) per wave
    int64_t cap = (T_cap + min_tokens - 1) / min_tokens;
    if (!pq && cap > 1 && units * cap < target / 2)
      cap = std::min((T_cap + min_tokens / 2 - 1) / (min_tokens / 2), (target / 2 + units - 1) / units);
    if (s > cap) s = cap;
    if (s < 1) s = 1;
  }
  if (s > 256) s = 256;  // the split merge keeps per-split scalars of a unit in LDS
  int64_t len = (T_cap + s - 1) / s;
  len = (len + 63) / 64 * 64;
  *split_len = len;
  *n_splits = (int)((T_cap + len - 1) / len);
}

struct ReadShape {
  int gg, n_groups;
  int64_t units;
};

kvq_status check_read(const kvq_codebook* cb, const int8_t* signs, const void* q, kvq_dtype qdtype,
                      const uint8_t* codes, const float* norms, int B, int Hq, int Hkv, int64_t T_cap,
                      kvq::AttnParams* p, ReadShape* rs) {
  kvq_status st = check_codebook(cb);
  if (st != KVQ_OK) return st;
  if (B <= 0 || Hq <= 0 || Hkv <= 0) return fail(KVQ_ERR_INVALID_ARG, "B=%d Hq=%d Hkv=%d must be positive", B, Hq, Hkv);
  if (Hq % Hkv != 0) return fail(KVQ_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (T_cap <= 0) return fail(KVQ_ERR_INVALID_ARG, "T_cap=%lld must be positive", (long long)T_cap);
  if ((int64_t)B * Hkv > 65535 * 8) return fail(KVQ_ERR_INVALID_ARG, "B*Hkv too large");
  // the kernels address a split's codes, norms and V and a unit's score rows with 32-bit byte offsets
  if (T_cap >= (((int64_t)1 << 31) / (4 * (int64_t)std::max(cb->d, 32))))
    return fail(KVQ_ERR_UNSUPPORTED, "T_cap=%lld too large for d=%d (32-bit offsets)", (long long)T_cap, cb->d);
  if (!valid_dtype(qdtype)) return fail(KVQ_ERR_INVALID_ARG, "bad q dtype %d", (int)qdtype);
  if (!q || !codes) return fail(KVQ_ERR_INVALID_ARG, "q or codes is NULL");
  if (!aligned16(q) || !aligned16(codes)) return fail(KVQ_ERR_INVALID_ARG, "q or codes not 16-byte aligned");
  std::memset(p, 0, sizeof *p);
  p->waves = 8;
  if (cb->kind == KVQ_HADAMARD_LM) {
    if (!norms) return fail(KVQ_ERR_INVALID_ARG, "norms is NULL");
    if (!aligned16(norms)) return fail(KVQ_ERR_INVALID_ARG, "norms not 16-byte aligned");
    st = pack_signs(signs, cb->d, p->signs);
    if (st != KVQ_OK) return st;
    for (int j = 0; j < 16; ++j) p->levels[j] = j < (1 << cb->b) ? cb->levels[j] : 0.0f;
  } else if (cb->kind == KVQ_POT) {
    if (!norms) return fail(KVQ_ERR_INVALID_ARG, "norms (per-key scales) is NULL");
    if (!aligned16(norms)) return fail(KVQ_ERR_INVALID_ARG, "norms not 16-byte aligned");
    for (int j = 0; j < 16; ++j) p->levels[j] = j < (1 << cb->b) ? cb->levels[j] : 0.0f;
  } else {
    if (cb->n_heads != Hkv) return fail(KVQ_ERR_INVALID_ARG, "PQ codebook has %d heads, Hkv=%d", cb->n_heads, Hkv);
    p->pq_cent = cb->pq_centroids;
    p->pq_K = cb->K;
  }
  const int G = Hq / Hkv;
  rs->gg = heads_per_wg(G);
  rs->n_groups = G / rs->gg;
  rs->units = (int64_t)B * Hkv * rs->n_groups;
  if (rs->units > 65535) return fail(KVQ_ERR_INVALID_ARG, "B*Hkv*(head groups)=%lld exceeds the grid", (long long)rs->units);
  p->q = q;
  p->q_f16 = qdtype == KVQ_F16;
  p->codes = codes;
  p->norms = norms;
  p->T_cap = T_cap;
  p->B = B;
  p->Hq = Hq;
  p->Hkv = Hkv;
  p->G = G;
  p->n_groups = rs->n_groups;
  return KVQ_OK;
}

// Workspace of a split decode: arrival counters (4 bytes per unit, padded to
// 256 bytes) followed by the fp32 partials [B][Hq][splits][d+4] (d accumulators,
// the running maximum and the sum, padded).
size_t workspace_bytes(int64_t units, int B, int Hq, int splits, int d) {
  if (splits <= 1) return 0;
  const size_t counters = ((size_t)units * 4 + 255) / 256 * 256;
  return counters + (size_t)B * Hq * splits * (d + 4) * sizeof(float);
}

}  // namespace

namespace kvq {
int set_error(int status, const char* msg) { return fail((kvq_status)status, "%s", msg); }
}  // namespace kvq

extern "C" {

int kvq_version(void) { return 100; }

const char* kvq_last_error(void) { return g_last_error.c_str(); }

kvq_status kvq_build_codebook(int d, int b, kvq_codebook* out) {
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out is NULL");
  if (!pow2(d) || d < 16 || d > 256) return fail(KVQ_ERR_INVALID_ARG, "d=%d: must be a power of two in [16, 256]", d);
  if (b < 1 || b > 4) return fail(KVQ_ERR_INVALID_ARG, "b=%d: must be 1..4", b);
  std::memset(out, 0, sizeof *out);
  double lv[16], th[15];
  kvq::lloyd_max_gaussian(b, lv, th);
  const double s = 1.0 / std::sqrt((double)d);
  const int L = 1 << b;
  for (int j = 0; j < L; ++j) out->levels[j] = (float)(lv[j] * s);
  for (int j = 0; j + 1 < L; ++j) out->thresholds[j] = (float)(th[j] * s);
  out->kind = KVQ_HADAMARD_LM;
  out->d = d;
  out->b = b;
  return ok();
}

kvq_status kvq_build_codebook_pot(int d, int b, int mantissa, kvq_codebook* out) {
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out is NULL");
  if (!pow2(d) || d < 16 || d > 256) return fail(KVQ_ERR_INVALID_ARG, "d=%d: must be a power of two in [16, 256]", d);
  if (b < 2 || b > 4) return fail(KVQ_ERR_INVALID_ARG, "b=%d: must be 2..4", b);
  if (mantissa != 0 && mantissa != 1) return fail(KVQ_ERR_INVALID_ARG, "mantissa=%d: must be 0 or 1", mantissa);
  pot_codebook(d, b, mantissa, out);
  return ok();
}

kvq_status kvq_build_codebook_pq(const float* train, int H, int64_t n, int d, int m, int K, int iters,
                                 const int64_t* start_rows, float* centroids) {
  if (!train || !start_rows || !centroids) return fail(KVQ_ERR_INVALID_ARG, "NULL pointer");
  if (H <= 0 || n <= 0 || d <= 0 || m <= 0 || d % m != 0)
    return fail(KVQ_ERR_INVALID_ARG, "H=%d n=%lld d=%d m=%d: need positive sizes and m | d", H, (long long)n, d, m);
  if (K < 2 || K > 256 || K > n) return fail(KVQ_ERR_INVALID_ARG, "K=%d: must be 2..256 and <= n", K);
  if (iters < 0) return fail(KVQ_ERR_INVALID_ARG, "iters=%d", iters);
  for (int64_t x = 0; x < (int64_t)H * m * K; ++x)
    if (start_rows[x] < 0 || start_rows[x] >= n)
      return fail(KVQ_ERR_INVALID_ARG, "start_rows[%lld]=%lld out of range", (long long)x, (long long)start_rows[x]);
  const int ds = d / m;
  std::vector<double> cent((size_t)K * ds);
  for (int h = 0; h < H; ++h)
    for (int s = 0; s < m; ++s) {
      kvq::kmeans_lloyd(train + (size_t)h * n * d + (size_t)s * ds, n, ds, d, K, iters,
                        start_rows + ((size_t)h * m + s) * K, cent.data());
      float* dst = centroids + ((size_t)h * m + s) * K * ds;
      for (size_t x = 0; x < cent.size(); ++x) dst[x] = (float)cent[x];
    }
  return ok();
}

kvq_status kvq_codebook_pq(int d, int m, int K, int n_heads, const float* centroids_device, kvq_codebook* out) {
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out is NULL");
  std::memset(out, 0, sizeof *out);
  out->kind = KVQ_PQ;
  out->d = d;
  out->m = m;
  out->K = K;
  out->b = K <= 16 && m % 2 == 0 ? 4 : 8;  // the narrowest code width that holds K centroids
  out->n_heads = n_heads;
  out->pq_centroids = centroids_device;
  kvq_status st = check_codebook(out);
  return st == KVQ_OK ? ok() : st;
}

kvq_status kvq_encode_keys(const kvq_codebook* cb, const int8_t* signs, const void* keys, kvq_dtype kdtype,
                           int B, int Hkv, int64_t T_new, uint8_t* codes, float* norms, int64_t T_cap, int64_t t0,
                           const int32_t* write_pos, void* stream) {
  kvq_status st = check_codebook(cb);
  if (st != KVQ_OK) return st;
  if (B <= 0 || Hkv <= 0 || T_new < 0 || T_cap <= 0)
    return fail(KVQ_ERR_INVALID_ARG, "B=%d Hkv=%d T_new=%lld T_cap=%lld out of range", B, Hkv, (long long)T_new,
                (long long)T_cap);
  if (!valid_dtype(kdtype)) return fail(KVQ_ERR_INVALID_ARG, "bad key dtype %d", (int)kdtype);
  if ((!keys && T_new > 0) || !codes) return fail(KVQ_ERR_INVALID_ARG, "keys or codes is NULL");
  if (!aligned16(keys) || !aligned16(codes)) return fail(KVQ_ERR_INVALID_ARG, "keys or codes not 16-byte aligned");
  if (!write_pos && (t0 < 0 || t0 + T_new > T_cap))
    return fail(KVQ_ERR_INVALID_ARG, "rows [%lld, %lld) do not fit T_cap=%lld", (long long)t0, (long long)(t0 + T_new),
                (long long)T_cap);
  if ((int64_t)B * Hkv > 65535) return fail(KVQ_ERR_INVALID_ARG, "B*Hkv too large");
  kvq::EncodeParams p;
  std::memset(&p, 0, sizeof p);
  p.keys = keys;
  p.codes = codes;
  p.norms = norms;
  p.write_pos = write_pos;
  p.T_new = T_new;
  p.T_cap = T_cap;
  p.t0 = t0;
  p.B = B;
  p.Hkv = Hkv;
  p.rows_whole = !write_pos && t0 == 0 && T_new == T_cap;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (cb->kind == KVQ_HADAMARD_LM) {
    if (!norms) return fail(KVQ_ERR_INVALID_ARG, "norms is NULL");
    if (!aligned16(norms)) return fail(KVQ_ERR_INVALID_ARG, "norms not 16-byte aligned");
    st = pack_signs(signs, cb->d, p.signs);
    if (st != KVQ_OK) return st;
    for (int j = 0; j < 15; ++j) p.thresholds[j] = j + 1 < (1 << cb->b) ? cb->thresholds[j] : INFINITY;
    if (!kvq::choose_encode_cells(cb->thresholds, (1 << cb->b) - 1, &p.n_cells, &p.cell_inv, &p.cell_shift))
      return fail(KVQ_ERR_UNSUPPORTED, "no cell grid separates the codebook's thresholds");
    if (T_new > 0 && (int64_t)B * Hkv * T_new >= ((int64_t)1 << 31))
      return fail(KVQ_ERR_UNSUPPORTED, "B*Hkv*T_new must stay below 2^31");
    if (T_new > 0) kvq::fast_div_magic((uint32_t)T_new, &p.tnew_magic, &p.tnew_shift);
    kvq::fast_div_magic((uint32_t)Hkv, &p.hkv_magic, &p.hkv_shift);
    if (T_new == 0) return ok();
    return from_hip(kvq::launch_hlm_encode(cb->d, cb->b, kdtype == KVQ_F16, p, s), "kvq_encode_keys");
  }
  if (cb->kind == KVQ_POT) {
    if (!norms) return fail(KVQ_ERR_INVALID_ARG, "norms (per-key scales) is NULL");
    if (!aligned16(norms)) return fail(KVQ_ERR_INVALID_ARG, "norms not 16-byte aligned");
    for (int j = 0; j < 15; ++j) p.thresholds[j] = j + 1 < (1 << (cb->b - 1)) ? cb->thresholds[j] : 0.0f;
    p.pot_mant = cb->m;
    if (T_new > 0 && (int64_t)B * Hkv * T_new >= ((int64_t)1 << 31))
      return fail(KVQ_ERR_UNSUPPORTED, "B*Hkv*T_new must stay below 2^31");
    if (T_new > 0) kvq::fast_div_magic((uint32_t)T_new, &p.tnew_magic, &p.tnew_shift);
    kvq::fast_div_magic((uint32_t)Hkv, &p.hkv_magic, &p.hkv_shift);
    if (T_new == 0) return ok();
    return from_hip(kvq::launch_pot_encode(cb->d, cb->b, kdtype == KVQ_F16, p, s), "kvq_encode_keys");
  }
  if (cb->n_heads != Hkv) return fail(KVQ_ERR_INVALID_ARG, "PQ codebook has %d heads, Hkv=%d", cb->n_heads, Hkv);
  p.pq_cent = cb->pq_centroids;
  p.pq_K = cb->K;
  if (T_new == 0) return ok();
  return from_hip(kvq::launch_pq_encode(cb->d, cb->m, cb->b, kdtype == KVQ_F16, p, s), "kvq_encode_keys");
}

kvq_status kvq_score(const kvq_codebook* cb, const int8_t* signs, const void* q, kvq_dtype qdtype,
                     const uint8_t* codes, const float* norms, int B, int Hq, int Hkv, int64_t T_cap,
                     const int32_t* seq_lens, float* scores, void* stream) {
  kvq::AttnParams p;
  ReadShape rs;
  kvq_status st = check_read(cb, signs, q, qdtype, codes, norms, B, Hq, Hkv, T_cap, &p, &rs);
  if (st != KVQ_OK) return st;
  if (!scores || !aligned16(scores)) return fail(KVQ_ERR_INVALID_ARG, "scores NULL or not 16-byte aligned");
  p.seq_lens = seq_lens;
  p.scores = scores;
  // two score workgroups fit a compute unit (registers and LDS), and the second hides the first's prologue
  // and memory latency
  choose_splits(rs.units, T_cap, 0, &p.n_splits, &p.split_len, 2);
  const dim3 grid((unsigned)p.n_splits, (unsigned)rs.units);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (cb->kind == KVQ_HADAMARD_LM) return from_hip(kvq::launch_hlm_score(cb->d, cb->b, rs.gg, p, grid, s), "kvq_score");
  if (cb->kind == KVQ_POT) return from_hip(kvq::launch_pot_score(cb->d, cb->b, rs.gg, p, grid, s), "kvq_score");
  return from_hip(kvq::launch_pq_score(cb->d, cb->m, cb->b, rs.gg, p, grid, s), "kvq_score");
}

size_t kvq_decode_attn_workspace(const kvq_codebook* cb, int B, int Hq, int Hkv, int64_t T_cap, int n_splits) {
  if (check_codebook(cb) != KVQ_OK || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || T_cap <= 0 || n_splits < 0)
    return 0;
  const int G = Hq / Hkv;
  const int gg = heads_per_wg(G);
  const int64_t units = (int64_t)B * Hkv * (G / gg);
  int splits;
  int64_t len;
  choose_splits(units, T_cap, n_splits, &splits, &len, 1, cb->kind == KVQ_PQ);
  return workspace_bytes(units, B, Hq, splits, cb->d);
}

}  // extern "C"

namespace {

// Shared body of kvq_decode_attn and kvq_decode_attn_append (new_keys == nullptr: no append).
kvq_status decode_common(const char* name, const kvq_codebook* cb, const int8_t* signs, const void* new_keys,
                         kvq_dtype kdtype, const void* q, kvq_dtype qdtype, const uint8_t* codes, const float* norms,
                         const void* v, kvq_dtype vdtype, int B, int Hq, int Hkv, int64_t T_cap,
                         const int32_t* seq_lens, float scale, void* out, kvq_dtype odtype, void* workspace,
                         size_t ws_bytes, int n_splits, void* stream) {
  kvq::AttnParams p;
  ReadShape rs;
  kvq_status st = check_read(cb, signs, q, qdtype, codes, norms, B, Hq, Hkv, T_cap, &p, &rs);
  if (st != KVQ_OK) return st;
  if (!valid_dtype(vdtype) || !valid_dtype(odtype)) return fail(KVQ_ERR_INVALID_ARG, "bad v/out dtype");
  if (!v || !out) return fail(KVQ_ERR_INVALID_ARG, "v or out is NULL");
  if (!aligned16(v) || !aligned16(out)) return fail(KVQ_ERR_INVALID_ARG, "v or out not 16-byte aligned");
  if (n_splits < 0) return fail(KVQ_ERR_INVALID_ARG, "n_splits=%d", n_splits);
  if (!std::isfinite(scale)) return fail(KVQ_ERR_INVALID_ARG, "scale is not finite");
  if (new_keys) {
    if (cb->kind == KVQ_PQ) return fail(KVQ_ERR_UNSUPPORTED, "the fused append supports the scalar codecs only");
    if (!valid_dtype(kdtype)) return fail(KVQ_ERR_INVALID_ARG, "bad key dtype %d", (int)kdtype);
    if (!aligned16(new_keys)) return fail(KVQ_ERR_INVALID_ARG, "new_keys not 16-byte aligned");
    p.new_keys = new_keys;
    p.new_f16 = kdtype == KVQ_F16;
    p.app_codes = const_cast<uint8_t*>(codes);
    p.app_norms = const_cast<float*>(norms);
    if (cb->kind == KVQ_POT) {  // midpoints of the 2^(b-1) magnitudes
      for (int j = 0; j < 15; ++j) p.thresholds[j] = j + 1 < (1 << (cb->b - 1)) ? cb->thresholds[j] : 0.0f;
      p.pot_mant = cb->m;
    } else {
      for (int j = 0; j < 15; ++j) p.thresholds[j] = j + 1 < (1 << cb->b) ? cb->thresholds[j] : INFINITY;
    }
  }
  p.seq_lens = seq_lens;
  p.v = v;
  p.out = out;
  p.out_f16 = odtype == KVQ_F16;
  p.zscale = scale * 1.4426950408889634f;
  choose_splits(rs.units, T_cap, n_splits, &p.n_splits, &p.split_len, 1, cb->kind == KVQ_PQ);
  if (p.n_splits > 1) {
    const size_t need = workspace_bytes(rs.units, B, Hq, p.n_splits, cb->d);
    if (!workspace || ws_bytes < need)
      return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
    if (!aligned16(workspace)) return fail(KVQ_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    const size_t counter_bytes = ((size_t)rs.units * 4 + 255) / 256 * 256;
    p.counters = reinterpret_cast<unsigned*>(workspace);
    p.ws = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + counter_bytes);
  }
  // Workgroups of 12 waves (three per SIMD) pay off only when every wave has several chunks to stream: d = 64,
  // fp16 V, a scalar codec and splits of at least 4096 tokens; otherwise 8 waves.
  p.waves = (cb->kind != KVQ_PQ && cb->d == 64 && vdtype == KVQ_F16 && p.split_len >= 4096) ? 12 : 8;
  const dim3 grid((unsigned)p.n_splits, (unsigned)rs.units);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = cb->kind == KVQ_HADAMARD_LM ? kvq::launch_hlm_decode(cb->d, cb->b, rs.gg, vdtype == KVQ_F16, p, grid, s)
                 : cb->kind == KVQ_POT      ? kvq::launch_pot_decode(cb->d, cb->b, rs.gg, vdtype == KVQ_F16, p, grid, s)
                                            : kvq::launch_pq_decode(cb->d, cb->m, cb->b, rs.gg, vdtype == KVQ_F16, p, grid, s);
  return from_hip(e, name);
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attn(const kvq_codebook* cb, const int8_t* signs, const void* q, kvq_dtype qdtype,
                           const uint8_t* codes, const float* norms, const void* v, kvq_dtype vdtype,
                           int B, int Hq, int Hkv, int64_t T_cap, const int32_t* seq_lens, float scale,
                           void* out, kvq_dtype odtype, void* workspace, size_t ws_bytes, int n_splits,
                           void* stream) {
  return decode_common("kvq_decode_attn", cb, signs, nullptr, KVQ_F32, q, qdtype, codes, norms, v, vdtype, B, Hq,
                       Hkv, T_cap, seq_lens, scale, out, odtype, workspace, ws_bytes, n_splits, stream);
}

kvq_status kvq_decode_attn_append(const kvq_codebook* cb, const int8_t* signs, const void* new_keys,
                                  kvq_dtype kdtype, const void* q, kvq_dtype qdtype, uint8_t* codes, float* norms,
                                  const void* v, kvq_dtype vdtype, int B, int Hq, int Hkv, int64_t T_cap,
                                  const int32_t* seq_lens, float scale, void* out, kvq_dtype odtype,
                                  void* workspace, size_t ws_bytes, int n_splits, void* stream) {
  if (!new_keys) return fail(KVQ_ERR_INVALID_ARG, "new_keys is NULL");
  return decode_common("kvq_decode_attn_append", cb, signs, new_keys, kdtype, q, qdtype, codes, norms, v, vdtype, B,
                       Hq, Hkv, T_cap, seq_lens, scale, out, odtype, workspace, ws_bytes, n_splits, stream);
}

kvq_status kvq_decode_attn_qv(const kvq_codebook* cb, const int8_t* signs, const void* q, kvq_dtype qdtype,
                              const uint8_t* codes, const float* norms, const uint8_t* vcodes, const float* vnorms,
                              int B, int Hq, int Hkv, int64_t T_cap, const int32_t* seq_lens, float scale, void* out,
                              kvq_dtype odtype, void* workspace, size_t ws_bytes, int n_splits, void* stream) {
  kvq::AttnParams p;
  ReadShape rs;
  kvq_status st = check_read(cb, signs, q, qdtype, codes, norms, B, Hq, Hkv, T_cap, &p, &rs);
  if (st != KVQ_OK) return st;
  if (cb->kind != KVQ_HADAMARD_LM)
    return fail(KVQ_ERR_UNSUPPORTED, "quantized values use the Hadamard/Lloyd-Max codec only");
  if (!vcodes || !vnorms || !out) return fail(KVQ_ERR_INVALID_ARG, "vcodes, vnorms or out is NULL");
  if (!aligned16(vcodes) || !aligned16(vnorms) || !aligned16(out))
    return fail(KVQ_ERR_INVALID_ARG, "vcodes, vnorms or out not 16-byte aligned");
  if (!valid_dtype(odtype)) return fail(KVQ_ERR_INVALID_ARG, "bad out dtype %d", (int)odtype);
  if (n_splits < 0) return fail(KVQ_ERR_INVALID_ARG, "n_splits=%d", n_splits);
  if (!std::isfinite(scale)) return fail(KVQ_ERR_INVALID_ARG, "scale is not finite");
  p.vcodes = vcodes;
  p.vnorms = vnorms;
  p.seq_lens = seq_lens;
  p.out = out;
  p.out_f16 = odtype == KVQ_F16;
  p.zscale = scale * 1.4426950408889634f;
  choose_splits(rs.units, T_cap, n_splits, &p.n_splits, &p.split_len);
  if (p.n_splits > 1) {
    const size_t need = workspace_bytes(rs.units, B, Hq, p.n_splits, cb->d);
    if (!workspace || ws_bytes < need)
      return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
    if (!aligned16(workspace)) return fail(KVQ_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    const size_t counter_bytes = ((size_t)rs.units * 4 + 255) / 256 * 256;
    p.counters = reinterpret_cast<unsigned*>(workspace);
    p.ws = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + counter_bytes);
  }
  const dim3 grid((unsigned)p.n_splits, (unsigned)rs.units);
  return from_hip(kvq::launch_hlm_decode_qv(cb->d, cb->b, rs.gg, p, grid, reinterpret_cast<hipStream_t>(stream)),
                  "kvq_decode_attn_qv");
}

}  // extern "C"

namespace {

size_t pad256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of kvq_select_signs: exact output, decode output, candidate errors, codes, norms, and the
// decode's own workspace, each 256-byte aligned.
struct SelectLayout {
  size_t exact, dec, err, codes, norms, dws, total, dws_bytes;
};

bool select_layout(const kvq_codebook* cb, int n, int Hq, int Hkv, int64_t T, int C, SelectLayout* L) {
  if (check_codebook(cb) != KVQ_OK || cb->kind != KVQ_HADAMARD_LM || n <= 0 || Hq <= 0 || Hkv <= 0 ||
      Hq % Hkv != 0 || T <= 0 || C <= 0)
    return false;
  const size_t outb = (size_t)n * Hq * cb->d * 4;
  const size_t nkeys = (size_t)n * Hkv * T;
  L->exact = 0;
  L->dec = L->exact + pad256(outb);
  L->err = L->dec + pad256(outb);
  L->codes = L->err + pad256((size_t)C * 4);
  L->norms = L->codes + pad256(nkeys * (size_t)(cb->d * cb->b / 8));
  L->dws = L->norms + pad256(nkeys * 4);
  L->dws_bytes = kvq_decode_attn_workspace(cb, n, Hq, Hkv, T, 0);
  L->total = L->dws + pad256(L->dws_bytes);
  return true;
}

}  // namespace

extern "C" {

size_t kvq_select_signs_workspace(const kvq_codebook* cb, int n_cal, int Hq, int Hkv, int64_t T, int C) {
  SelectLayout L;
  return select_layout(cb, n_cal, Hq, Hkv, T, C, &L) ? L.total : 0;
}

kvq_status kvq_select_signs(const kvq_codebook* cb, const int8_t* candidates, int C, const void* q,
                            kvq_dtype qdtype, const void* keys, kvq_dtype kdtype, const void* v, kvq_dtype vdtype,
                            int n_cal, int Hq, int Hkv, int64_t T, float scale, float* errors, int* best,
                            void* workspace, size_t ws_bytes, void* stream) {
  kvq_status st = check_codebook(cb);
  if (st != KVQ_OK) return st;
  if (cb->kind != KVQ_HADAMARD_LM) return fail(KVQ_ERR_UNSUPPORTED, "sign patterns belong to the Hadamard codec");
  if (!candidates || C <= 0) return fail(KVQ_ERR_INVALID_ARG, "need at least one candidate pattern");
  if (!errors || !best) return fail(KVQ_ERR_INVALID_ARG, "errors or best is NULL");
  if (n_cal <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(KVQ_ERR_INVALID_ARG, "n_cal=%d Hq=%d Hkv=%d", n_cal, Hq, Hkv);
  if (T <= 0 || T > kvq::kCalibMaxT)
    return fail(KVQ_ERR_UNSUPPORTED, "T=%lld: calibration samples hold 1..%d keys", (long long)T, kvq::kCalibMaxT);
  if (!valid_dtype(qdtype) || !valid_dtype(kdtype) || !valid_dtype(vdtype))
    return fail(KVQ_ERR_INVALID_ARG, "bad dtype");
  if (!q || !keys || !v) return fail(KVQ_ERR_INVALID_ARG, "q, keys or v is NULL");
  if (!aligned16(q) || !aligned16(keys) || !aligned16(v))
    return fail(KVQ_ERR_INVALID_ARG, "q, keys or v not 16-byte aligned");
  if (!std::isfinite(scale)) return fail(KVQ_ERR_INVALID_ARG, "scale is not finite");
  uint32_t packed[8];
  for (int c = 0; c < C; ++c) {
    st = pack_signs(candidates + (size_t)c * cb->d, cb->d, packed);
    if (st != KVQ_OK) {
      const std::string why = g_last_error;
      return fail(KVQ_ERR_INVALID_ARG, "candidate %d: %s", c, why.c_str());
    }
  }
  SelectLayout L;
  select_layout(cb, n_cal, Hq, Hkv, T, C, &L);
  if (!workspace || ws_bytes < L.total)
    return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, L.total);
  if (((uintptr_t)workspace & 255) != 0) return fail(KVQ_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  char* ws = reinterpret_cast<char*>(workspace);
  float* exact = reinterpret_cast<float*>(ws + L.exact);
  float* dec = reinterpret_cast<float*>(ws + L.dec);
  float* err_dev = reinterpret_cast<float*>(ws + L.err);
  uint8_t* codes = reinterpret_cast<uint8_t*>(ws + L.codes);
  float* norms = reinterpret_cast<float*>(ws + L.norms);
  void* dws = L.dws_bytes ? ws + L.dws : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the decode's arrival counters must start at zero (a fill kernel, not a memset)
  if (L.dws_bytes) {
    st = from_hip(kvq::launch_zero_words(reinterpret_cast<uint32_t*>(dws), L.dws_bytes / 4, s), "kvq_select_signs");
    if (st != KVQ_OK) return st;
  }

  kvq::CalibParams cp;
  cp.q = q;
  cp.keys = keys;
  cp.v = v;
  cp.out = exact;
  cp.n = n_cal;
  cp.Hq = Hq;
  cp.Hkv = Hkv;
  cp.T = (int)T;
  cp.q_f16 = qdtype == KVQ_F16;
  cp.k_f16 = kdtype == KVQ_F16;
  cp.v_f16 = vdtype == KVQ_F16;
  cp.scale = scale;
  st = from_hip(kvq::launch_exact_attn(cb->d, cp, s), "kvq_select_signs");
  if (st != KVQ_OK) return st;
  const int64_t nout = (int64_t)n_cal * Hq * cb->d;
  for (int c = 0; c < C; ++c) {
    const int8_t* sg = candidates + (size_t)c * cb->d;
    st = kvq_encode_keys(cb, sg, keys, kdtype, n_cal, Hkv, T, codes, norms, T, 0, nullptr, stream);
    if (st != KVQ_OK) return st;
    st = kvq_decode_attn(cb, sg, q, qdtype, codes, norms, v, vdtype, n_cal, Hq, Hkv, T, nullptr, scale, dec, KVQ_F32,
                         dws, L.dws_bytes, 0, stream);
    if (st != KVQ_OK) return st;
    st = from_hip(kvq::launch_rel_err(dec, exact, nout, err_dev, c, s), "kvq_select_signs");
    if (st != KVQ_OK) return st;
  }
  if (hipMemcpyAsync(errors, err_dev, (size_t)C * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(KVQ_ERR_DEVICE, "kvq_select_signs: reading the errors back failed");
  int b = 0;
  for (int c = 1; c < C; ++c)
    if (errors[c] < errors[b]) b = c;
  *best = b;
  return ok();
}

}  // extern "C"
