// Host-side checks of libkvq's C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built by tests/test_sanitize.py with the host compiler from the library's own api.cpp and codebook.cpp
// and this file, which stands in for everything that would reach a GPU: the kernel launchers record what
// they were asked to launch (and check it against the launch's documented invariants) instead of launching,
// and the few HIP runtime calls of the host code are stubs (no device: hipGetDevice fails, so the library's
// compute-unit count falls back to 256).  Device pointers are plain host buffers, never dereferenced by the
// host code.  Every entry point is driven through valid calls and through each of its argument checks; the
// program prints one line per failed expectation and exits nonzero if there was any, and the sanitizers
// abort it on the first memory or undefined-behaviour error.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

static int g_fail = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::printf("FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, kvq_last_error()); \
      ++g_fail;                                                                   \
    }                                                                             \
  } while (0)

// ---------------------------------------------------------------- stand-ins for the GPU side
static int g_launches = 0;
static kvq::AttnParams g_attn;
static dim3 g_grid;
static kvq::EncodeParams g_enc;

static hipError_t record_attn(const kvq::AttnParams& p, dim3 grid, bool merge = true) {
  ++g_launches;
  g_attn = p;
  g_grid = grid;
  // the read kernels' launch invariants: whole 64-token chunks per split, splits covering T_cap, at most
  // 256 splits (the merge keeps per-split scalars in LDS), one grid column per split
  if (p.split_len <= 0 || p.split_len % 64 != 0) return hipErrorInvalidValue;
  if (p.n_splits < 1 || p.n_splits > 256 || (int64_t)p.n_splits * p.split_len < p.T_cap) return hipErrorInvalidValue;
  if ((int64_t)(p.n_splits - 1) * p.split_len >= p.T_cap) return hipErrorInvalidValue;
  if ((int)grid.x != p.n_splits || grid.y == 0) return hipErrorInvalidValue;
  if (merge && p.n_splits > 1 && (!p.ws || !p.counters)) return hipErrorInvalidValue;  // decode: split merge
  if (!merge && !p.scores) return hipErrorInvalidValue;                               // score: the output
  return hipSuccess;
}

namespace kvq {
hipError_t launch_hlm_decode(int, int, int, bool, const AttnParams& p, dim3 g, hipStream_t) { return record_attn(p, g); }
hipError_t launch_hlm_score(int, int, int, const AttnParams& p, dim3 g, hipStream_t) { return record_attn(p, g, false); }
hipError_t launch_hlm_decode_qv(int, int, int, const AttnParams& p, dim3 g, hipStream_t) { return record_attn(p, g); }
hipError_t launch_pq_decode(int, int, int, int, bool, const AttnParams& p, dim3 g, hipStream_t) {
  return record_attn(p, g);
}
hipError_t launch_pq_score(int, int, int, int, const AttnParams& p, dim3 g, hipStream_t) {
  return record_attn(p, g, false);
}
hipError_t launch_pot_decode(int, int, int, bool, const AttnParams& p, dim3 g, hipStream_t) { return record_attn(p, g); }
hipError_t launch_pot_score(int, int, int, const AttnParams& p, dim3 g, hipStream_t) { return record_attn(p, g, false); }
static hipError_t record_enc(const EncodeParams& p) {
  ++g_launches;
  g_enc = p;
  return (p.T_new > 0 && p.B > 0 && p.Hkv > 0) ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_hlm_encode(int, int, bool, const EncodeParams& p, hipStream_t) { return record_enc(p); }
hipError_t launch_pot_encode(int, int, bool, const EncodeParams& p, hipStream_t) { return record_enc(p); }
hipError_t launch_pq_encode(int, int, int, bool, const EncodeParams& p, hipStream_t) { return record_enc(p); }
hipError_t launch_exact_attn(int, const CalibParams&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_rel_err(const float*, const float*, int64_t n, float* errors, int c, hipStream_t) {
  ++g_launches;
  errors[c] = 1.0f / (float)(1 + (c * 7919) % 13) + (float)(n > 0 ? 0 : 1);  // a recognisable ranking
  return hipSuccess;
}
hipError_t launch_zero_words(uint32_t* p, size_t n_words, hipStream_t) {
  std::memset(p, 0, n_words * 4);
  return hipSuccess;
}
}  // namespace kvq

extern "C" {
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

// ---------------------------------------------------------------- helpers
template <class T>
static T* buf(std::vector<unsigned char>& store, size_t n) {  // 256-byte aligned storage of n Ts
  store.assign(n * sizeof(T) + 256, 0);
  const uintptr_t p = (reinterpret_cast<uintptr_t>(store.data()) + 255) & ~(uintptr_t)255;
  return reinterpret_cast<T*>(p);
}
template <class T>
static T* misalign(T* p) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + 4);
}

static void check_codebooks() {
  for (int d : {16, 32, 64, 128, 256})
    for (int b = 1; b <= 4; ++b) {
      kvq_codebook cb;
      EXPECT(kvq_build_codebook(d, b, &cb) == KVQ_OK);
      EXPECT(cb.kind == KVQ_HADAMARD_LM && cb.d == d && cb.b == b);
      for (int j = 0; j + 1 < (1 << b); ++j) {
        EXPECT(cb.levels[j] < cb.levels[j + 1]);
        EXPECT(cb.levels[j] < cb.thresholds[j] && cb.thresholds[j] < cb.levels[j + 1]);
        EXPECT(cb.levels[j] == -cb.levels[(1 << b) - 1 - j]);  // symmetric codebook
      }
    }
  kvq_codebook cb;
  for (int d : {0, 8, 24, 48, 512}) EXPECT(kvq_build_codebook(d, 4, &cb) != KVQ_OK);
  for (int b : {0, 5, -1}) EXPECT(kvq_build_codebook(64, b, &cb) != KVQ_OK);
  EXPECT(kvq_build_codebook(64, 4, nullptr) != KVQ_OK);
  EXPECT(std::strlen(kvq_last_error()) > 0);

  for (int b = 2; b <= 4; ++b)
    for (int mant = 0; mant <= 1; ++mant) {
      const kvq_status s = kvq_build_codebook_pot(64, b, mant, &cb);
      if (mant && b < 3) continue;  // the mantissa term needs room for two midpoint families
      EXPECT(s == KVQ_OK);
    }
  EXPECT(kvq_build_codebook_pot(64, 1, 0, &cb) != KVQ_OK);
  EXPECT(kvq_build_codebook_pot(64, 4, 2, &cb) != KVQ_OK);

  // product quantization: host k-means, then the device-centroid codebook
  const int H = 2, n = 300, d = 32, m = 4, K = 16, iters = 4;
  std::vector<float> train((size_t)H * n * d);
  for (size_t i = 0; i < train.size(); ++i) train[i] = std::sin(0.37 * (double)i) + 0.1f * (float)(i % 7);
  std::vector<int64_t> start((size_t)H * m * K);
  for (size_t i = 0; i < start.size(); ++i) start[i] = (int64_t)((i * 37) % n);
  std::vector<float> cent((size_t)H * m * K * (d / m));
  EXPECT(kvq_build_codebook_pq(train.data(), H, n, d, m, K, iters, start.data(), cent.data()) == KVQ_OK);
  for (float c : cent) EXPECT(std::isfinite(c));
  EXPECT(kvq_build_codebook_pq(train.data(), H, n, d, 5, K, iters, start.data(), cent.data()) != KVQ_OK);
  EXPECT(kvq_build_codebook_pq(train.data(), H, n, d, m, 300, iters, start.data(), cent.data()) != KVQ_OK);
  EXPECT(kvq_build_codebook_pq(nullptr, H, n, d, m, K, iters, start.data(), cent.data()) != KVQ_OK);
  std::vector<int64_t> bad = start;
  bad[3] = n;  // a start row past the training set
  EXPECT(kvq_build_codebook_pq(train.data(), H, n, d, m, K, iters, bad.data(), cent.data()) != KVQ_OK);
  EXPECT(kvq_codebook_pq(d, m, K, H, cent.data(), &cb) == KVQ_OK);
  EXPECT(cb.kind == KVQ_PQ && cb.b == 4);  // K <= 16 with m even: 4-bit codes
  EXPECT(kvq_codebook_pq(d, m, 256, H, cent.data(), &cb) == KVQ_OK && cb.b == 8);
  EXPECT(kvq_codebook_pq(d, 3, K, H, cent.data(), &cb) != KVQ_OK);
  EXPECT(kvq_codebook_pq(d, m, K, H, nullptr, &cb) != KVQ_OK);
}

static void check_encode() {
  kvq_codebook cb;
  EXPECT(kvq_build_codebook(64, 4, &cb) == KVQ_OK);
  const int B = 2, Hkv = 2;
  const int64_t T = 100;
  std::vector<unsigned char> sk, sc, sn, ss, sw;
  uint16_t* keys = buf<uint16_t>(sk, (size_t)B * Hkv * T * 64);
  uint8_t* codes = buf<uint8_t>(sc, (size_t)B * Hkv * T * 32);
  float* norms = buf<float>(sn, (size_t)B * Hkv * T);
  int8_t* signs = buf<int8_t>(ss, 64);
  for (int i = 0; i < 64; ++i) signs[i] = (i % 3) ? 1 : -1;
  int32_t* wpos = buf<int32_t>(sw, B);
  wpos[0] = 5;
  wpos[1] = 90;

  g_launches = 0;
  EXPECT(kvq_encode_keys(&cb, signs, keys, KVQ_F16, B, Hkv, T, codes, norms, T, 0, nullptr, nullptr) == KVQ_OK);
  EXPECT(g_launches == 1 && g_enc.rows_whole == 1 && g_enc.T_new == T);
  EXPECT(kvq_encode_keys(&cb, signs, keys, KVQ_F16, B, Hkv, 7, codes, norms, T, 3, nullptr, nullptr) == KVQ_OK);
  EXPECT(g_enc.rows_whole == 0 && g_enc.t0 == 3);
  EXPECT(kvq_encode_keys(&cb, signs, keys, KVQ_F16, B, Hkv, 7, codes, norms, T, 0, wpos, nullptr) == KVQ_OK);
  EXPECT(g_enc.write_pos == wpos);
  const int before = g_launches;
  EXPECT(kvq_encode_keys(nullptr, signs, keys, KVQ_F16, B, Hkv, T, codes, norms, T, 0, nullptr, nullptr) != KVQ_OK);
  EXPECT(kvq_encode_keys(&cb, nullptr, keys, KVQ_F16, B, Hkv, T, codes, norms, T, 0, nullptr, nullptr) != KVQ_OK);
  EXPECT(kvq_encode_keys(&cb, signs, nullptr, KVQ_F16, B, Hkv, T, codes, norms, T, 0, nullptr, nullptr) != KVQ_OK);
  EXPECT(kvq_encode_keys(&cb, signs, keys, (kvq_dtype)7, B, Hkv, T, codes, norms, T, 0, nullptr, nullptr) != KVQ_OK);
  EXPECT(kvq_encode_keys(&cb, signs, misalign(keys), KVQ_F16, B, Hkv, T, codes, norms, T, 0, nullptr, nullptr) !=
         KVQ_OK);
  EXPECT(kvq_encode_keys(&cb, signs, keys, KVQ_F16, -1, Hkv, T, codes, norms, T, 0, nullptr, nullptr) != KVQ_OK);
  EXPECT(kvq_encode_keys(&cb, signs, keys, KVQ_F16, B, Hkv, T + 1, codes, norms, T, 0, nullptr, nullptr) != KVQ_OK);
  EXPECT(kvq_encode_keys(&cb, signs, keys, KVQ_F16, B, Hkv, 10, codes, norms, T, T - 5, nullptr, nullptr) != KVQ_OK);
  kvq_codebook broken = cb;
  broken.b = 9;
  EXPECT(kvq_encode_keys(&broken, signs, keys, KVQ_F16, B, Hkv, T, codes, norms, T, 0, nullptr, nullptr) != KVQ_OK);
  int8_t bad_signs[64];
  std::memcpy(bad_signs, signs, 64);
  bad_signs[17] = 0;  // a sign that is neither +1 nor -1
  EXPECT(kvq_encode_keys(&cb, bad_signs, keys, KVQ_F16, B, Hkv, T, codes, norms, T, 0, nullptr, nullptr) != KVQ_OK);
  EXPECT(g_launches == before);  // no failed call reached a launcher
}

static void check_read_paths() {
  kvq_codebook cb;
  EXPECT(kvq_build_codebook(64, 4, &cb) == KVQ_OK);
  const int B = 2, Hq = 8, Hkv = 2;
  std::vector<unsigned char> sq, sc, sn, sv, so, sw, ss, sl, sk, svc, svn, ssc;
  int8_t* signs = buf<int8_t>(ss, 64);
  for (int i = 0; i < 64; ++i) signs[i] = (i % 5) ? 1 : -1;
  for (int64_t T : {1, 63, 64, 1000, 8192, 40000}) {
    uint16_t* q = buf<uint16_t>(sq, (size_t)B * Hq * 64);
    uint8_t* codes = buf<uint8_t>(sc, (size_t)B * Hkv * T * 32);
    float* norms = buf<float>(sn, (size_t)B * Hkv * T);
    uint16_t* v = buf<uint16_t>(sv, (size_t)B * Hkv * T * 64);
    float* out = buf<float>(so, (size_t)B * Hq * 64);
    int32_t* lens = buf<int32_t>(sl, B);
    lens[0] = (int32_t)T;
    lens[1] = (int32_t)(T / 2);
    uint16_t* nk = buf<uint16_t>(sk, (size_t)B * Hkv * 64);
    uint8_t* vcodes = buf<uint8_t>(svc, (size_t)B * Hkv * T * 32);
    float* vnorms = buf<float>(svn, (size_t)B * Hkv * T);
    float* scores = buf<float>(ssc, (size_t)B * Hq * T);

    g_launches = 0;
    EXPECT(kvq_score(&cb, signs, q, KVQ_F16, codes, norms, B, Hq, Hkv, T, lens, scores, nullptr) == KVQ_OK);
    EXPECT(g_launches == 1);
    for (int req : {0, 1, 3, 7, 256, 1000}) {
      const size_t need = kvq_decode_attn_workspace(&cb, B, Hq, Hkv, T, req);
      float* ws = buf<float>(sw, need / 4 + 64);
      EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, v, KVQ_F16, B, Hq, Hkv, T, lens, 0.125f, out,
                             KVQ_F32, ws, need, req, nullptr) == KVQ_OK);
      EXPECT(req == 0 || g_attn.n_splits <= req);
      EXPECT((need == 0) == (g_attn.n_splits == 1));
      EXPECT(kvq_decode_attn_append(&cb, signs, nk, KVQ_F16, q, KVQ_F16, codes, norms, v, KVQ_F16, B, Hq, Hkv, T,
                                    lens, 0.125f, out, KVQ_F16, ws, need, req, nullptr) == KVQ_OK);
      EXPECT(g_attn.new_keys == nk && g_attn.app_codes == codes);
      EXPECT(kvq_decode_attn_qv(&cb, signs, q, KVQ_F16, codes, norms, vcodes, vnorms, B, Hq, Hkv, T, lens, 0.125f,
                                out, KVQ_F32, ws, need, req, nullptr) == KVQ_OK);
      if (need > 0) {  // a workspace one byte short, or absent
        EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, v, KVQ_F16, B, Hq, Hkv, T, lens, 0.125f, out,
                               KVQ_F32, ws, need - 1, req, nullptr) == KVQ_ERR_WORKSPACE);
        EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, v, KVQ_F16, B, Hq, Hkv, T, lens, 0.125f, out,
                               KVQ_F32, nullptr, 0, req, nullptr) == KVQ_ERR_WORKSPACE);
      }
    }
    // argument checks
    const int before = g_launches;
    size_t need = kvq_decode_attn_workspace(&cb, B, Hq, Hkv, T, 0);
    float* ws = buf<float>(sw, need / 4 + 64);
    EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, v, KVQ_F16, B, 7, Hkv, T, lens, 0.125f, out, KVQ_F32,
                           ws, need, 0, nullptr) != KVQ_OK);
    EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, v, KVQ_F16, B, Hq, Hkv, T, lens, NAN, out, KVQ_F32,
                           ws, need, 0, nullptr) != KVQ_OK);
    EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, v, KVQ_F16, B, Hq, Hkv, T, lens, 0.125f, out, KVQ_F32,
                           ws, need, -2, nullptr) != KVQ_OK);
    EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, nullptr, KVQ_F16, B, Hq, Hkv, T, lens, 0.125f, out,
                           KVQ_F32, ws, need, 0, nullptr) != KVQ_OK);
    EXPECT(kvq_decode_attn(&cb, signs, misalign(q), KVQ_F16, codes, norms, v, KVQ_F16, B, Hq, Hkv, T, lens, 0.125f,
                           out, KVQ_F32, ws, need, 0, nullptr) != KVQ_OK);
    EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, v, (kvq_dtype)3, B, Hq, Hkv, T, lens, 0.125f, out,
                           KVQ_F32, ws, need, 0, nullptr) != KVQ_OK);
    EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, v, KVQ_F16, 0, Hq, Hkv, T, lens, 0.125f, out, KVQ_F32,
                           ws, need, 0, nullptr) != KVQ_OK);
    EXPECT(kvq_decode_attn(&cb, signs, q, KVQ_F16, codes, norms, v, KVQ_F16, B, Hq, Hkv, 0, lens, 0.125f, out, KVQ_F32,
                           ws, need, 0, nullptr) != KVQ_OK);
    EXPECT(kvq_score(&cb, signs, q, KVQ_F16, codes, norms, B, Hq, Hkv, T, lens, misalign(scores), nullptr) != KVQ_OK);
    EXPECT(kvq_score(&cb, nullptr, q, KVQ_F16, codes, norms, B, Hq, Hkv, T, lens, scores, nullptr) != KVQ_OK);
    EXPECT(g_launches == before);
  }
  EXPECT(kvq_decode_attn_workspace(nullptr, 1, 8, 2, 100, 0) == 0);
  EXPECT(kvq_decode_attn_workspace(&cb, 1, 8, 3, 100, 0) == 0);  // Hq % Hkv != 0

  // power-of-two and PQ read paths (no signs)
  kvq_codebook pcb;
  EXPECT(kvq_build_codebook_pot(64, 4, 1, &pcb) == KVQ_OK);
  const int64_t T = 777;
  std::vector<unsigned char> a, c2, n2, v2, o2;
  uint16_t* q = buf<uint16_t>(a, (size_t)B * Hq * 64);
  uint8_t* codes = buf<uint8_t>(c2, (size_t)B * Hkv * T * 32);
  float* norms = buf<float>(n2, (size_t)B * Hkv * T);
  uint16_t* v = buf<uint16_t>(v2, (size_t)B * Hkv * T * 64);
  float* out = buf<float>(o2, (size_t)B * Hq * 64);
  size_t need = kvq_decode_attn_workspace(&pcb, B, Hq, Hkv, T, 0);
  std::vector<unsigned char> w2;
  float* ws = buf<float>(w2, need / 4 + 64);
  EXPECT(kvq_decode_attn(&pcb, nullptr, q, KVQ_F16, codes, norms, v, KVQ_F16, B, Hq, Hkv, T, nullptr, 0.125f, out,
                         KVQ_F32, ws, need, 0, nullptr) == KVQ_OK);
  std::vector<float> cent((size_t)Hkv * 8 * 256 * 8, 0.5f);
  kvq_codebook qcb;
  EXPECT(kvq_codebook_pq(64, 8, 256, Hkv, cent.data(), &qcb) == KVQ_OK);
  need = kvq_decode_attn_workspace(&qcb, B, Hq, Hkv, T, 0);
  ws = buf<float>(w2, need / 4 + 64);
  EXPECT(kvq_decode_attn(&qcb, nullptr, q, KVQ_F16, codes, nullptr, v, KVQ_F16, B, Hq, Hkv, T, nullptr, 0.125f, out,
                         KVQ_F32, ws, need, 0, nullptr) == KVQ_OK);
  EXPECT(kvq_decode_attn_append(&qcb, nullptr, q, KVQ_F16, q, KVQ_F16, codes, nullptr, v, KVQ_F16, B, Hq, Hkv, T,
                                nullptr, 0.125f, out, KVQ_F32, ws, need, 0, nullptr) == KVQ_ERR_UNSUPPORTED);
}

static void check_select_signs() {
  kvq_codebook cb;
  EXPECT(kvq_build_codebook(64, 2, &cb) == KVQ_OK);
  const int n = 2, Hq = 4, Hkv = 2, C = 5;
  const int64_t T = 200;
  std::vector<unsigned char> sc, sq, sk, sv, sw, se;
  int8_t* cands = buf<int8_t>(sc, (size_t)C * 64);
  for (int i = 0; i < C * 64; ++i) cands[i] = ((i * 31) % 7 < 3) ? -1 : 1;
  uint16_t* q = buf<uint16_t>(sq, (size_t)n * Hq * 64);
  uint16_t* keys = buf<uint16_t>(sk, (size_t)n * Hkv * T * 64);
  uint16_t* v = buf<uint16_t>(sv, (size_t)n * Hkv * T * 64);
  const size_t need = kvq_select_signs_workspace(&cb, n, Hq, Hkv, T, C);
  EXPECT(need > 0);
  void* ws = buf<unsigned char>(sw, need);
  float* errors = buf<float>(se, C);
  int best = -1;
  EXPECT(kvq_select_signs(&cb, cands, C, q, KVQ_F16, keys, KVQ_F16, v, KVQ_F16, n, Hq, Hkv, T, 0.125f, errors, &best,
                          ws, need, nullptr) == KVQ_OK);
  EXPECT(best >= 0 && best < C);
  for (int c = 0; c < C; ++c) EXPECT(errors[best] <= errors[c]);
  EXPECT(kvq_select_signs(&cb, cands, C, q, KVQ_F16, keys, KVQ_F16, v, KVQ_F16, n, Hq, Hkv, T, 0.125f, errors, &best,
                          ws, need - 1, nullptr) == KVQ_ERR_WORKSPACE);
  EXPECT(kvq_select_signs(&cb, cands, 0, q, KVQ_F16, keys, KVQ_F16, v, KVQ_F16, n, Hq, Hkv, T, 0.125f, errors, &best,
                          ws, need, nullptr) != KVQ_OK);
  EXPECT(kvq_select_signs(&cb, cands, C, q, KVQ_F16, keys, KVQ_F16, v, KVQ_F16, n, Hq, Hkv, kvq::kCalibMaxT + 1,
                          0.125f, errors, &best, ws, need, nullptr) != KVQ_OK);
}

// The encode kernel's cell search, replayed on the CPU with the same fp32 operations (fmaf rounds once, as
// the GPU's fused multiply-add does): the cell table the kernel builds from the host's grid, then for y the
// cell offset from the bits of fmaf(y, cell_inv, cell_shift + 2^20) masked to a multiple of 8, and the
// count (thresholds below the cell) + (y >= the threshold inside it).  It must equal the plain count of
// thresholds <= y for every y in [-1, 1]: checked at and around every threshold and every cell edge (the
// neighbouring floats included) and on a fine sweep.
static void check_cell_search() {
  for (int d : {16, 32, 64, 128, 256})
    for (int b = 1; b <= 4; ++b) {
      kvq_codebook cb;
      EXPECT(kvq_build_codebook(d, b, &cb) == KVQ_OK);
      const int nt = (1 << b) - 1;
      int n_cells = 0;
      float inv = 0.0f, shift = 0.0f;
      EXPECT(kvq::choose_encode_cells(cb.thresholds, nt, &n_cells, &inv, &shift));
      if (n_cells <= 0) continue;
      std::vector<float> inside(n_cells, INFINITY);
      std::vector<uint32_t> below(n_cells, 0);
      for (int c = 0; c < n_cells; ++c)
        for (int j = 0; j < nt; ++j) {
          const int cj = (int)std::floor(std::fmaf(cb.thresholds[j], inv, shift));
          below[c] += cj < c ? 1u : 0u;
          if (cj == c) inside[c] = cb.thresholds[j];
        }
      const float shift20 = shift + 0x1p20f;
      EXPECT(shift20 - 0x1p20f == shift);  // exact
      auto kernel_code = [&](float y) -> uint32_t {
        uint32_t bits;
        const float v = std::fmaf(y, inv, shift20);
        std::memcpy(&bits, &v, 4);
        const uint32_t c = (bits & 0x7ffff8u) / 8;
        if (c >= (uint32_t)n_cells) return 999u;  // out of the table: a failure
        return below[c] + (y >= inside[c] ? 1u : 0u);
      };
      auto plain_code = [&](float y) -> uint32_t {
        uint32_t k = 0;
        for (int j = 0; j < nt; ++j) k += (y >= cb.thresholds[j]) ? 1u : 0u;
        return k;
      };
      int bad = 0;
      auto probe = [&](float y) {
        for (int s2 = -3; s2 <= 3; ++s2) {  // y and its three neighbouring floats either side
          float z = y;
          for (int i = 0; i < (s2 < 0 ? -s2 : s2); ++i) z = std::nextafter(z, s2 < 0 ? -2.0f : 2.0f);
          if (z < -1.0f || z > 1.0f) continue;
          if (kernel_code(z) != plain_code(z)) ++bad;
        }
      };
      for (int j = 0; j < nt; ++j) probe(cb.thresholds[j]);
      for (int c = 0; c <= n_cells; ++c) probe(((float)c - shift) / inv);  // near every cell edge
      for (int i = 0; i <= 200000; ++i) probe(-1.0f + 2.0f * (float)i / 200000.0f);
      probe(-0.0f);
      EXPECT(bad == 0);
    }
}

int main() {
  EXPECT(kvq_version() > 0);
  EXPECT(kvq_last_error() != nullptr);
  check_codebooks();
  check_cell_search();
  check_encode();
  check_read_paths();
  check_select_signs();
  std::printf("%s: %d failed expectation(s)\n", g_fail ? "FAIL" : "OK", g_fail);
  return g_fail ? 1 : 0;
}
