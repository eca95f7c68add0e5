/*
 * kvq.h -- C ABI of libkvq: attention computed directly from quantized
 * key-cache codes on AMD Instinct MI355X (gfx950).
 *
 * Method (web pages, cited by title and section):
 *   "AXELRAM: Quantize Once, Never Dequantize" -- Key Points and Abstract:
 *     keys are transformed on write (an orthogonal transform with a +-1 sign
 *     pattern, which spreads every coordinate of the rotated unit key like
 *     N(0, 1/d)) and stored as indices of a codebook fixed at design time that
 *     depends only on the head dimension d and the bit width b; on read the
 *     query is transformed once and scores come from table lookups over the
 *     stored indices, with no inverse transform.
 *   "LOOKAT: Lookup-Optimized Key-Attention" summary page -- AI Summary and
 *     Abstract: product quantization (m subspaces, a learned codebook each)
 *     with asymmetric distance computation through lookup tables.
 *   Shift-accumulate attention page (arxivdaily 2609.09208) -- English
 *     abstract: a fused decode-attention kernel with online softmax.
 *
 * Concretely, with H the normalised Sylvester Walsh-Hadamard matrix
 * (H[i][j] = (-1)^popcount(i&j) / sqrt(d)) and D = diag(signs):
 *   write:  n = ||k||,  y = H D k / n,  code_i = #{ j : t_j <= y_i }
 *           (t = thresholds of the Lloyd-Max codebook for N(0, 1/d))
 *   read:   q' = H D q,  LUT[i][j] = q'_i * c_j,
 *           s_t = n_t * sum_i LUT[i][code_{t,i}],
 *           out = sum_t softmax_t(scale * s) * v_t
 *   PQ:     LUT[s][c] = q_s . C_{s,c},  s_t = sum_s LUT[s][code_{t,s}]
 *
 * Conventions shared by every entry point
 *   - Layouts are row-major and contiguous.  B = batch, Hq = query heads,
 *     Hkv = key/value heads (Hq % Hkv == 0; query head h reads kv head
 *     h / (Hq/Hkv)), T_cap = capacity of the cache along the token axis,
 *     d = head dimension.
 *   - Codes are packed LSB-first: coordinate i of a key occupies bits
 *     [i*b, i*b + b) of the key's byte row of d*b/8 bytes, bit 0 of byte 0
 *     first (for b = 4: low nibble = even coordinate).
 *   - Every pointer marked "device" is caller-owned device memory (e.g. a
 *     PyTorch tensor); the library never allocates, frees or retains it.
 *     Pointers marked "host" are read during the call only.
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t; NULL
 *     means the default stream); outputs are valid once the caller
 *     synchronizes that stream.  Calls are reentrant; two calls that write
 *     the same buffers must be ordered by the caller.
 *   - Every function validates its arguments before launching anything and
 *     returns a kvq_status; on failure nothing is launched and
 *     kvq_last_error() describes the problem.  The library never prints,
 *     aborts or throws across this boundary.
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1, /* a size, pointer, alignment or enum is out of range */
  KVQ_ERR_UNSUPPORTED = 2, /* valid but not built (e.g. an untemplated d) */
  KVQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  KVQ_ERR_DEVICE = 4       /* a HIP call failed; the HIP error string is in kvq_last_error() */
} kvq_status;

typedef enum kvq_dtype { KVQ_F32 = 0, KVQ_F16 = 1 } kvq_dtype;

typedef enum kvq_kind {
  KVQ_HADAMARD_LM = 0, /* Walsh-Hadamard rotation + Lloyd-Max scalar codebook */
  KVQ_PQ = 1,          /* product quantization, asymmetric distance computation */
  KVQ_POT = 2          /* signed power-of-two element codes with a per-key scale */
} kvq_kind;

#define KVQ_MAX_LEVELS 16

/* A codebook.  Plain data: copy it freely.  For KVQ_HADAMARD_LM and KVQ_POT it
 * is fully described by its sizes and the arrays; for KVQ_PQ it refers to
 * caller-owned device centroids. */
typedef struct kvq_codebook {
  int32_t kind;                            /* kvq_kind */
  int32_t d;                               /* head dimension */
  int32_t b;                               /* HLM: bits per coordinate, 1..4; POT: bits per element, 2..4;
                                              PQ: bits per subspace code, 8 or 4 (K <= 16, m even: two
                                              codes per byte, the even subspace in the low nibble) */
  int32_t m;                               /* PQ: number of subspaces (d % m == 0); POT: 1 with the mantissa term */
  int32_t K;                               /* PQ: centroids per subspace, 2..256 */
  int32_t n_heads;                         /* PQ: kv heads covered by pq_centroids */
  float levels[KVQ_MAX_LEVELS];            /* HLM: ascending levels c_0..c_{2^b-1};
                                              POT: signed level of every code value */
  float thresholds[KVQ_MAX_LEVELS - 1];    /* HLM: t_j = (c_j + c_{j+1}) / 2;
                                              POT: midpoints of the descending magnitudes */
  const float* pq_centroids;               /* PQ: device [n_heads][m][K][d/m] fp32 */
} kvq_codebook;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int kvq_version(void);

/* Thread-local, NUL-terminated description of the last failure on this
 * thread ("" if none).  Valid until the next kvq_* call on the thread. */
const char* kvq_last_error(void);

/* Lloyd-Max codebook for N(0, 1/d) with 2^b levels (AXELRAM, Abstract: the
 * quantizer depends only on d and b).  Host only, deterministic: the Lloyd
 * iteration on N(0,1) in double precision, made exactly odd-symmetric, scaled
 * by 1/sqrt(d) and rounded to fp32; thresholds are the midpoints.
 *   d: power of two, 16 <= d <= 256.   b: 1..4.   out: host, written.
 * Errors: KVQ_ERR_INVALID_ARG for d, b out of range or out == NULL. */
kvq_status kvq_build_codebook(int d, int b, kvq_codebook* out);

/* Product-quantization codebooks by Lloyd k-means (LOOKAT, AI Summary:
 * codebook learning per subspace).  Host only, double precision.
 *   train:      host [H][n][d] fp32 training keys.
 *   start_rows: host [H][m][K] int64, rows of train[h] that seed the
 *               centroids of (h, s) (sub-vector s of those rows); each in [0, n).
 *   iters:      assignment/update rounds (>= 0).  Ties go to the lowest
 *               centroid index; a centroid with no members keeps its place.
 *   centroids:  host [H][m][K][d/m] fp32, written.
 * Errors: KVQ_ERR_INVALID_ARG for sizes out of range (d % m != 0, K > 256,
 *   K > n, a start row out of range) or NULL pointers. */
kvq_status kvq_build_codebook_pq(const float* train, int H, int64_t n, int d, int m, int K, int iters,
                                 const int64_t* start_rows, float* centroids);

/* Signed power-of-two element codes (shift-accumulate attention page, English
 * abstract: keys as signed power-of-two fixed-point codes, so that every
 * product in q.k is a sign flip and a shift, with an optional sub-power
 * mantissa term).  Host only, deterministic.  A key k is stored as
 * alpha = max_i |k_i| (in the norms buffer) and one b-bit field per element:
 * bit b-1 = sign (k_i < 0), bits 0..b-2 = the index j of the magnitude nearest
 * to |k_i| / alpha (ties to the larger) in the descending set
 *   mantissa == 0:  2^-j,
 *   mantissa == 1:  2^-(j/2) for even j, (3/4) 2^-((j-1)/2) for odd j.
 * The element's value is alpha * (-1)^sign * magnitude(j); levels[c] holds
 * (-1)^sign * magnitude(j) for every code value c, thresholds the midpoints.
 * No rotation and no sign pattern (signs may be NULL in every call).  The
 * kernels rely on these exact levels and midpoints: every call that takes a
 * KVQ_POT codebook returns KVQ_ERR_INVALID_ARG if a level or midpoint differs
 * from what this function writes for (d, b, mantissa).
 *   d: power of two, 16 <= d <= 256.   b: 2..4.   mantissa: 0 or 1.
 * Errors: KVQ_ERR_INVALID_ARG for d, b, mantissa out of range or out == NULL. */
kvq_status kvq_build_codebook_pot(int d, int b, int mantissa, kvq_codebook* out);

/* Fill a KVQ_PQ codebook that refers to device centroids
 * [n_heads][m][K][d/m] fp32 (caller-owned; must outlive every call using
 * the codebook).  Host only.  The code width b is set to 4 when K <= 16 and m
 * is even (LOOKAT's 32x and 64x compressions at d = 64 are m = 8 and m = 4
 * with K = 16), else 8; a caller may set b = 8 afterwards to keep one byte per
 * subspace. */
kvq_status kvq_codebook_pq(int d, int m, int K, int n_heads, const float* centroids_device, kvq_codebook* out);

/* Write path: encode keys into the code cache (AXELRAM, Abstract: transform on
 * write; for KVQ_POT the shift-accumulate page's power-of-two code).
 *   cb:        codebook (HLM, POT or PQ).
 *   signs:     host [d] int8, each +1 or -1 (HLM); ignored for POT and PQ (may be NULL).
 *   keys:      device [B][Hkv][T_new][d], dtype kdtype (may be NULL when T_new == 0).
 *   codes:     device [B][Hkv][T_cap][d*b/8] (HLM, POT) or [B][Hkv][T_cap][m*b/8] (PQ)
 *              uint8; rows pos_b .. pos_b+T_new-1 of every (b, h) are written.
 *   norms:     device [B][Hkv][T_cap] fp32, same rows written (HLM);
 *              ignored for PQ (may be NULL).
 *   t0:        write position used for every batch when write_pos is NULL.
 *   write_pos: device [B] int32 per-batch write positions, or NULL.
 *              Rows that would fall outside [0, T_cap) are skipped.
 *   For PQ the kv head index selects that head's centroids (Hkv == n_heads).
 * A zero key gets norm 0 and the codes of the zero vector.  Every finite
 * Hadamard/Lloyd-Max key is encoded from its unit vector whatever its scale
 * (its fp32 norm is +inf only where |k| exceeds the fp32 range); a key with an
 * infinite or NaN element gets the codes of the zero vector and the norm its
 * sum of squares gives (+inf, or NaN when an element is NaN).
 * kvq_decode_attn_append encodes every key the same way.
 * Errors: KVQ_ERR_INVALID_ARG (sizes, NULL, misaligned, signs not +-1, t0 out
 *   of range when write_pos == NULL), KVQ_ERR_UNSUPPORTED (d, b not built),
 *   KVQ_ERR_DEVICE. */
kvq_status kvq_encode_keys(const kvq_codebook* cb, const int8_t* signs, const void* keys, kvq_dtype kdtype,
                           int B, int Hkv, int64_t T_new, uint8_t* codes, float* norms, int64_t T_cap,
                           int64_t t0, const int32_t* write_pos, void* stream);

/* Read path, scores only (AXELRAM, Abstract: table lookup on read; LOOKAT for
 * PQ; for POT the table holds the query elements sign-flipped and shifted by
 * each magnitude, so a score is a sum of shifted query elements times alpha).
 * scores[b][h][t] = raw estimate of q.k_t (no softmax scale) for
 * t < len_b; scores at t >= len_b are set to -inf.
 *   q:        device [B][Hq][d], dtype qdtype.
 *   codes, norms: as written by kvq_encode_keys (norms ignored for PQ).
 *   seq_lens: device [B] int32 valid lengths (0..T_cap), or NULL for T_cap.
 *   scores:   device [B][Hq][T_cap] fp32, written.
 * Errors: as kvq_encode_keys. */
kvq_status kvq_score(const kvq_codebook* cb, const int8_t* signs, const void* q, kvq_dtype qdtype,
                     const uint8_t* codes, const float* norms, int B, int Hq, int Hkv, int64_t T_cap,
                     const int32_t* seq_lens, float* scores, void* stream);

/* Bytes of device workspace kvq_decode_attn needs for this shape and split
 * count (n_splits = 0: the library's choice).  0 on invalid arguments.  The
 * workspace holds one arrival counter per (batch, kv head, head group) and
 * the split partials, exchanged between workgroups as device-scope atomic
 * words; a zero word is an empty slot. */
size_t kvq_decode_attn_workspace(const kvq_codebook* cb, int B, int Hq, int Hkv, int64_t T_cap, int n_splits);

/* Fused decode attention from codes (AXELRAM, Abstract: scores by table
 * lookup on read, no inverse transform; shift-accumulate attention page,
 * English abstract: decode attention fused with an online softmax): scores,
 * online softmax over t of scale * s, and the AV product over v, in one pass
 * over the cache split along T across workgroups, followed by a log-sum-exp
 * merge of the splits.
 *   v:        device [B][Hkv][T_cap][d], dtype vdtype.
 *   scale:    softmax scale (1/sqrt(d) for standard attention).
 *   out:      device [B][Hq][d], dtype odtype, written.  A sequence of
 *             length 0 gives zeros.
 *   workspace: device, at least kvq_decode_attn_workspace(...) bytes with the
 *             same n_splits (may be NULL when that size is 0).  All of it must
 *             be zero before the first call using this workspace (allocate it
 *             zero-filled); every completed call leaves it zero again, so the
 *             workspace can be reused by later calls ordered on the device,
 *             with any shape, without clearing.  Calls that share a workspace
 *             concurrently race.
 *   n_splits: 0 = library's choice; otherwise 1..T_cap/64 rounded up (the
 *             result is the same up to rounding for every n_splits).
 * Errors: as kvq_encode_keys, plus KVQ_ERR_WORKSPACE, and KVQ_ERR_UNSUPPORTED
 *   when T_cap * 4 * max(d, 32) >= 2^31 (the kernels address a cache split
 *   with 32-bit offsets). */
kvq_status kvq_decode_attn(const kvq_codebook* cb, const int8_t* signs, const void* q, kvq_dtype qdtype,
                           const uint8_t* codes, const float* norms, const void* v, kvq_dtype vdtype,
                           int B, int Hq, int Hkv, int64_t T_cap, const int32_t* seq_lens, float scale,
                           void* out, kvq_dtype odtype, void* workspace, size_t ws_bytes, int n_splits,
                           void* stream);

/* Size in bytes of the device array that kvq_decode_attn_noalloc uses as its
 * workspace (one array per device, held by the library until the process ends). */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

/* kvq_decode_attn without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The split partials and arrival counters
 * live in a library-owned device array of KVQ_NOALLOC_SCRATCH_BYTES bytes per
 * device; the call allocates nothing (no hipMalloc, no hipFree).  The caller
 * still passes every input and the output.  Arguments, layouts, results and
 * errors are those of kvq_decode_attn (same kernels, same split choice, so the
 * output equals kvq_decode_attn's for the same n_splits, bit for bit).
 * The first call on a device (that device current) looks up the array's
 * device address and clears it with a fill kernel on `stream`; every completed
 * call leaves it ready for the next.  All calls on one device share the one
 * array: two calls on the same device that are not ordered with respect to
 * each other (different streams with no dependency, or host threads racing)
 * corrupt each other's partials.
 * Errors: those of kvq_decode_attn, and KVQ_ERR_WORKSPACE when the shape needs
 *   more than KVQ_NOALLOC_SCRATCH_BYTES of workspace
 *   (kvq_decode_attn_workspace(...) > KVQ_NOALLOC_SCRATCH_BYTES). */
kvq_status kvq_decode_attn_noalloc(const kvq_codebook* cb, const int8_t* signs, const void* q, kvq_dtype qdtype,
                                   const uint8_t* codes, const float* norms, const void* v, kvq_dtype vdtype,
                                   int B, int Hq, int Hkv, int64_t T_cap, const int32_t* seq_lens, float scale,
                                   void* out, kvq_dtype odtype, int n_splits, void* stream);

/* One decode step in one launch: write path and read path together (AXELRAM,
 * Abstract: transform on write, table lookup on read).  For every (b, kv
 * head) the key new_keys[b][h] is encoded exactly as kvq_encode_keys does and
 * stored at position len_b - 1 of codes and norms (len_b = seq_lens[b]
 * clamped to T_cap, or T_cap when seq_lens is NULL; nothing is stored when
 * len_b = 0), and attention over positions [0, len_b), the new key included,
 * is computed exactly as kvq_decode_attn does.  The result equals
 * kvq_encode_keys(write_pos = len - 1) followed by kvq_decode_attn, bit for
 * bit.  The new token's value must already be in v at position len_b - 1.
 *   new_keys: device [B][Hkv][d], dtype kdtype, 16-byte aligned.
 *   codes, norms: the cache, read and written (rows len_b - 1).
 *   Every other argument as kvq_decode_attn, including the workspace (same
 *   size, from kvq_decode_attn_workspace).
 * Hadamard/Lloyd-Max and power-of-two codebooks (for the latter, norms holds
 * the per-key scales and signs may be NULL).
 * Errors: as kvq_decode_attn; KVQ_ERR_UNSUPPORTED for a PQ codebook. */
kvq_status kvq_decode_attn_append(const kvq_codebook* cb, const int8_t* signs, const void* new_keys,
                                  kvq_dtype kdtype, const void* q, kvq_dtype qdtype, uint8_t* codes, float* norms,
                                  const void* v, kvq_dtype vdtype, int B, int Hq, int Hkv, int64_t T_cap,
                                  const int32_t* seq_lens, float scale, void* out, kvq_dtype odtype,
                                  void* workspace, size_t ws_bytes, int n_splits, void* stream);

/* Decode attention with the values quantized too (an extension of the key
 * codec of AXELRAM, Abstract, to V; the shift-accumulate attention page,
 * English abstract, quantizes V in its own codec).  The value rows are encoded
 * by kvq_encode_keys with the same codebook and signs (vcodes, vnorms have the
 * layout of codes, norms), and the output is
 *   out[b][h] = sum_t p_t * |v_t| * D H^T c_hat(v_t) / sum_t p_t
 * with p_t the softmax weights of kvq_decode_attn.  The weighted sum is taken
 * in the rotated domain and D H^T is applied once per query head.
 *   vcodes: device [B][Hkv][T_cap][d*b/8], vnorms: device [B][Hkv][T_cap]
 *   fp32, both 16-byte aligned.  Every other argument, the workspace
 *   (kvq_decode_attn_workspace) and the errors are those of kvq_decode_attn.
 *   The products run in fp16 with fp32 accumulation: |v_t| times a level
 *   must stay within the fp16 range.
 * Hadamard/Lloyd-Max codebooks only (KVQ_ERR_UNSUPPORTED for PQ and POT). */
kvq_status kvq_decode_attn_qv(const kvq_codebook* cb, const int8_t* signs, const void* q, kvq_dtype qdtype,
                              const uint8_t* codes, const float* norms, const uint8_t* vcodes, const float* vnorms,
                              int B, int Hq, int Hkv, int64_t T_cap, const int32_t* seq_lens, float scale, void* out,
                              kvq_dtype odtype, void* workspace, size_t ws_bytes, int n_splits, void* stream);

/* Bytes of device workspace kvq_select_signs needs (0 on invalid arguments or
 * a PQ codebook). */
size_t kvq_select_signs_workspace(const kvq_codebook* cb, int n_cal, int Hq, int Hkv, int64_t T, int C);

/* One-time choice of the sign pattern D (AXELRAM, Key Points / Abstract: a
 * gradient-free selection among candidate sign patterns, evaluated once on a
 * few calibration samples).  The pages rank candidates by perplexity, which
 * needs a model; here candidate c is ranked by the attention-output error it
 * causes:
 *   errors[c] = sum ||o_c - o||^2 / sum ||o||^2 over every (sample, query head),
 * o = exact attention (fp32, no quantization), o_c = kvq_decode_attn of the
 * calibration keys encoded with pattern c (kvq_encode_keys, same codebook).
 *   candidates: host [C][d] int8, each entry +1 or -1.
 *   q: device [n_cal][Hq][d]; keys, v: device [n_cal][Hkv][T][d] (dtypes as
 *      given, 16-byte aligned), 1 <= T <= 8192.
 *   scale: softmax scale.
 *   errors: host [C] fp32, written.  best: host, the index of the smallest
 *      error (lowest index on ties), written.
 *   workspace: device, >= kvq_select_signs_workspace(...) bytes, 256-byte
 *      aligned; its contents on entry do not matter.
 * Synchronous: the call waits for `stream` before it returns.
 * Errors: KVQ_ERR_INVALID_ARG (sizes, NULL, misaligned, a candidate entry not
 *   +-1), KVQ_ERR_UNSUPPORTED (PQ codebook, T out of range), KVQ_ERR_WORKSPACE,
 *   KVQ_ERR_DEVICE. */
kvq_status kvq_select_signs(const kvq_codebook* cb, const int8_t* candidates, int C, const void* q,
                            kvq_dtype qdtype, const void* keys, kvq_dtype kdtype, const void* v, kvq_dtype vdtype,
                            int n_cal, int Hq, int Hkv, int64_t T, float scale, float* errors, int* best,
                            void* workspace, size_t ws_bytes, void* stream);

/* Measurement aid, not a step of the method: the streaming ceiling of
 * kvq_decode_attn on this cache.  Reads every byte a decode call reads from
 * the cache -- codes, norms and fp16 V of every (batch, kv head) row below
 * T_cap -- with the decode kernel's grid (the token axis cut into n_splits
 * spans of a multiple of 64 tokens, one workgroup of 12 waves per span and
 * (batch, kv head)) and access pattern (64 tokens per wave and chunk, one
 * chunk requested ahead, non-temporal loads), and discards it.
 *   codes: device [B][Hkv][T_cap][bytes_per_key]; norms: device
 *     [B][Hkv][T_cap] fp32; v: device [B][Hkv][T_cap][d] fp16; all 16-byte
 *     aligned.  Built for d = 64 with 32-byte code rows and d = 128 with
 *     64-byte code rows.
 *   n_splits: 1..256 (the split kvq_decode_attn_workspace's n_splits picks).
 *   sink: device, >= 4 bytes; written only when a checksum of the data hits a
 *     fixed value (so the loads cannot be elided).
 * Errors: KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED (other d or row size, or
 *   T_cap * 4 * max(d, 32) >= 2^31), KVQ_ERR_DEVICE. */
kvq_status kvq_stream_read(const uint8_t* codes, const float* norms, const void* v, int B, int Hkv, int64_t T_cap,
                           int d, int bytes_per_key, int n_splits, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
