// Read-path kernels of libkvq: per-query lookup tables in LDS, scores from
// stored codes, and fused decode attention (online softmax + AV product).
//
// Method: "AXELRAM: Quantize Once, Never Dequantize" (Abstract): the query is
// transformed once, a table of query-coordinate x codebook-level products is
// built, and a key's score is the sum over coordinates of the table entries
// its stored indices select, times the key norm -- no inverse transform.
// "LOOKAT" summary page (AI Summary, Abstract): the product-quantization
// variant, whose table holds query-subvector x centroid inner products.
// Shift-accumulate attention page (English abstract): decode attention fused
// with an online softmax.
//
// Work decomposition (one workgroup = 8 waves of 64 lanes, or 12 for d = 64 with fp16 V and long splits):
//   workgroup <- (batch b, kv head, group of GG query heads, split of T);
//   prologue: each of the GG queries is held by one wave for d <= 128 (coordinate i on lane i % 64), else
//   16 coordinates per lane as in the write path; for the Hadamard codec it is sign-flipped and rotated
//   with the write path's sums and differences (lane exchanges, and in-register stages where a lane holds
//   several coordinates) and scaled per head; the table for all GG heads is in LDS as
//   [GG/HW][rows][cols] vectors of HW heads (HW = min(GG, 4)): 32-bit fixed-point entries for the scalar
//   codecs (each head at its own power-of-two scale), fp32 for PQ, so one ds_read_b128 at (row, code)
//   returns the entries of four heads.  Where a row holds one coordinate, the lanes of the prologue write
//   the rows themselves; otherwise q' goes through LDS to a separate table build;
//   main loop: a wave takes 64 keys at a time, lane <-> key.  The next chunk's codes and norms are
//   fetched while the current one is scored; fp16 V slices are fetched one chunk ahead (8 waves, d <= 64)
//   or when their chunk starts (12 waves, d = 128), and just before their products at d = 256.
//   Every lane unpacks its key's codes from registers and gathers one vector
//   per (row, head quad); all lanes read the same row at once and a row
//   holds at most `cols` entries, so a wave's gather touches one contiguous
//   span of LDS (no bank conflicts for cols <= 16).  Scores feed an online
//   softmax whose running maximum is only raised when a score exceeds it by
//   more than 2^8 (so probabilities stay <= 256), and the probabilities are
//   staged through LDS as the B operand of MFMA 16x16x16 f16 (fp32 values:
//   16x16x4 f32) whose A operand is V^T, giving out^T[dim][head] in the
//   matrix-core accumulators.  The waves merge their (max, sum, acc)
//   through LDS; the splits of one (b, kv head, head group) are merged by
//   the last of its workgroups to finish (log-sum-exp merge), elected by an
//   arrival counter in the workspace that it resets to zero; the partials
//   travel as device-scope atomic words that are never zero, so the merger
//   reads each word until it has been written and then clears it.
#pragma once

#include <type_traits>

#include "encode_dev.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kThreads = kReadThreads;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 64;
constexpr float kLazyHeadroom = 8.0f;  // log2 of the largest probability allowed before rescaling
constexpr int kMaxSplits = 256;        // T splits per (b, kv head, head group)
constexpr int kRecPad = 4;             // split partial record = D accumulators + max + sum, padded to D + 4
constexpr int kMergeTile = 16;         // splits whose partials the merging workgroup loads at once

// ---- buffer-resource loads: 32-bit offsets from a per-split base, and every byte past the split's valid
// range reads as 0, so the last (partial) chunk needs neither clamping nor branches.
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufFlags);
}

template <int B, int NW>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[NW], int i) {
  const int bit = i * B;
  const int word = bit >> 5;
  const int off = bit & 31;
  uint32_t x = w[word] >> off;
  if (off + B > 32) x |= w[word + 1 < NW ? word + 1 : NW - 1] << (32 - off);
  return x & ((1u << B) - 1u);
}

// Table of a scalar codec (one b-bit code per coordinate, one level per code value, a per-key factor
// stored beside the codes).  A table row covers GRP consecutive coordinates whose codes fill one 4-bit
// field of the packed row (GRP = 4 / b for b = 1, 2, 4; one coordinate for b = 3): its column is that
// field, and entry (r, n) = sum_k q'_{r GRP + k} * lv[code_k(n)] with code_k(n) the k-th b-bit part of n and
// lv the level of each code value.  So every table lookup adds 4 bits' worth of codes, and a key takes
// d b / 4 lookups (d for b = 3) however many coordinates a row spans.
template <int D_, int BITS>
struct ScalarTable {
  static constexpr int D = D_;
  static constexpr int LEVELS = 1 << BITS;
  static constexpr int GRP = BITS == 3 ? 1 : 4 / BITS;  // coordinates per table row
  static constexpr int ROWS = D / GRP;
  static constexpr int COLS = 1 << (BITS * GRP);
  static constexpr int CODE_BITS = BITS;
  static constexpr int BPK = D * BITS / 8;
  static constexpr int NW = (BPK + 3) / 4;
  static constexpr bool kNorm = true;
  static constexpr bool kNibbles = BITS * GRP == 4;  // rows indexed by the 4-bit fields of the packed codes
  static constexpr bool kIntLut = true;              // fixed-point table entries, summed exactly in 32-bit integers
  static constexpr bool kRowPerCoord = GRP == 1;     // a table row holds one coordinate's entries
  // where the query prologue writes the table itself (d <= 128, one coordinate per row) rows are padded by 16
  // bytes: the lanes of a wave, each writing one row, then spread over the LDS banks instead of all landing
  // on the same one
  static constexpr int kRowPad = D <= 128 && GRP == 1 ? 16 : 0;
  // cache policy of the decode's streaming loads (codes, norms, values, new keys): non-temporal, since each
  // byte is read once per call and by a single load
  static constexpr int kLoadPolicy = kStreamLoad;
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[NW], int i) { return code_at<BITS, NW>(w, i); }
  __device__ static __forceinline__ float level_max(const float* lv) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < LEVELS; ++j) m = fmaxf(m, fabsf(lv[j]));
    return m;
  }
  // Table of head g, with the (transformed) query q' times 2^e_g (fix_exp) held in qs: every entry is the
  // integer nearest to its value times 2^e_g, so the table of head g sums to at most 2^30 in magnitude along
  // any choice of one entry per row and integer sums never overflow.  One HW-wide entry (HW heads) per (head group, row,
  // column); each work item fills JPT consecutive columns of one (head group, row).
  // nothing to request before the queries arrive
  template <int GG, int NT>
  struct Pre {};
  template <int GG, int HW, int NT = kThreads>
  __device__ static Pre<GG, NT> prefetch(const AttnParams&, int, int) {
    return {};
  }
  template <int GG, int HW, int NT = kThreads>
  __device__ static void build(const AttnParams&, const float* qs, const float* qa, const float* lv, float* lut,
                               int, int tid, const Pre<GG, NT>&) {
    using E = typename VecI<HW>::type;
    constexpr int JPT = COLS < 4 ? COLS : 4;
    constexpr int NJ = COLS / JPT;
    constexpr int total = (GG / HW) * ROWS * NJ;
    E* L = reinterpret_cast<E*>(lut);
    for (int e = tid; e < total; e += NT) {
      const int j0 = (e % NJ) * JPT;
      const int r = (e / NJ) % ROWS;
      const int g0 = (e / (NJ * ROWS)) * HW;
      float qv[HW][GRP];  // the rotated query elements, already times the head's scale 2^e_g
#pragma unroll
      for (int h = 0; h < HW; ++h)
#pragma unroll
        for (int k = 0; k < GRP; ++k) qv[h][k] = qs[(g0 + h) * D + r * GRP + k];
      E* row = reinterpret_cast<E*>(reinterpret_cast<char*>(L) + (size_t)(e / NJ) * (COLS * sizeof(E) + kRowPad)) + j0;
#pragma unroll
      for (int jj = 0; jj < JPT; ++jj) {
        const int n = j0 + jj;
        int x[HW];
#pragma unroll
        for (int h = 0; h < HW; ++h) {
          float t = qv[h][0] * lv[n & (LEVELS - 1)];
#pragma unroll
          for (int k = 1; k < GRP; ++k) t += qv[h][k] * lv[(n >> (k * BITS)) & (LEVELS - 1)];
          x[h] = (int)__builtin_rintf(t);
        }
        if constexpr (HW == 4) row[jj] = make_int4(x[0], x[1], x[2], x[3]);
        else if constexpr (HW == 2) row[jj] = make_int2(x[0], x[1]);
        else row[jj] = x[0];
      }
    }
  }
};

// Hadamard + Lloyd-Max codec: the query is rotated, q' = H D q / sqrt(d), and the levels are the Lloyd-Max
// levels of N(0, 1/d); the per-key factor is the key norm.
template <int D_, int BITS>
struct HlmScorer : ScalarTable<D_, BITS> {
  static constexpr bool kRotate = true;
};

// Power-of-two codec (shift-accumulate attention page, English abstract): no rotation, q' = q; the level of
// code value c is (-1)^sign * 2^-j (or (3/4) 2^-j', the mantissa term), so a table entry is a query element
// with its sign flipped and shifted (for fp16 queries the scaled entries are the exact shifted integers
// whenever the element is at least 2^-10 of the query's sum of magnitudes); the per-key factor is max |k_i|.
template <int D_, int BITS>
struct PotScorer : ScalarTable<D_, BITS> {
  static constexpr bool kRotate = false;
};

// Scorer for product quantization: rows = subspaces, cols = centroids.  CB = 8: one byte per subspace
// (K <= 256); CB = 4: two subspaces per byte, the even one in the low nibble (K <= 16), so a row holds 16
// entries and the gathers of a wave stay within one row like the scalar codecs' (no bank conflicts).
template <int D_, int M, int CB = 8>
struct PqScorer {
  static_assert(CB == 8 || (CB == 4 && M % 2 == 0), "4-bit codes pair up subspaces");
  static constexpr int D = D_;
  static constexpr int ROWS = M;
  static constexpr int COLS = 1 << CB;
  static constexpr int CODE_BITS = CB;
  static constexpr int BPK = M * CB / 8;
  static constexpr int NW = (BPK + 3) / 4;
  static constexpr int DS = D / M;
  static constexpr bool kRotate = false;
  static constexpr bool kNorm = false;
  static constexpr bool kNibbles = CB == 4;
  static constexpr bool kIntLut = false;
  static constexpr bool kRowPerCoord = false;
  static constexpr int kRowPad = 0;
  static constexpr int kLoadPolicy = 0;  // default policy: the non-temporal one measured slower on these small launches
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[NW], int i) {
    if constexpr (CB == 4) return (w[i >> 3] >> (4 * (i & 7))) & 15u;
    else return (w[i >> 2] >> (8 * (i & 3))) & 255u;
  }
  __device__ static __forceinline__ float level_max(const float*) { return 1.0f; }
  // LUT[g][s][c] = q_{g,s} . C_{s,c}; columns c >= K are zero (never selected).
  // The centroids come in as 16-byte buffer loads of up to four entries at once, issued before any is used
  // (behind a branch on c < K each entry's load would wait for the one before); a load past the head's
  // centroids reads zeros, and entries with c >= K are set to zero after the loads.  The first batch is
  // requested by prefetch, before the queries arrive (the centroids do not depend on them), except for
  // 32-coordinate sub-vectors, whose batch would hold 128 registers through the query prologue.
  template <int GG, int NT>
  static constexpr int kIT = (GG * ROWS * COLS + NT - 1) / NT;  // entries per thread
  template <int GG, int NT>
  static constexpr int kBatch = kIT<GG, NT> < 4 ? kIT<GG, NT> : 4;
  static constexpr bool kPrefetch = DS <= 16;
  template <int GG, int NT>
  struct Pre {
    float cv[kPrefetch ? kBatch<GG, NT> : 1][DS];
  };
  template <int GG, int HW, int NT>
  __device__ static void load_batch(const AttnParams& p, int kvh, int tid, int i0, float (&cv)[kBatch<GG, NT>][DS]) {
    static_assert(DS % 4 == 0, "sub-vectors of whole 16-byte loads");
    const int K = p.pq_K;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.pq_cent + (size_t)kvh * M * K * DS, (int64_t)M * K * DS * 4);
#pragma unroll
    for (int b = 0; b < kBatch<GG, NT>; ++b) {
      const int idx = tid + (i0 + b) * NT;
      const int c = (idx / HW) % COLS;
      const int s = (idx / (HW * COLS)) % ROWS;
#pragma unroll
      for (int k4 = 0; k4 < DS / 4; ++k4) {
        const float4_t v = __builtin_bit_cast(
            float4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, ((s * K + c) * DS + 4 * k4) * 4, 0, 0));
        cv[b][4 * k4 + 0] = v[0]; cv[b][4 * k4 + 1] = v[1]; cv[b][4 * k4 + 2] = v[2]; cv[b][4 * k4 + 3] = v[3];
      }
    }
  }
  template <int GG, int HW, int NT = kThreads>
  __device__ static Pre<GG, NT> prefetch(const AttnParams& p, int kvh, int tid) {
    Pre<GG, NT> pre;
    if constexpr (kPrefetch) load_batch<GG, HW, NT>(p, kvh, tid, 0, pre.cv);
    return pre;
  }
  template <int GG, int HW, int NT = kThreads>
  __device__ static void build(const AttnParams& p, const float* qs, const float*, const float*, float* lut, int kvh,
                               int tid, const Pre<GG, NT>& pre) {
    constexpr int total = GG * ROWS * COLS;
    constexpr int IT = kIT<GG, NT>, BATCH = kBatch<GG, NT>;
    const int K = p.pq_K;
    for (int i0 = 0; i0 < IT; i0 += BATCH) {
      float cv[BATCH][DS];
      if (kPrefetch && i0 == 0) {
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
#pragma unroll
          for (int k = 0; k < DS; ++k) cv[b][k] = pre.cv[kPrefetch ? b : 0][k];
      } else {
        load_batch<GG, HW, NT>(p, kvh, tid, i0, cv);
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int idx = tid + (i0 + b) * NT;
        if (i0 + b >= IT || idx >= total) continue;
        const int hh = idx % HW;
        const int c = (idx / HW) % COLS;
        const int s = (idx / (HW * COLS)) % ROWS;
        const int g = (idx / (HW * COLS * ROWS)) * HW + hh;
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < DS; ++k) acc += qs[g * D + s * DS + k] * cv[b][k];
        lut[idx] = c < K ? acc : 0.0f;
      }
    }
  }
};

// LDS layout of the read kernels.  kRec: the decode kernels' per-wave records (accumulators padded to RS floats
// per row, maxima, sums) and the workgroup's merged partials; they get a region of their own when the whole
// layout still fits comfortably in the 160 KB of LDS (so a wave can write its record as soon as its loop
// ends), else they reuse the table's space once every wave is done with it.
template <class S, int GG, int NWV = kWaves, bool kRec = true>
struct LdsPlan {
  static constexpr int HW = GG < 4 ? GG : 4;
  static constexpr int NQ = GG / HW;
  static constexpr int RS = S::D + 4;
  static constexpr size_t lut_bytes = (size_t)NQ * S::ROWS * (S::COLS * HW * 4 + S::kRowPad);
  static constexpr size_t lut_al = (lut_bytes + 15) / 16 * 16;
  static constexpr size_t red_bytes = kRec ? (size_t)NWV * GG * (RS + 2) * 4 + (size_t)GG * (S::D + 2) * 4 : 0;
  static constexpr bool kRedSeparate = kRec && lut_al + red_bytes + 48 * 1024 <= 160 * 1024;
  static constexpr size_t red_off = kRedSeparate ? lut_al : 0;
  static constexpr size_t red_end = red_off + red_bytes;
  static constexpr size_t region0 = ((red_end > lut_bytes ? red_end : lut_bytes) + 15) / 16 * 16;
  // consts: 16 levels (+0), merge flag (+96), per-wave progress (+128, up to 16 waves), appended key's codes
  // (+192), its norm (+320) and its ready flag (+324)
  static constexpr size_t consts_off = region0;
  static constexpr size_t newcode_off = consts_off + 192;
  static constexpr size_t newnorm_off = consts_off + 320;
  static constexpr size_t qs_off = consts_off + 336;              // GG * D floats
  static constexpr size_t qa_off = qs_off + (size_t)GG * S::D * 4;  // GG floats: sum_i |q'_{g,i}|
  static constexpr size_t pst_off = qa_off + 32;
  // probability staging rows, padded so that the GG rows a matrix-core operand read touches fall in
  // different LDS banks: fp16 rows 72 halves (36 words) apart, fp32 rows 68 words apart
  static constexpr int pst_row(bool f16) { return kChunk + (f16 ? 8 : 4); }
  static constexpr size_t pst_bytes(bool f16) { return (size_t)NWV * GG * pst_row(f16) * (f16 ? 2 : 4); }
  static constexpr size_t total(bool f16) { return pst_off + pst_bytes(f16); }
};

// Unit decomposition shared by the read kernels.
struct Unit {
  int b, kvh, h0;
  int64_t len;
};

__device__ __forceinline__ Unit decode_unit(const AttnParams& p, int GG) {
  int u = blockIdx.y;
  const int grp = u % p.n_groups;
  u /= p.n_groups;
  Unit r;
  r.kvh = u % p.Hkv;
  r.b = u / p.Hkv;
  r.h0 = r.kvh * p.G + grp * GG;
  int64_t len = p.seq_lens ? (int64_t)p.seq_lens[r.b] : p.T_cap;
  r.len = len < 0 ? 0 : (len > p.T_cap ? p.T_cap : len);
  return r;
}

// Loads the GG queries into qs[g][i] (fp32) and copies the codebook levels into LDS.  For the scalar codecs a
// query takes 16 consecutive coordinates per lane and d/16 lanes (the write path's lane layout).  For the
// Hadamard codec every query is rotated, q' = H D q / sqrt(d), with the write path's arithmetic: sign flip
// folded into the first butterflies, in-register stages for coordinate distances 1 .. 8, lane swizzles for
// 16 .. d/2 (Sylvester order, each stage a + b and a - b).  With fixed-point tables (qa != nullptr) qa[g]
// receives sum_i |q'_{g,i}|, the bound that sets the head's table scale 2^e_g (fix_exp), and qs holds q'
// already multiplied by 2^e_g, so the table build only multiplies by the levels and rounds.
// `between` runs after this thread's query loads are issued and before they are used: the caller issues
// its first cache loads there, so they are in flight during the rotation and the table build (vector
// memory loads complete in order, so waiting for the query does not wait for them).
// Query layout of the read prologue for d <= 128: coordinate i of a query on lane i % 64 of its own wave
// (for d < 64, d lanes of one wave), d / 64 coordinates per lane at d = 128.
template <class S>
struct LaneCoords {
  static constexpr int LPQ = S::D < 64 ? S::D : 64;  // lanes per query
  static constexpr int CPL = S::D / LPQ;             // coordinates per lane: i = l + 64 k
};
template <class S, int GG, int NT>
constexpr bool lane_coord_prologue() {
  return (S::kIntLut || S::kRotate) && S::D <= 128 && GG * LaneCoords<S>::LPQ <= NT;
}
// With one coordinate per table row (b = 3, 4), the lane of q'_{g,i} writes head g's entries of row i itself:
// no pass through qs and no second barrier before the table is used.
template <class S, int GG, int NT>
constexpr bool direct_table() {
  return lane_coord_prologue<S, GG, NT>() && S::kIntLut && S::kRowPerCoord;
}

// TABLE: the caller builds a scalar codec's lookup table from the prologue (the decode and score kernels);
// where direct_table holds, the prologue writes it into `lut` and leaves qs unwritten.
template <class S, int GG, int NT = kThreads, bool TABLE = false, class F>
__device__ void prologue(const AttnParams& p, const Unit& u, float* qs, float* qa, float* lv, int tid, F&& between,
                         void* lut = nullptr) {
  constexpr int D = S::D;
  // the levels come from the kernel arguments with wave-uniform (scalar) reads: indexed per lane they would be
  // a vector load from the argument segment whose wait would hold up everything issued after it
  if (tid == 0) {
#pragma unroll
    for (int t = 0; t < 16; ++t) lv[t] = p.levels[t];
  }
  if constexpr (lane_coord_prologue<S, GG, NT>()) {
    // Every butterfly stage of coordinate distance < 64 is a lane exchange and the one of distance 64
    // (d = 128) is in registers, so the rotation's chain is log2(d) steps instead of 16 coordinates' worth of
    // in-register stages per lane.  The stages run in the write path's order (distances 1, 2, 4, ...) with
    // its sums and differences (signs folded into the first, the lower coordinate of a pair keeps x + partner
    // and the upper one partner - x, as fused multiply-adds with +-1), so q' is the same to the bit.
    constexpr int LPQ = LaneCoords<S>::LPQ, CPL = LaneCoords<S>::CPL;
    const int g = tid / LPQ, l = tid % LPQ;
    const size_t off = ((size_t)u.b * p.Hq + u.h0 + (g < GG ? g : 0)) * D + l;
    float x[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      x[k] = 0.0f;
      if (g < GG)
        x[k] = p.q_f16 ? (float)reinterpret_cast<const _Float16*>(p.q)[off + 64 * k]
                       : reinterpret_cast<const float*>(p.q)[off + 64 * k];
    }
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
    if (g < GG) {  // whole waves or aligned groups of d lanes, so the exchanges stay within the query
      auto lane_xor = [&](float v, auto h_tag) -> float {
        constexpr int H = decltype(h_tag)::value;
        if constexpr (H < 32) return xor_lane<H>(v);
        else return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((tid ^ 32) << 2, __builtin_bit_cast(int, v)));
      };
      if constexpr (S::kRotate) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          // the sign words through wave-uniform (scalar) reads, then selected per lane: coordinate l + 64 k
          // is bit l % 32 of word 2k + l / 32
          const uint32_t sw = (D > 32 && (l >> 5)) ? p.signs[D > 32 ? 2 * k + 1 : 0] : p.signs[D > 32 ? 2 * k : 0];
          x[k] *= ((sw >> (l & 31)) & 1u) ? -1.0f : 1.0f;  // exact
        }
        auto stage = [&](auto h_tag) {
          constexpr int H = decltype(h_tag)::value;
          const float s = (l & H) ? -1.0f : 1.0f;
#pragma unroll
          for (int k = 0; k < CPL; ++k) x[k] = __builtin_fmaf(x[k], s, lane_xor(x[k], h_tag));
        };
        stage(std::integral_constant<int, 1>{});
        stage(std::integral_constant<int, 2>{});
        stage(std::integral_constant<int, 4>{});
        stage(std::integral_constant<int, 8>{});
        if constexpr (D >= 32) stage(std::integral_constant<int, 16>{});
        if constexpr (D >= 64) stage(std::integral_constant<int, 32>{});
        if constexpr (CPL == 2) {  // distance 64: coordinate l keeps a + c, coordinate l + 64 gets a - c
          const float a = x[0], c = x[1];
          x[0] = a + c;
          x[1] = a - c;
        }
      }
      const float rs = S::kRotate ? 1.0f / __builtin_sqrtf((float)D) : 1.0f;
      float sc = 1.0f;
      if (qa != nullptr) {  // sum_i |q'_i| of the query: the bound that scales its fixed-point table
        float a = fabsf(x[0]);
#pragma unroll
        for (int k = 1; k < CPL; ++k) a += fabsf(x[k]);
        a += lane_xor(a, std::integral_constant<int, 1>{});
        a += lane_xor(a, std::integral_constant<int, 2>{});
        a += lane_xor(a, std::integral_constant<int, 4>{});
        a += lane_xor(a, std::integral_constant<int, 8>{});
        if constexpr (D >= 32) a += lane_xor(a, std::integral_constant<int, 16>{});
        if constexpr (D >= 64) a += lane_xor(a, std::integral_constant<int, 32>{});
        a *= rs;
        if (l == 0) qa[g] = a;
        sc = pow2f(fix_exp(a, S::level_max(p.levels)));
      }
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int i = l + 64 * k;
        const float qv = (x[k] * rs) * sc;
        if constexpr (TABLE && direct_table<S, GG, NT>()) {
          // entry (row i, column n) of head g: component g % HW of the HW-wide vector at [g / HW][i][n]
          // (the same products and rounding as the table build below)
          constexpr int HW = GG < 4 ? GG : 4;
          int* row = reinterpret_cast<int*>(reinterpret_cast<char*>(lut) +
                                            ((g / HW) * S::ROWS + i) * (S::COLS * HW * 4 + S::kRowPad)) + g % HW;
#pragma unroll
          for (int n = 0; n < S::COLS; ++n) row[n * HW] = (int)__builtin_rintf(qv * p.levels[n]);
        } else {
          qs[g * D + i] = qv;
        }
      }
    }
  } else if constexpr (S::kIntLut || S::kRotate) {
    constexpr int LPQ = EncLanes<D>::LPK;  // lanes per query (a power of two <= 16, so groups never straddle waves)
    static_assert(GG * LPQ <= NT, "one lane per 16 coordinates of every query");
    const int g = tid / LPQ, k = tid % LPQ;
    const size_t off = ((size_t)u.b * p.Hq + u.h0 + (g < GG ? g : 0)) * D + kEncCpl * k;
    uint32_t raw[kEncCpl];
#pragma unroll
    for (int j = 0; j < kEncCpl; ++j) raw[j] = 0u;
    if (g < GG) {  // 16 coordinates: two 16-byte loads (fp16) or four (fp32)
      if (p.q_f16) {
        const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(p.q) + off);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint4 v = src[h];
          raw[4 * h + 0] = v.x; raw[4 * h + 1] = v.y; raw[4 * h + 2] = v.z; raw[4 * h + 3] = v.w;
        }
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(p.q) + off);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint4 v = src[h];
          raw[4 * h + 0] = v.x; raw[4 * h + 1] = v.y; raw[4 * h + 2] = v.z; raw[4 * h + 3] = v.w;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
    if (g < GG) {  // whole groups of LPQ lanes, so the swizzles stay within the query's lanes
      float x[kEncCpl];
      if (p.q_f16) key_lane_floats<true>(raw, x);
      else key_lane_floats<false>(raw, x);
      if constexpr (S::kRotate) {
        float sg[kEncCpl];
        lane_signs<D>(p.signs, k, sg);
        (void)rotate_key_lane<D>(x, k, sg);
      }
      const float rs = S::kRotate ? 1.0f / __builtin_sqrtf((float)D) : 1.0f;
      float sc = 1.0f;
      if (qa != nullptr) {  // sum_i |q'_i| of the query: the bound that scales its fixed-point table
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < kEncCpl; ++j) a += fabsf(x[j]);
        a = key_lanes_sum<LPQ>(a) * rs;
        if (k == 0) qa[g] = a;
        sc = pow2f(fix_exp(a, S::level_max(p.levels)));
      }
#pragma unroll
      for (int j = 0; j < kEncCpl; ++j) qs[g * D + kEncCpl * k + j] = (x[j] * rs) * sc;
    }
  } else {
    // the queries first, then the caller's loads, so that waiting for the queries does not wait for those
    constexpr int QPT = (GG * D + NT - 1) / NT;  // query elements per thread
    float qv[QPT];
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int idx = tid + j * NT;
      const size_t off = ((size_t)u.b * p.Hq + u.h0 + (idx < GG * D ? idx : 0) / D) * D + idx % D;
      qv[j] = idx >= GG * D ? 0.0f
              : p.q_f16   ? (float)reinterpret_cast<const _Float16*>(p.q)[off]
                          : reinterpret_cast<const float*>(p.q)[off];
    }
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < QPT; ++j)
      if (tid + j * NT < GG * D) qs[tid + j * NT] = qv[j];
  }
  lds_barrier();
}

// Accumulator of a scorer's table sums: 32-bit integers for fixed-point tables, else fp32.
template <class S>
using ScoreAcc = typename std::conditional<S::kIntLut, uint32_t, float>::type;

// Scores of the key held by this lane for all GG heads (before the norm; for fixed-point tables before the
// head's scale 2^-e_g as well).  `lut` is the byte address of the table in LDS.
//
// Every coordinate i contributes the table entry at (row i, column code_i) for each head group; its LDS
// byte offset within the row is code_i * ES.  The gathers run one stage (4 coordinates x NQ head groups)
// ahead of the adds that consume them, so 2*4*NQ reads are in flight; the scheduling barriers keep the
// compiler from folding the stages back together (which would hold every gather of the key in registers).
// The first stage initialises the sums.
template <class S, int GG, int ST = 4>
__device__ __forceinline__ void lut_scores(const unsigned char* __restrict__ lut, const uint32_t (&w)[S::NW],
                                           ScoreAcc<S> (&acc)[GG]) {
  constexpr int HW = GG < 4 ? GG : 4;
  constexpr int NQ = GG / HW;
  constexpr int ES = HW * 4;  // bytes per table entry
  constexpr int LG = ES == 16 ? 4 : (ES == 8 ? 3 : 2);
  constexpr uint32_t NMASK = 0xFu << LG;
  using E = typename std::conditional<S::kIntLut, typename VecI<HW>::type, typename VecF<HW>::type>::type;
  static_assert(S::ROWS % ST == 0, "rows come in whole stages");  // ST: rows per stage
  constexpr int NST = S::ROWS / ST;

  // byte offset of coordinate i's entry within its row
  auto col_offset = [&](int i) -> uint32_t {
    if constexpr (S::kNibbles) {
      // Two 4-bit codes per byte.  For the odd coordinate of byte m the offset is (w >> 8m) masked to the
      // nibble's bits shifted by LG, for the even one the same with w shifted left by 4 first, so each
      // address costs one masked byte extract (for ES = 16 a single byte-select AND).  The left shift is
      // kept opaque so that the compiler does not merge it into the extracts.
      const int k = i / 8, m = (i % 8) / 2;
      uint32_t x;
      if (i % 2) {
        x = w[k] >> (4 - LG);
      } else if constexpr (LG == 4) {
        asm("v_lshlrev_b32 %0, 4, %1" : "=v"(x) : "v"(w[k]));
      } else {
        x = w[k] << LG;
      }
      uint32_t a;
      if (LG == 4 && m == 1)  // byte 1 under the mask in one byte-select AND (the compiler emits shift + AND)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
            : "=v"(a) : "v"(x), "s"(NMASK));
      else
        a = (m == 0 ? x : __builtin_amdgcn_ubfe(x, 8 * m, 8)) & NMASK;
      return a;
    } else {
      return S::code(w, i) * (uint32_t)ES;
    }
  };
  E buf[2][ST * NQ];
  auto issue = [&](int st, E* b) {
#pragma unroll
    for (int cc = 0; cc < ST; ++cc) {
      const int i = ST * st + cc;
      const uint32_t a = col_offset(i);
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq)
        b[cc * NQ + qq] = *reinterpret_cast<const E*>(lut + (size_t)(qq * S::ROWS + i) * (S::COLS * ES + S::kRowPad) + a);
    }
  };
  issue(0, buf[0]);
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    if (st + 1 < NST) issue(st + 1, buf[(st + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cc = 0; cc < ST; ++cc)
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) {
        if (st == 0 && cc == 0) set_from(acc + qq * HW, buf[0][qq]);
        else add_into(acc + qq * HW, buf[st & 1][cc * NQ + qq]);
      }
    // the stage's sums are materialised here: the compiler may not sink the adds past the later gathers
#pragma unroll
    for (int g = 0; g < GG; ++g) asm volatile("" : "+v"(acc[g]));
    __builtin_amdgcn_sched_barrier(0);
  }
}


// The N-byte code row at voff + soff into little-endian 32-bit words, loaded with cache policy POL.
template <int N, int POL = 0>
__device__ __forceinline__ void load_code_row_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t (&w)[(N + 3) / 4]) {
  if constexpr (N % 16 == 0) {
#pragma unroll
    for (int k = 0; k < N / 16; ++k) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16 * k, POL);
      w[4 * k + 0] = x[0]; w[4 * k + 1] = x[1]; w[4 * k + 2] = x[2]; w[4 * k + 3] = x[3];
    }
  } else if constexpr (N % 8 == 0) {
#pragma unroll
    for (int k = 0; k < N / 8; ++k) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff + 8 * k, POL);
      w[2 * k + 0] = x[0]; w[2 * k + 1] = x[1];
    }
  } else if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) w[k] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff + 4 * k, POL);
  } else {
    static_assert(N % 2 == 0, "code rows are an even number of bytes");
#pragma unroll
    for (int k = 0; k < (N + 3) / 4; ++k) w[k] = 0;
#pragma unroll
    for (int k = 0; k < N / 2; ++k)
      w[k / 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff + 2 * k, POL) << (16 * (k % 2));
  }
}

// DPL consecutive V elements (fp16 or fp32) at voff + soff: the slice this lane contributes to the MFMA
// A operand, loaded with cache policy POL.  Past the split's valid range the elements read as 0.
template <typename PT, int DPL, typename VR, int POL = 0>
__device__ __forceinline__ VR load_vrow_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  VR out;
  if constexpr (DPL == 1) {
    out = VR{};
    if constexpr (sizeof(PT) == 2) out[0] = __builtin_bit_cast(PT, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, POL));
    else out[0] = __builtin_bit_cast(PT, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POL));
  } else {
    constexpr int BYTES = DPL * (int)sizeof(PT);
    static_assert(BYTES == (int)sizeof(VR), "slice type");
    if constexpr (BYTES == 4) {
      out = __builtin_bit_cast(VR, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POL));
    } else if constexpr (BYTES == 8) {
      out = __builtin_bit_cast(VR, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POL));
    } else if constexpr (BYTES == 16) {
      out = __builtin_bit_cast(VR, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POL));
    } else {
      static_assert(BYTES % 16 == 0, "V slice is a multiple of 16 bytes");
      typedef unsigned u4 __attribute__((ext_vector_type(4)));
      struct Parts { u4 x[BYTES / 16]; } parts;
#pragma unroll
      for (int k = 0; k < BYTES / 16; ++k) parts.x[k] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16 * k, POL);
      out = __builtin_bit_cast(VR, parts);
    }
  }
  return out;
}

// The fp16 V slice of DPL consecutive elements at voff + soff as raw 32-bit words (element e in the low
// (e even) or high (e odd) half of word e/2; a single element sits in the low half).  Past the split's
// valid range the words read as 0.  POL is the loads' cache policy.
template <int DPL, int POL = 0>
__device__ __forceinline__ void load_vwords_f16(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                uint32_t (&w)[DPL < 2 ? 1 : DPL / 2]) {
  if constexpr (DPL == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, POL);
  } else if constexpr (DPL == 2) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POL);
  } else if constexpr (DPL == 4) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POL);
    w[0] = x[0]; w[1] = x[1];
  } else {
    static_assert(DPL % 8 == 0, "V slice is a multiple of 16 bytes");
#pragma unroll
    for (int k = 0; k < DPL / 8; ++k) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16 * k, POL);
      w[4 * k + 0] = x[0]; w[4 * k + 1] = x[1]; w[4 * k + 2] = x[2]; w[4 * k + 3] = x[3];
    }
  }
}

// Element j of four fp16 slices (rows 0..3) packed as the four halves of an MFMA operand.
template <int VW>
__device__ __forceinline__ half4_t gather_col_f16(const uint32_t (&r0)[VW], const uint32_t (&r1)[VW],
                                                  const uint32_t (&r2)[VW], const uint32_t (&r3)[VW], int j) {
  const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of the two sources
  const int k = j >> 1;
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  const u2 x = u2{__builtin_amdgcn_perm(r1[k], r0[k], sel), __builtin_amdgcn_perm(r3[k], r2[k], sel)};
  return __builtin_bit_cast(half4_t, x);
}

// ---- split merge across the workgroups of one (b, kv head, head group)
//
// Each split's workgroup counts itself in on an arrival counter once its own loop and wave merge are done;
// the last one to arrive merges every split (log-sum-exp) and puts the counter back to zero.  Since every
// other workgroup has arrived by then, and publishes its partials without waiting for anything, the merger
// may simply read each partial until it is there.  The partials are 32-bit device-scope atomic words
// (relaxed: each word carries its own value, so no fence and no cache maintenance is needed; device-scope
// accesses reach the coherence point shared by all XCDs).  A word is the value's bits with the sign bit
// flipped and a negative zero stored as +0, so a written word is never 0: the workspace starts zeroed, a
// zero word is an empty slot, and the merger clears every slot it has read, leaving the workspace zeroed for
// the next call.  Record of split s of query-head row r: words [D sums, max, total, pad] at
// ws + (r * n_splits + s) * (D + kRecPad).

__device__ __forceinline__ uint32_t enc_word(float x) {
  uint32_t b = __builtin_bit_cast(uint32_t, x);
  if (b == 0x80000000u) b = 0u;
  return b ^ 0x80000000u;
}
__device__ __forceinline__ float dec_word(uint32_t w) { return __builtin_bit_cast(float, w ^ 0x80000000u); }
__device__ __forceinline__ void st_word(uint32_t* p, uint32_t w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_word(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// a word that is still 0 has not landed yet; its writer has arrived, so it will
__device__ __forceinline__ uint32_t await_word(const uint32_t* p, uint32_t w) {
  while (w == 0u) {
    __builtin_amdgcn_s_sleep(2);
    w = ld_word(p);
  }
  return w;
}

// Counts this workgroup in (one device-scope fetch-add, no retry loop) and returns the count before it.  The
// caller requests it before the wave merge and reads it after (merger_from_count), so the round trip runs
// under that merge.
__device__ __forceinline__ unsigned count_arrival(unsigned* c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Whether the workgroup whose arrival found `before` others is the last of the n_splits, which then merges
// them; the last one resets the counter for the next call.
__device__ __forceinline__ bool merger_from_count(unsigned* c, unsigned before, int n_splits) {
  const bool last = before + 1u == (unsigned)n_splits;
  if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// Element dc of this split's partials (and, for dc == 0, the head's running maximum and total).
template <int D>
__device__ __forceinline__ void publish_partial(uint32_t* rec, int dc, float num, float M, float den) {
  st_word(rec + dc, enc_word(num));
  if (dc == 0) {
    st_word(rec + D, enc_word(M));
    st_word(rec + D + 1, enc_word(den));
  }
}

// The merger's log-sum-exp of element dc over every split of one query-head row, folded in split order (so
// the result does not depend on which workgroup merges): its own split `own` from (M, num, den), the others
// from their records at base, loads of kMergeTile splits issued together.  Returns the merged maximum, sum
// and total in M, num, den.
template <int D>
__device__ __forceinline__ void merge_partials(const uint32_t* base, int n_splits, int own, int dc, float& M,
                                               float& num, float& den) {
  const float own_m = M, own_n = num, own_d = den;
  M = -INFINITY;
  num = den = 0.0f;
  for (int s0 = 0; s0 < n_splits; s0 += kMergeTile) {
    uint32_t mw[kMergeTile], dw[kMergeTile], nw[kMergeTile];
#pragma unroll
    for (int k = 0; k < kMergeTile; ++k) {
      mw[k] = dw[k] = nw[k] = 1u;
      if (s0 + k < n_splits && s0 + k != own) {
        const uint32_t* rec = base + (size_t)(s0 + k) * (D + kRecPad);
        mw[k] = ld_word(rec + D);
        dw[k] = ld_word(rec + D + 1);
        nw[k] = ld_word(rec + dc);
      }
    }
    float mv[kMergeTile], dv[kMergeTile], nv[kMergeTile];
#pragma unroll
    for (int k = 0; k < kMergeTile; ++k) {
      mv[k] = -INFINITY;
      dv[k] = nv[k] = 0.0f;
      if (s0 + k == own) {
        mv[k] = own_m;
        dv[k] = own_d;
        nv[k] = own_n;
      } else if (s0 + k < n_splits) {
        const uint32_t* rec = base + (size_t)(s0 + k) * (D + kRecPad);
        mv[k] = dec_word(await_word(rec + D, mw[k]));
        dv[k] = dec_word(await_word(rec + D + 1, dw[k]));
        nv[k] = dec_word(await_word(rec + dc, nw[k]));
      }
    }
    float Mt = M;
#pragma unroll
    for (int k = 0; k < kMergeTile; ++k) Mt = fmaxf(Mt, mv[k]);
    if (Mt == -INFINITY) continue;
    const float f = M == -INFINITY ? 0.0f : fast_exp2(M - Mt);
    num *= f;
    den *= f;
#pragma unroll
    for (int k = 0; k < kMergeTile; ++k) {
      const float wt = mv[k] == -INFINITY ? 0.0f : fast_exp2(mv[k] - Mt);
      num += wt * nv[k];
      den += wt * dv[k];
    }
    M = Mt;
  }
}

// Clears the words of element dc (and, for dc == 0, the maximum and total) of every split but `own`, whose
// record the merger never wrote.  Called once every thread of the merger has read its words.
template <int D>
__device__ __forceinline__ void clear_partials(uint32_t* base, int n_splits, int own, int dc) {
  for (int s2 = 0; s2 < n_splits; ++s2) {
    if (s2 == own) continue;
    uint32_t* rec = base + (size_t)s2 * (D + kRecPad);
    st_word(rec + dc, 0u);
    if (dc == 0) {
      st_word(rec + D, 0u);
      st_word(rec + D + 1, 0u);
    }
  }
}

// Per-wave progress counters in LDS, read and written with workgroup-scope relaxed atomics.  They must stay
// LDS accesses: a volatile access through a generic pointer compiles to a flat access, whose completion wait
// also waits for every outstanding global load of the wave (the prefetched chunk included).
struct WaveProgress {
  int* p;
  __device__ int get(int w) const { return __hip_atomic_load(p + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
  __device__ void set(int w, int v) const { __hip_atomic_store(p + w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
};

// NWV waves per workgroup: 8 (two per SIMD), or 12 (three per SIMD, for d = 64 with fp16 V and long splits:
// the third wave hides more latency, paid for with a shallower gather pipeline and V requested when its
// chunk starts rather than one chunk ahead, to fit 168 registers).
template <class S, int GG, bool VF16, int NWV = 8>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(NWV == 8 ? 1 : NWV / 4, NWV / 4)))
void decode_kernel(const AttnParams p) {
  constexpr int D = S::D;
  constexpr int DPL = D / 16;  // V columns per lane per MFMA tile set
  constexpr int NT = 64 * NWV;
  constexpr int kPol = S::kLoadPolicy;
  using Plan = LdsPlan<S, GG, NWV>;
  constexpr int HW = Plan::HW;
  using PT = typename std::conditional<VF16, _Float16, float>::type;
  typedef PT vrow_t __attribute__((ext_vector_type(DPL < 2 ? 2 : DPL)));
  __shared__ __align__(16) unsigned char smem[Plan::total(VF16)];
  float* lv = reinterpret_cast<float*>(smem + Plan::consts_off);
  int* s_flag = reinterpret_cast<int*>(smem + Plan::consts_off + 96);
  const WaveProgress s_prog{reinterpret_cast<int*>(smem + Plan::consts_off + 128)};  // [NWV] chunks done
  uint32_t* s_newc = reinterpret_cast<uint32_t*>(smem + Plan::newcode_off);
  float* s_newn = reinterpret_cast<float*>(smem + Plan::newnorm_off);
  int* s_newready = reinterpret_cast<int*>(smem + Plan::newnorm_off + 4);
  static_assert(S::NW * 4 <= 128, "appended key's codes fit their LDS slot");
  float* qs = reinterpret_cast<float*>(smem + Plan::qs_off);
  float* qa = reinterpret_cast<float*>(smem + Plan::qa_off);
  PT* pst = reinterpret_cast<PT*>(smem + Plan::pst_off);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kq = lane >> 4;
  const Unit u = decode_unit(p, GG);
  const int split = blockIdx.x;
  const int64_t t_begin = (int64_t)split * p.split_len;
  int64_t t_end = t_begin + p.split_len;
  if (t_end > u.len) t_end = u.len;
  const int n_valid = t_end > t_begin ? (int)(t_end - t_begin) : 0;  // keys of this split
  const int64_t rowb = ((int64_t)u.b * p.Hkv + u.kvh) * p.T_cap + t_begin;  // first cache row of the split
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.codes + (size_t)rowb * S::BPK, (int64_t)n_valid * S::BPK);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(S::kNorm ? (const void*)(p.norms + rowb) : (const void*)p.codes,
                                              S::kNorm ? (int64_t)n_valid * 4 : 0);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(reinterpret_cast<const PT*>(p.v) + (size_t)rowb * D, (int64_t)n_valid * D * (int)sizeof(PT));
  // per-lane byte offsets (fixed for the whole loop); the chunk position goes in the scalar offset
  const int voff_code = lane * S::BPK;
  const int voff_v = VF16 ? ((4 * kq) * D + DPL * r16) * (int)sizeof(PT) : (kq * D + DPL * r16) * (int)sizeof(PT);

  // Loads run one chunk (of this wave) ahead of the arithmetic: the codes and norms of the next chunk,
  // and for d <= 64 its fp16 V slices, are requested before the current one is scored.  Two register sets
  // alternate (the loop is unrolled by two), so nothing is copied between iterations and the wait for a
  // chunk's data leaves the next chunk's requests in flight.  For d = 128 two chunks of V do not fit the
  // register budget: a chunk's V is requested when the chunk starts and arrives behind its table
  // gathers; for d = 256 four slices at a time are loaded just before their matrix products.  The first
  // chunk's loads are requested before the prologue so they arrive while the table is built.  Loads past
  // the split's end read as zeros, so the fetches need no guard (a guard would also make the compiler
  // wait for every outstanding load wherever it cannot count them).
  constexpr int STR = NWV * kChunk;  // distance between a wave's consecutive chunks
  constexpr int VW = DPL < 2 ? 1 : DPL / 2;  // 32-bit words per fp16 V slice
  constexpr bool kVPre = VF16 && VW <= 2 && NWV == 8;
  constexpr bool kVChunk = VF16 && (VW == 4 || (NWV > 8 && VW <= 4));
  struct Chunk {
    uint32_t w[S::NW];
    float nrm;
    uint32_t v[4][4][kVPre ? VW : 1];  // fp16 V slices as raw words, when prefetched
  };
  auto load_v = [&](int cc, int ks, uint32_t (&vb)[4][VW]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) load_vwords_f16<DPL, kPol>(rv, voff_v, (cc + 16 * ks + s) * D * (int)sizeof(PT), vb[s]);
  };
  auto fetch_codes = [&](int cc, Chunk& k) {
    load_code_row_buf<S::BPK, kPol>(rc, voff_code, cc * S::BPK, k.w);
    k.nrm = 1.0f;
    if constexpr (S::kNorm) k.nrm = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rn, lane * 4, cc * 4, kPol));
  };
  auto fetch_v = [&](int cc, Chunk& k) {
    if constexpr (kVPre) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) load_v(cc, ks, k.v[ks]);
    }
  };
  auto fetch = [&](int cc, Chunk& k) {
    fetch_codes(cc, k);
    fetch_v(cc, k);
  };
  int c = wid * kChunk;  // chunk start, relative to t_begin
  Chunk ka, kb;

  // Fused append (the scalar codecs): the workgroup whose split holds the sequence's last position
  // encodes the new key itself -- its last wave, which has the fewest chunks of the split, D/16 lanes, with
  // the arithmetic of the encode kernel, after the table is built (so the encode holds up no other wave) --
  // keeps its codes and norm in LDS for the wave that scores that position, and (head group 0 only) writes
  // them to the cache.
  constexpr int LPK = EncLanes<D>::LPK;
  constexpr int kEncWave = NWV - 1;
  const bool app = S::kIntLut && p.new_keys != nullptr && n_valid > 0 && u.len <= t_begin + p.split_len;
  const int rel = n_valid - 1;  // the new key's position within the split, when app
  const bool enc_lanes = app && wid == kEncWave && lane < LPK;
  const int64_t new_row = (int64_t)u.b * p.Hkv + u.kvh;
  const int kesz = p.new_f16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(app ? (const void*)(reinterpret_cast<const char*>(p.new_keys) + new_row * D * kesz) : p.codes,
                app && wid == kEncWave ? D * kesz : 0);

  // the lane's 16 coordinates of the new key (fp16 in the first 8 words): four 16-byte loads for fp32, two
  // for fp16 (the rest read zeros), nonzero in the encoding lanes only; requested first, so that they have
  // arrived when the encoding wave gets to them after the table is built
  uint32_t kraw[kEncCpl];
  if constexpr (S::kIntLut) {
    if (app && wid == kEncWave) {
      const int ko = lane * kEncCpl * kesz;
#pragma unroll
      for (int h = 0; h < kEncCpl / 4; ++h) {
        const auto r = __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 16 * h, 0, kPol);
#pragma unroll
        for (int j = 0; j < 4; ++j) kraw[4 * h + j] = r[j];
      }
    }
  }
  // What the table build can request before the queries arrive (the PQ centroids), then the first chunk's
  // codes, norms and V, so that this first burst streams in while the queries are rotated and the table is
  // built.
  const auto pre = S::template prefetch<GG, HW, NT>(p, u.kvh, tid);
  if (lane == 0) s_prog.set(wid, 0);
  if (tid == 0) *s_newready = 0;
  prologue<S, GG, NT, true>(p, u, qs, qa, lv, tid, [&] {
    fetch_codes(c, ka);
    fetch_v(c, ka);
  }, smem);
  if constexpr (!direct_table<S, GG, NT>()) {
    S::template build<GG, HW, NT>(p, qs, qa, lv, reinterpret_cast<float*>(smem), u.kvh, tid, pre);
    lds_barrier();
  }
  if constexpr (S::kIntLut) {
    if (app && wid == kEncWave) {
      // Hadamard codes: the key's D/16 lanes rotate and scale it as the encode kernel does, then the whole wave
      // counts thresholds (each lane one coordinate per 64) instead of 16 coordinates' comparisons with every
      // threshold on D/16 lanes; same comparisons, same codes.  Codes of 1, 2 or 4 bits in rows of whole
      // words are packed with lane exchanges, the others by the key's lanes.  Keys with a non-finite sum of
      // squares take the write path's own route below.
      constexpr int CB = S::CODE_BITS;
      bool fast = false;
      constexpr bool kWords = (CB == 1 || CB == 2 || CB == 4) && (D * CB) % 32 == 0;  // rows of whole words
      if constexpr (S::kRotate) {
        float x[kEncCpl];
        float nrm = 0.0f;
        bool fin = false;
        if (enc_lanes) {
          if (p.new_f16) key_lane_floats<true>(kraw, x);
          else key_lane_floats<false>(kraw, x);
          float sg[kEncCpl];
          lane_signs<D>(p.signs, lane, sg);
          const float ss = rotate_key_lane<D>(x, lane, sg);
          const float inv = unit_scale_ss<D>(ss, nrm);
          fin = ss <= 0x1.fffffep127f;
          if (fin) unit_vector(x, inv);
        }
        fast = __builtin_amdgcn_readfirstlane(fin ? 1 : 0) != 0;  // lane 0 holds the key
        if (fast) {
          float* ys = qs;  // the queries' staging area is free once the table is built: D floats
          if (enc_lanes) {
#pragma unroll
            for (int h = 0; h < kEncCpl / 4; ++h)
              *reinterpret_cast<float4*>(ys + kEncCpl * lane + 4 * h) = make_float4(x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]);
          }
          wave_lds_sync();
          const bool row_writer = blockIdx.y % p.n_groups == 0;  // one cache writer per (b, kv head)
          const int64_t row = new_row * p.T_cap + (u.len - 1);
          if constexpr (!kWords) {
            // other rows: the codes go back to the key's lanes as bytes over the coordinates just read, and
            // are packed there as in the write path
            constexpr int NCI = (D + 63) / 64;
            uint32_t cv[NCI];
#pragma unroll
            for (int k = 0; k < NCI; ++k) {
              const int i = 64 * k + lane;
              cv[k] = i < D ? code_by_count<CB>(ys[i], p.thresholds) : 0u;
            }
            wave_lds_sync();  // every lane has read its coordinates before the bytes overwrite them
            uint8_t* cb8 = reinterpret_cast<uint8_t*>(ys);
#pragma unroll
            for (int k = 0; k < NCI; ++k)
              if (64 * k + lane < D) cb8[64 * k + lane] = (uint8_t)cv[k];
            wave_lds_sync();
            if (enc_lanes) {
              const uint4 q4 = *reinterpret_cast<const uint4*>(cb8 + kEncCpl * lane);
              const uint32_t wd[4] = {q4.x, q4.y, q4.z, q4.w};
              uint64_t packed = 0;
#pragma unroll
              for (int j = 0; j < kEncCpl; ++j) packed |= (uint64_t)((wd[j / 4] >> (8 * (j % 4))) & 0xffu) << (CB * j);
              store_code_bits<CB>(reinterpret_cast<uint8_t*>(s_newc), lane, packed);
              if (row_writer) store_code_bits<CB>(p.app_codes + row * S::BPK, lane, packed);
            }
          }
#pragma unroll
          for (int k0 = 0; k0 < (kWords ? D : 0); k0 += 64) {
            const int i = k0 + lane;
            constexpr int CPW = 32 / CB;  // coordinates per 32-bit word of the code row
            uint32_t w = 0;
            if (i < D) w = code_by_count<CB>(ys[i], p.thresholds);
            // CPW consecutive coordinates' codes into one word, LSB first, in lane CPW m of each group
            auto merge = [&](auto dl_tag) {
              constexpr int DL = decltype(dl_tag)::value;
              if constexpr (DL < CPW) w |= __builtin_bit_cast(uint32_t, xor_lane<DL>(__builtin_bit_cast(float, w))) << (CB * DL);
            };
            merge(std::integral_constant<int, 1>{});
            merge(std::integral_constant<int, 2>{});
            merge(std::integral_constant<int, 4>{});
            merge(std::integral_constant<int, 8>{});
            merge(std::integral_constant<int, 16>{});
            if (i < D && (lane & (CPW - 1)) == 0) {
              s_newc[i / CPW] = w;
              if (row_writer) reinterpret_cast<uint32_t*>(p.app_codes + row * S::BPK)[i / CPW] = w;
            }
          }
          if (lane == 0) {
            *s_newn = nrm;
            if (row_writer) p.app_norms[row] = nrm;
          }
        }
      }
      if (enc_lanes && !fast) {
        float nrm;  // the key's norm (Hadamard codec) or max |k_i| (power-of-two codec)
        uint64_t packed;
        if constexpr (S::kRotate) {
          packed = encode_key_lane<D, S::CODE_BITS>(kraw, p.new_f16 != 0, lane, p.signs, p.thresholds, nrm);
        } else {
          float x[kEncCpl];
          if (p.new_f16) key_lane_floats<true>(kraw, x);
          else key_lane_floats<false>(kraw, x);
          packed = p.pot_mant ? pot_encode_lane<D, S::CODE_BITS, true>(x, p.thresholds, nrm)
                             : pot_encode_lane<D, S::CODE_BITS, false>(x, p.thresholds, nrm);
        }
        store_code_bits<S::CODE_BITS>(reinterpret_cast<uint8_t*>(s_newc), lane, packed);
        if (lane == 0) *s_newn = nrm;
        if (blockIdx.y % p.n_groups == 0) {  // one writer per (b, kv head)
          const int64_t row = new_row * p.T_cap + (u.len - 1);
          store_code_bits<S::CODE_BITS>(p.app_codes + row * S::BPK, lane, packed);
          if (lane == 0) p.app_norms[row] = nrm;
        }
      }
      // publish the codes and norm in LDS to the wave that scores the new position
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0) __hip_atomic_store(s_newready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  // softmax argument of head g per unit of table sum and of key norm: scale * log2(e) (* 2^-e_g)
  float hz[GG];
#pragma unroll
  for (int g = 0; g < GG; ++g) {
    hz[g] = p.zscale;
    if constexpr (S::kIntLut) hz[g] *= pow2f(-fix_exp(qa[g], S::level_max(lv)));
  }

  float m_run[GG], l_lane[GG];
#pragma unroll
  for (int g = 0; g < GG; ++g) {
    m_run[g] = -INFINITY;
    l_lane[g] = 0.0f;
  }
  float4_t oacc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) oacc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
  constexpr int PST = Plan::pst_row(VF16);
  PT* pw = pst + wid * GG * PST;
  int done = 0;  // chunks this wave has processed

  // score one chunk (keys cc .. cc+63 of the split) and fold it into the softmax state and the output
  auto process = [&](int cc, Chunk& k) {
    if (app && cc <= rel && rel < cc + kChunk) {  // the appended key: codes and norm from LDS
      // written by the encoding wave right after the table barrier; it waits for nothing, so this ends
      while (__hip_atomic_load(s_newready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
        __builtin_amdgcn_s_sleep(1);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      if (lane == rel - cc) {
#pragma unroll
        for (int kk = 0; kk < S::NW; ++kk) k.w[kk] = s_newc[kk];
        k.nrm = *s_newn;
      }
    }
    uint32_t vc[kVChunk ? 4 : 1][4][VW];  // d = 128: this chunk's V, requested before the gathers
    if constexpr (kVChunk) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) load_v(cc, ks, vc[ks]);
    }
    // ---- scores from the table
    ScoreAcc<S> acc[GG];
    lut_scores<S, GG, NWV == 8 ? 4 : 2>(smem, k.w, acc);
    float z[GG];
#pragma unroll
    for (int g = 0; g < GG; ++g) {
      if constexpr (S::kIntLut) z[g] = (float)(int)acc[g] * (k.nrm * hz[g]);
      else z[g] = acc[g] * (S::kNorm ? k.nrm * hz[g] : hz[g]);
    }
    if (cc + kChunk > n_valid) {  // the split's last, partial chunk
      const bool valid = cc + lane < n_valid;
#pragma unroll
      for (int g = 0; g < GG; ++g) z[g] = valid ? z[g] : -INFINITY;
    }
    // ---- online softmax: raise the running maximum only when some score exceeds it by the headroom
    float rise = z[0] - m_run[0];
#pragma unroll
    for (int g = 1; g < GG; ++g) rise = fmaxf(rise, z[g] - m_run[g]);
    if (__any(rise > kLazyHeadroom)) {
      float my_alpha = 1.0f;
#pragma unroll
      for (int g = 0; g < GG; ++g) {
        const float mn = fmaxf(m_run[g], wave_max(z[g]));
        const float alpha = fast_exp2(m_run[g] - mn);
        m_run[g] = mn;
        l_lane[g] *= alpha;
        if (r16 == g) my_alpha = alpha;
      }
#pragma unroll
      for (int j = 0; j < DPL; ++j) oacc[j] *= my_alpha;
    }
#pragma unroll
    for (int g = 0; g < GG; ++g) {
      const float pr = fast_exp2(z[g] - m_run[g]);
      l_lane[g] += pr;
      pw[g * PST + lane] = (PT)pr;
    }
    wave_lds_sync();

    // ---- out^T += V^T P^T on the matrix cores
    if constexpr (VF16) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half4_t bop = half4_t{0, 0, 0, 0};
        if (r16 < GG) bop = *reinterpret_cast<const half4_t*>(pw + r16 * PST + 16 * ks + 4 * kq);
        uint32_t vl[kVPre || kVChunk ? 1 : 4][VW];  // d = 256: four slices loaded here
        if constexpr (!kVPre && !kVChunk) load_v(cc, ks, vl);
        const auto& vb = [&]() -> const uint32_t(&)[4][VW] {
          if constexpr (kVPre) return k.v[ks];
          else if constexpr (kVChunk) return vc[ks];
          else return vl;
        }();
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          const half4_t a = gather_col_f16<VW>(vb[0], vb[1], vb[2], vb[3], j);
          oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bop, oacc[j], 0, 0, 0);
        }
      }
    } else {
#pragma unroll 4
      for (int ks = 0; ks < 16; ++ks) {
        const vrow_t a = load_vrow_buf<PT, DPL, vrow_t, kPol>(rv, voff_v, (cc + 4 * ks) * D * (int)sizeof(PT));
        float bop = 0.0f;
        if (r16 < GG) bop = pw[r16 * PST + 4 * ks + kq];
#pragma unroll
        for (int j = 0; j < DPL; ++j) oacc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], bop, oacc[j], 0, 0, 0);
      }
    }
    wave_lds_sync();

    // ---- keep the waves that share a SIMD (wid, wid + 4, ...) level: the instruction arbiter favours the
    // older wave, which would otherwise finish well before its partners and leave the SIMD partly idle for
    // the rest of the split.  A wave that is ahead of the slowest of its partners drops its priority.
    ++done;
    if (lane == 0) s_prog.set(wid, done);
    int other = __builtin_amdgcn_readfirstlane(s_prog.get((wid + 4) % NWV));
#pragma unroll
    for (int k = 2; k < NWV / 4; ++k) {
      const int o = __builtin_amdgcn_readfirstlane(s_prog.get((wid + 4 * k) % NWV));
      other = o < other ? o : other;
    }
    if (done > other) __builtin_amdgcn_s_setprio(0);
    else __builtin_amdgcn_s_setprio(1);
  };

  for (; c < n_valid; c += 2 * STR) {
    fetch(c + STR, kb);
    process(c, ka);
    if (c + STR >= n_valid) break;
    fetch(c + 2 * STR, ka);
    process(c + STR, kb);
  }

  // ---- merge the waves' records (max, total, sums) through LDS
  float l_w[GG];
#pragma unroll
  for (int g = 0; g < GG; ++g) l_w[g] = wave_sum(l_lane[g]);
  __builtin_amdgcn_s_setprio(0);
  constexpr int RS = Plan::RS;
  float* red = reinterpret_cast<float*>(smem + Plan::red_off);  // [NWV][GG][RS]
  float* red_m = red + NWV * GG * RS;                           // [NWV][GG]
  float* red_l = red_m + NWV * GG;                              // [NWV][GG]
  float* mine = red_l + NWV * GG;                               // [GG][D] the workgroup's merged sums
  float* mine_m = mine + GG * D;                                // [GG]
  float* mine_d = mine_m + GG;                                  // [GG]
  if constexpr (!Plan::kRedSeparate) lds_barrier();  // the records overwrite the table
  if (r16 < GG) {
    // the lane's 4 DPL sums are dims DPL (4 kq + r) + j: one contiguous run, written as 16-byte vectors
    float* dst = red + (wid * GG + r16) * RS + DPL * 4 * kq;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (DPL % 4 == 0) {
#pragma unroll
        for (int j0 = 0; j0 < DPL; j0 += 4)
          *reinterpret_cast<float4*>(dst + DPL * r + j0) =
              make_float4(oacc[j0][r], oacc[j0 + 1][r], oacc[j0 + 2][r], oacc[j0 + 3][r]);
      } else {
#pragma unroll
        for (int j = 0; j < DPL; ++j) dst[DPL * r + j] = oacc[j][r];
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GG; ++g)
    if (lane == g) {
      red_m[wid * GG + g] = m_run[g];
      red_l[wid * GG + g] = l_w[g];
    }
  lds_barrier();
  const bool split_merge = p.n_splits > 1;
  unsigned arrived = 0u;  // the arrival count, requested here and read after the wave merge
  if (split_merge && tid == NT - 1) arrived = count_arrival(p.counters + blockIdx.y);
  for (int idx = tid; idx < GG * D; idx += NT) {
    const int g = idx / D, dc = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NWV; ++w2) M = fmaxf(M, red_m[w2 * GG + g]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < NWV; ++w2) {
        const float wt = fast_exp2(red_m[w2 * GG + g] - M);
        num += wt * red[(w2 * GG + g) * RS + dc];
        den += wt * red_l[w2 * GG + g];
      }
    }
    if (!split_merge) {
      const size_t row = (size_t)u.b * p.Hq + u.h0 + g;
      const float o = den > 0.0f ? num / den : 0.0f;
      if (p.out_f16) reinterpret_cast<_Float16*>(p.out)[row * D + dc] = (_Float16)o;
      else reinterpret_cast<float*>(p.out)[row * D + dc] = o;
    } else {
      mine[idx] = num;
      if (dc == 0) {
        mine_m[g] = M;
        mine_d[g] = den;
      }
    }
  }
  if (!split_merge) return;

  // ---- split merge: every workgroup but the last publishes its partials; the last merges all splits
  if (tid == NT - 1) *s_flag = merger_from_count(p.counters + blockIdx.y, arrived, p.n_splits);
  lds_barrier();
  const bool last = *s_flag;
  uint32_t* wsw = reinterpret_cast<uint32_t*>(p.ws);
  for (int idx = tid; idx < GG * D; idx += NT) {
    const int g = idx / D, dc = idx % D;
    const size_t row = (size_t)u.b * p.Hq + u.h0 + g;
    uint32_t* base = wsw + row * (size_t)p.n_splits * (D + kRecPad);
    float M = mine_m[g], num = mine[idx], den = mine_d[g];
    if (!last) {
      publish_partial<D>(base + (size_t)split * (D + kRecPad), dc, num, M, den);
      continue;
    }
    merge_partials<D>(base, p.n_splits, split, dc, M, num, den);
    const float o = den > 0.0f ? num / den : 0.0f;
    if (p.out_f16) reinterpret_cast<_Float16*>(p.out)[row * D + dc] = (_Float16)o;
    else reinterpret_cast<float*>(p.out)[row * D + dc] = o;
  }
  if (!last) return;
  __syncthreads();  // every thread of the merger has read its words
  for (int idx = tid; idx < GG * D; idx += NT) {
    const int g = idx / D, dc = idx % D;
    const size_t row = (size_t)u.b * p.Hq + u.h0 + g;
    clear_partials<D>(wsw + row * (size_t)p.n_splits * (D + kRecPad), p.n_splits, split, dc);
  }
}

template <class S, int GG, int NWV = kWaves>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(NWV <= 8 ? 1 : NWV / 4, NWV <= 8 ? 2 : NWV / 4)))
void score_kernel(const AttnParams p) {
  constexpr int NT = 64 * NWV;
  using Plan = LdsPlan<S, GG, NWV, false>;
  constexpr int HW = Plan::HW;
  __shared__ __align__(16) unsigned char smem[Plan::pst_off];
  float* lv = reinterpret_cast<float*>(smem + Plan::consts_off);
  float* qs = reinterpret_cast<float*>(smem + Plan::qs_off);
  float* qa = reinterpret_cast<float*>(smem + Plan::qa_off);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Unit u = decode_unit(p, GG);
  const int64_t t_begin = (int64_t)blockIdx.x * p.split_len;
  int64_t t_stop = t_begin + p.split_len;
  if (t_stop > p.T_cap) t_stop = p.T_cap;
  const int64_t t_valid = t_stop < u.len ? t_stop : u.len;  // codes are read only below this
  const int n_stop = (int)(t_stop - t_begin);
  const int n_valid = t_valid > t_begin ? (int)(t_valid - t_begin) : 0;
  const int64_t rowb = ((int64_t)u.b * p.Hkv + u.kvh) * p.T_cap + t_begin;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.codes + (size_t)rowb * S::BPK, (int64_t)n_valid * S::BPK);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(S::kNorm ? (const void*)(p.norms + rowb) : (const void*)p.codes,
                                              S::kNorm ? (int64_t)n_valid * 4 : 0);

  // codes and norms one chunk (of this wave) ahead, in two alternating register sets (as in decode_kernel)
  constexpr int STR = NWV * kChunk;
  uint32_t wa[S::NW], wb[S::NW];
  float na = 1.0f, nb = 1.0f;
  auto fetch = [&](int cc, uint32_t (&w)[S::NW], float& n) {
    load_code_row_buf<S::BPK>(rc, lane * S::BPK, cc * S::BPK, w);
    if constexpr (S::kNorm) n = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rn, lane * 4, cc * 4, 0));
  };
  // the unit's GG score rows through a buffer resource: 32-bit offsets, head row in the scalar offset,
  // and stores at or past T_cap are dropped by the bounds check
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.scores + ((size_t)u.b * p.Hq + u.h0) * p.T_cap,
                                              (int64_t)GG * p.T_cap * 4);
  float hs[GG];  // score per unit of table sum: 2^-e_g for fixed-point tables
  auto score = [&](int cc, const uint32_t (&w)[S::NW], float n) {
    ScoreAcc<S> acc[GG];
    lut_scores<S, GG>(smem, w, acc);
    const int t = cc + lane;
    const bool valid = t < n_valid;
    // past the split: an offset beyond the resource (2^30 > GG*T_cap*4, which the host checks), so dropped
    const int voff = t < n_stop ? (int)(t_begin + t) * 4 : 0x40000000;
#pragma unroll
    for (int g = 0; g < GG; ++g) {
      const float sc = S::kIntLut ? n * ((float)(int)acc[g] * hs[g]) : (S::kNorm ? n * acc[g] : acc[g]);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, valid ? sc : -INFINITY), rs, voff,
                                            g * p.T_cap * 4, 0);
    }
  };
  int c = wid * kChunk;
  const auto pre = S::template prefetch<GG, HW, NT>(p, u.kvh, tid);
  prologue<S, GG, NT, true>(p, u, qs, qa, lv, tid, [&] { fetch(c, wa, na); }, smem);
  if constexpr (!direct_table<S, GG, NT>()) {
    S::template build<GG, HW, NT>(p, qs, qa, lv, reinterpret_cast<float*>(smem), u.kvh, tid, pre);
    lds_barrier();
  }
#pragma unroll
  for (int g = 0; g < GG; ++g)
    hs[g] = S::kIntLut ? pow2f(-fix_exp(qa[g], S::level_max(lv))) : 1.0f;

  for (; c < n_stop; c += 2 * STR) {
    fetch(c + STR, wb, nb);
    score(c, wa, na);
    if (c + STR >= n_stop) break;
    fetch(c + 2 * STR, wa, na);
    score(c + STR, wb, nb);
  }
}

// The kernels' LDS is static (sized per instantiation), so nothing is requested at launch.
template <class Kern>
hipError_t launch_attn(Kern kernel, size_t lds, dim3 grid, hipStream_t s, const AttnParams& p, int threads = kThreads) {
  if (lds > 160 * 1024) return hipErrorNotSupported;
  hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, p);
  return hipGetLastError();
}

// p.waves selects the workgroup size: 12 waves are built for d = 64 with fp16 V and the scalar codecs only.
template <class S, int GG>
hipError_t run_decode_gg(bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  if (p.waves == 12) {
    if constexpr (S::D == 64 && S::kIntLut) {
      if (!v_f16) return hipErrorNotSupported;
      return launch_attn(decode_kernel<S, GG, true, 12>, LdsPlan<S, GG, 12>::total(true), grid, s, p, 12 * 64);
    }
    return hipErrorNotSupported;
  }
  using Plan = LdsPlan<S, GG>;
  if (v_f16) return launch_attn(decode_kernel<S, GG, true>, Plan::total(true), grid, s, p);
  return launch_attn(decode_kernel<S, GG, false>, Plan::total(false), grid, s, p);
}

template <class S>
hipError_t run_decode(int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (gg) {
    case 1: return run_decode_gg<S, 1>(v_f16, p, grid, s);
    case 2: return run_decode_gg<S, 2>(v_f16, p, grid, s);
    case 4: return run_decode_gg<S, 4>(v_f16, p, grid, s);
    case 8: return run_decode_gg<S, 8>(v_f16, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

template <class S>
hipError_t run_score(int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (gg) {
    case 1: return launch_attn(score_kernel<S, 1>, LdsPlan<S, 1, kWaves, false>::pst_off, grid, s, p);
    case 2: return launch_attn(score_kernel<S, 2>, LdsPlan<S, 2, kWaves, false>::pst_off, grid, s, p);
    case 4: return launch_attn(score_kernel<S, 4>, LdsPlan<S, 4, kWaves, false>::pst_off, grid, s, p);
    case 8: return launch_attn(score_kernel<S, 8>, LdsPlan<S, 8, kWaves, false>::pst_off, grid, s, p);
    default: return hipErrorNotSupported;
  }
}

// Hadamard/Lloyd-Max dispatch for one head dimension (instantiated per D).
template <int D>
hipError_t run_hlm_decode(int bits, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (bits) {
    case 1: return run_decode<HlmScorer<D, 1>>(gg, v_f16, p, grid, s);
    case 2: return run_decode<HlmScorer<D, 2>>(gg, v_f16, p, grid, s);
    case 3: return run_decode<HlmScorer<D, 3>>(gg, v_f16, p, grid, s);
    case 4: return run_decode<HlmScorer<D, 4>>(gg, v_f16, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

template <int D>
hipError_t run_hlm_score(int bits, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (bits) {
    case 1: return run_score<HlmScorer<D, 1>>(gg, p, grid, s);
    case 2: return run_score<HlmScorer<D, 2>>(gg, p, grid, s);
    case 3: return run_score<HlmScorer<D, 3>>(gg, p, grid, s);
    case 4: return run_score<HlmScorer<D, 4>>(gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

// Power-of-two codec dispatch for one head dimension (instantiated per D): 2..4 bits per element.
template <int D>
hipError_t run_pot_decode(int bits, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (bits) {
    case 2: return run_decode<PotScorer<D, 2>>(gg, v_f16, p, grid, s);
    case 3: return run_decode<PotScorer<D, 3>>(gg, v_f16, p, grid, s);
    case 4: return run_decode<PotScorer<D, 4>>(gg, v_f16, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

template <int D>
hipError_t run_pot_score(int bits, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (bits) {
    case 2: return run_score<PotScorer<D, 2>>(gg, p, grid, s);
    case 3: return run_score<PotScorer<D, 3>>(gg, p, grid, s);
    case 4: return run_score<PotScorer<D, 4>>(gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace kvq
