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
// Work decomposition (one workgroup = 8 waves of 64 lanes):
//   workgroup <- (batch b, kv head, group of GG query heads, split of T);
//   prologue: the GG queries are loaded into LDS, sign-flipped and put
//   through an in-LDS fast Walsh-Hadamard transform (Hadamard codec), then
//   the table for all GG heads is written to LDS as [GG/HW][rows][cols] of
//   HW-wide float vectors (HW = min(GG, 4)), so one ds_read_b128 at
//   (row, code) returns the entries of four heads;
//   main loop: a wave takes 64 consecutive keys at a time, lane <-> key.
//   The next chunk's codes and norms are fetched while the current one is
//   scored, and the current chunk's V slices are fetched before its gathers.
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
//   the last of its workgroups to finish (log-sum-exp merge), found with an
//   arrival counter in the workspace that the last workgroup resets to zero.
#pragma once

#include <type_traits>

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

template <int B, int NW>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[NW], int i) {
  const int bit = i * B;
  const int word = bit >> 5;
  const int off = bit & 31;
  uint32_t x = w[word] >> off;
  if (off + B > 32) x |= w[word + 1 < NW ? word + 1 : NW - 1] << (32 - off);
  return x & ((1u << B) - 1u);
}

// Scorer for the Hadamard + Lloyd-Max codec: rows = coordinates, cols = levels.
template <int D_, int BITS>
struct HlmScorer {
  static constexpr int D = D_;
  static constexpr int ROWS = D;
  static constexpr int COLS = 1 << BITS;
  static constexpr int BPK = D * BITS / 8;
  static constexpr int NW = (BPK + 3) / 4;
  static constexpr bool kRotate = true;
  static constexpr bool kNorm = true;
  static constexpr bool kNibbles = BITS == 4;  // two codes per byte: byte-wise address extraction
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[NW], int i) { return code_at<BITS, NW>(w, i); }
  // LUT[g][i][j] = q'_{g,i} * c_j with q' = H D q / sqrt(d) held in qs; one HW-wide entry (HW heads) per
  // (head group, coordinate, level).
  template <int GG, int HW>
  __device__ static void build(const AttnParams&, const float* qs, const float* lv, float* lut, int, int tid) {
    using E = typename VecF<HW>::type;
    constexpr int total = (GG / HW) * ROWS * COLS;
    E* L = reinterpret_cast<E*>(lut);
    for (int e = tid; e < total; e += kThreads) {
      const int j = e % COLS;
      const int i = (e / COLS) % ROWS;
      const int g0 = (e / (COLS * ROWS)) * HW;
      const float c = lv[j];
      float v[4];
#pragma unroll
      for (int h = 0; h < HW; ++h) v[h] = qs[(g0 + h) * D + i] * c;
      if constexpr (HW == 4) L[e] = make_float4(v[0], v[1], v[2], v[3]);
      else if constexpr (HW == 2) L[e] = make_float2(v[0], v[1]);
      else L[e] = v[0];
    }
  }
};

// Scorer for product quantization: rows = subspaces, cols = centroids (<= 256).
template <int D_, int M>
struct PqScorer {
  static constexpr int D = D_;
  static constexpr int ROWS = M;
  static constexpr int COLS = 256;
  static constexpr int BPK = M;
  static constexpr int NW = (BPK + 3) / 4;
  static constexpr int DS = D / M;
  static constexpr bool kRotate = false;
  static constexpr bool kNorm = false;
  static constexpr bool kNibbles = false;
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[NW], int i) {
    return (w[i >> 2] >> (8 * (i & 3))) & 255u;
  }
  // LUT[g][s][c] = q_{g,s} . C_{s,c}; columns c >= K are zero (never selected).
  template <int GG, int HW>
  __device__ static void build(const AttnParams& p, const float* qs, const float*, float* lut, int kvh, int tid) {
    constexpr int total = GG * ROWS * COLS;
    const int K = p.pq_K;
    const float* cent = p.pq_cent + (size_t)kvh * M * K * DS;
    for (int idx = tid; idx < total; idx += kThreads) {
      const int hh = idx % HW;
      const int c = (idx / HW) % COLS;
      const int s = (idx / (HW * COLS)) % ROWS;
      const int g = (idx / (HW * COLS * ROWS)) * HW + hh;
      float acc = 0.0f;
      if (c < K) {
#pragma unroll
        for (int k = 0; k < DS; ++k) acc += qs[g * D + s * DS + k] * cent[((size_t)s * K + c) * DS + k];
      }
      lut[idx] = acc;
    }
  }
};

template <class S, int GG>
struct LdsPlan {
  static constexpr int HW = GG < 4 ? GG : 4;
  static constexpr int NQ = GG / HW;
  static constexpr size_t lut_bytes = (size_t)GG * S::ROWS * S::COLS * 4;
  static constexpr size_t red_bytes = (size_t)kWaves * GG * (S::D + 2) * 4;
  static constexpr size_t region0 = ((lut_bytes > red_bytes ? lut_bytes : red_bytes) + 15) / 16 * 16;
  static constexpr size_t consts_off = region0;                   // 16 levels, 8 sign words, flags
  static constexpr size_t qs_off = consts_off + 128;              // GG * D floats
  static constexpr size_t pst_off = qs_off + (size_t)GG * S::D * 4;
  static constexpr size_t pst_bytes(bool f16) { return (size_t)kWaves * GG * kChunk * (f16 ? 2 : 4); }
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

// Loads the GG queries into qs[g][i] (fp32) and copies the codebook levels into LDS.  For the Hadamard
// codec every query is also rotated, q' = H D q / sqrt(d): 8 consecutive coordinates per lane and d/8
// lanes per query, sign flip, then a radix-2 fast Walsh-Hadamard transform (Sylvester order) in registers
// (distances 1, 2, 4) and across the query's lanes (distances 8 .. d/2).
// `between` runs after this thread's query loads are issued and before they are used: the caller issues
// its first cache loads there, so they are in flight during the rotation and the table build (vector
// memory loads complete in order, so waiting for the query does not wait for them).
template <class S, int GG, class F>
__device__ void prologue(const AttnParams& p, const Unit& u, float* qs, float* lv, int tid, F&& between) {
  constexpr int D = S::D;
  if (tid < 16) lv[tid] = p.levels[tid];
  if constexpr (S::kRotate) {
    constexpr int LPQ = D / 8;  // lanes per query (a power of two <= 32, so groups never straddle waves)
    static_assert(GG * LPQ <= kThreads, "one lane per 8 coordinates of every query");
    const int g = tid / LPQ, k = tid % LPQ;
    const size_t off = ((size_t)u.b * p.Hq + u.h0 + (g < GG ? g : 0)) * D + 8 * k;
    const uint32_t sb = (p.signs[(8 * k) >> 5] >> ((8 * k) & 31)) & 0xffu;
    uint4 raw0 = make_uint4(0, 0, 0, 0), raw1 = make_uint4(0, 0, 0, 0);
    if (g < GG) {
      if (p.q_f16) {
        raw0 = *reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(p.q) + off);
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(p.q) + off);
        raw0 = src[0];
        raw1 = src[1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
    if (g < GG) {
      float x[8];
      if (p.q_f16) {
        const uint32_t r[4] = {raw0.x, raw0.y, raw0.z, raw0.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          x[2 * t] = h2f((uint16_t)(r[t] & 0xffffu));
          x[2 * t + 1] = h2f((uint16_t)(r[t] >> 16));
        }
      } else {
        const uint32_t r[8] = {raw0.x, raw0.y, raw0.z, raw0.w, raw1.x, raw1.y, raw1.z, raw1.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) x[t] = __builtin_bit_cast(float, r[t]);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if ((sb >> t) & 1u) x[t] = -x[t];
#pragma unroll
      for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if ((t & h) == 0) {
            const float a = x[t], b = x[t + h];
            x[t] = a + b;
            x[t + h] = a - b;
          }
#pragma unroll
      for (int dl = 1; dl < LPQ; dl <<= 1) {
        const bool upper = (k & dl) != 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float o = __shfl_xor(x[t], dl, 64);
          x[t] = upper ? (o - x[t]) : (x[t] + o);
        }
      }
      const float rs = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
      for (int t = 0; t < 8; ++t) qs[g * D + 8 * k + t] = x[t] * rs;
    }
  } else {
    between();
    for (int idx = tid; idx < GG * D; idx += kThreads) {
      const size_t off = ((size_t)u.b * p.Hq + u.h0 + idx / D) * D + idx % D;
      qs[idx] = p.q_f16 ? (float)reinterpret_cast<const _Float16*>(p.q)[off] : reinterpret_cast<const float*>(p.q)[off];
    }
  }
  lds_barrier();
}

// Scores of the key held by this lane for all GG heads (before the norm).
// `lut` is the byte address of the table in LDS.
template <class S, int GG>
__device__ __forceinline__ void lut_scores(const unsigned char* __restrict__ lut, const uint32_t (&w)[S::NW],
                                           float (&acc)[GG]) {
  constexpr int HW = GG < 4 ? GG : 4;
  constexpr int NQ = GG / HW;
  constexpr int ES = HW * 4;  // bytes per table entry
  using E = typename VecF<HW>::type;
#pragma unroll
  for (int g = 0; g < GG; ++g) acc[g] = 0.0f;
  if constexpr (S::kNibbles) {
    // Two 4-bit codes per byte: shift every nibble into place as a byte offset (code * ES) so that one
    // byte extract gives the LDS address of a coordinate's entry.  The gathers run one stage (4
    // coordinates x NQ head groups) ahead of the adds that consume them, so 2*4*NQ reads are in flight;
    // the scheduling barriers keep the compiler from folding the stages back together.
    constexpr int LG = ES == 16 ? 4 : (ES == 8 ? 3 : 2);
    constexpr uint32_t MASK = 0x0F0F0F0Fu << LG;
    constexpr int ST = 4;                     // coordinates per stage
    constexpr int NST = S::ROWS / ST;
    E buf[2][ST * NQ];
    auto issue = [&](int st, E* b) {
      const int k = st / 2, half = st % 2;
      const uint32_t e = (w[k] << LG) & MASK;        // even coordinates of word k
      const uint32_t o = (w[k] >> (4 - LG)) & MASK;  // odd coordinates of word k
#pragma unroll
      for (int cc = 0; cc < ST; ++cc) {
        const int m = 2 * half + cc / 2;
        const uint32_t a = __builtin_amdgcn_ubfe(cc % 2 ? o : e, 8 * m, 8);
        const int i = ST * st + cc;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq)
          b[cc * NQ + qq] = *reinterpret_cast<const E*>(lut + (size_t)((qq * S::ROWS + i) * S::COLS) * ES + a);
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
        for (int qq = 0; qq < NQ; ++qq) add_into(acc + qq * HW, buf[st & 1][cc * NQ + qq]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < S::ROWS; ++i) {
      const uint32_t c = S::code(w, i);
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq)
        add_into(acc + qq * HW, reinterpret_cast<const E*>(lut)[(qq * S::ROWS + i) * S::COLS + c]);
    }
  }
}

// ---- buffer-resource loads: 32-bit offsets from a per-split base, and every byte past the split's valid
// range reads as 0, so the last (partial) chunk needs neither clamping nor branches.
constexpr int kBufFlags = 0x00020000;  // raw buffer, 32-bit data (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufFlags);
}

// The N-byte code row at voff + soff into little-endian 32-bit words.
template <int N>
__device__ __forceinline__ void load_code_row_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t (&w)[(N + 3) / 4]) {
  if constexpr (N % 16 == 0) {
#pragma unroll
    for (int k = 0; k < N / 16; ++k) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16 * k, 0);
      w[4 * k + 0] = x[0]; w[4 * k + 1] = x[1]; w[4 * k + 2] = x[2]; w[4 * k + 3] = x[3];
    }
  } else if constexpr (N % 8 == 0) {
#pragma unroll
    for (int k = 0; k < N / 8; ++k) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff + 8 * k, 0);
      w[2 * k + 0] = x[0]; w[2 * k + 1] = x[1];
    }
  } else if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) w[k] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff + 4 * k, 0);
  } else {
    static_assert(N % 2 == 0, "code rows are an even number of bytes");
#pragma unroll
    for (int k = 0; k < (N + 3) / 4; ++k) w[k] = 0;
#pragma unroll
    for (int k = 0; k < N / 2; ++k)
      w[k / 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff + 2 * k, 0) << (16 * (k % 2));
  }
}

// DPL consecutive V elements (fp16 or fp32) at voff + soff: the slice this lane contributes to the MFMA
// A operand.  Past the split's valid range the elements read as 0.
template <typename PT, int DPL, typename VR>
__device__ __forceinline__ VR load_vrow_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  VR out;
  if constexpr (DPL == 1) {
    out = VR{};
    if constexpr (sizeof(PT) == 2) out[0] = __builtin_bit_cast(PT, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
    else out[0] = __builtin_bit_cast(PT, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
  } else {
    constexpr int BYTES = DPL * (int)sizeof(PT);
    static_assert(BYTES == (int)sizeof(VR), "slice type");
    if constexpr (BYTES == 4) {
      out = __builtin_bit_cast(VR, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    } else if constexpr (BYTES == 8) {
      out = __builtin_bit_cast(VR, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    } else if constexpr (BYTES == 16) {
      out = __builtin_bit_cast(VR, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    } else {
      static_assert(BYTES % 16 == 0, "V slice is a multiple of 16 bytes");
      typedef unsigned u4 __attribute__((ext_vector_type(4)));
      struct Parts { u4 x[BYTES / 16]; } parts;
#pragma unroll
      for (int k = 0; k < BYTES / 16; ++k) parts.x[k] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 16 * k, 0);
      out = __builtin_bit_cast(VR, parts);
    }
  }
  return out;
}

// Arrival counter of one (b, kv head, head group): zero before the call, incremented once by every
// split's workgroup (a single device-scope fetch-add: no retry loop, so late arrivals do not queue behind
// each other), and put back to zero by the last one, which merges the splits.
__device__ __forceinline__ unsigned arrive(unsigned* c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}

// Split partials are exchanged between workgroups (possibly on different XCDs, whose L2 caches are not
// coherent with each other) with device-scope stores and loads, which go to the device coherence point
// instead of a non-coherent cache; a writer waits for its stores to complete before it counts itself in.
__device__ __forceinline__ void st_dev(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class S, int GG, bool VF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void decode_kernel(const AttnParams p) {
  constexpr int D = S::D;
  constexpr int DPL = D / 16;  // V columns per lane per MFMA tile set
  using Plan = LdsPlan<S, GG>;
  constexpr int HW = Plan::HW;
  using PT = typename std::conditional<VF16, _Float16, float>::type;
  typedef PT vrow_t __attribute__((ext_vector_type(DPL < 2 ? 2 : DPL)));
  __shared__ __align__(16) unsigned char smem[Plan::total(VF16)];
  float* lv = reinterpret_cast<float*>(smem + Plan::consts_off);
  int* s_flag = reinterpret_cast<int*>(smem + Plan::consts_off + 96);
  float* qs = reinterpret_cast<float*>(smem + Plan::qs_off);
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

  // Loads run one chunk ahead of the arithmetic: the codes, norms and (fp16) V slices of chunk c+1 are
  // requested before chunk c is scored.  The first chunk's are requested before the prologue so they
  // arrive while the table is built.
  constexpr int KS16 = VF16 ? 4 : 1;
  int c = wid * kChunk;  // chunk start, relative to t_begin
  uint32_t wn[S::NW];
  float nn = 1.0f;
  vrow_t vn[KS16][4];
  auto fetch = [&](int cc) {
    load_code_row_buf<S::BPK>(rc, voff_code, cc * S::BPK, wn);
    if constexpr (S::kNorm) nn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rn, lane * 4, cc * 4, 0));
    if constexpr (VF16) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          vn[ks][s] = load_vrow_buf<PT, DPL, vrow_t>(rv, voff_v, (cc + 16 * ks + s) * D * (int)sizeof(PT));
    }
  };
  // (loads past the split's end read as zeros, so the fetches need no guard: a guard would also make the
  // compiler wait for every outstanding load wherever it cannot count them)
  prologue<S, GG>(p, u, qs, lv, tid, [&] { fetch(c); });
  S::template build<GG, HW>(p, qs, lv, reinterpret_cast<float*>(smem), u.kvh, tid);
  lds_barrier();

  float m_run[GG], l_lane[GG];
#pragma unroll
  for (int g = 0; g < GG; ++g) {
    m_run[g] = -INFINITY;
    l_lane[g] = 0.0f;
  }
  float4_t oacc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) oacc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
  PT* pw = pst + wid * GG * kChunk;

#pragma unroll 2
  for (; c < n_valid; c += kWaves * kChunk) {
    // this chunk's data (fetched one iteration earlier), then the next chunk's requests
    uint32_t w[S::NW];
#pragma unroll
    for (int k = 0; k < S::NW; ++k) w[k] = wn[k];
    const float nrm = nn;
    vrow_t vr[KS16][4];
#pragma unroll
    for (int ks = 0; ks < KS16; ++ks)
#pragma unroll
      for (int s = 0; s < 4; ++s) vr[ks][s] = vn[ks][s];
    fetch(c + kWaves * kChunk);

    // ---- scores from the table
    float acc[GG];
    lut_scores<S, GG>(smem, w, acc);
    float z[GG];
    const float zs = S::kNorm ? nrm * p.zscale : p.zscale;
#pragma unroll
    for (int g = 0; g < GG; ++g) z[g] = acc[g] * zs;
    if (c + kChunk > n_valid) {  // the split's last, partial chunk
      const bool valid = c + lane < n_valid;
#pragma unroll
      for (int g = 0; g < GG; ++g) z[g] = valid ? z[g] : -INFINITY;
    }
    bool need = false;
#pragma unroll
    for (int g = 0; g < GG; ++g) need |= z[g] > m_run[g] + kLazyHeadroom;
    // ---- online softmax: raise the running maximum only when needed
    if (__any(need)) {
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
      pw[g * kChunk + lane] = (PT)pr;
    }
    wave_lds_sync();

    // ---- out^T += V^T P^T on the matrix cores
    if constexpr (VF16) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half4_t bop = half4_t{0, 0, 0, 0};
        if (r16 < GG) bop = *reinterpret_cast<const half4_t*>(pw + r16 * kChunk + 16 * ks + 4 * kq);
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          half4_t a = half4_t{vr[ks][0][j], vr[ks][1][j], vr[ks][2][j], vr[ks][3][j]};
          oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bop, oacc[j], 0, 0, 0);
        }
      }
    } else {
#pragma unroll 4
      for (int ks = 0; ks < 16; ++ks) {
        const vrow_t a = load_vrow_buf<PT, DPL, vrow_t>(rv, voff_v, (c + 4 * ks) * D * (int)sizeof(PT));
        float bop = 0.0f;
        if (r16 < GG) bop = pw[r16 * kChunk + 4 * ks + kq];
#pragma unroll
        for (int j = 0; j < DPL; ++j) oacc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], bop, oacc[j], 0, 0, 0);
      }
    }
    wave_lds_sync();
  }

  // ---- merge the four waves through LDS (the table is no longer needed)
  float l_w[GG];
#pragma unroll
  for (int g = 0; g < GG; ++g) l_w[g] = wave_sum(l_lane[g]);
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);            // [kWaves][GG][D]
  float* red_m = red + kWaves * GG * D;                    // [kWaves][GG]
  float* red_l = red_m + kWaves * GG;                      // [kWaves][GG]
  if (r16 < GG) {
#pragma unroll
    for (int j = 0; j < DPL; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wid * GG + r16) * D + DPL * (4 * kq + r) + j] = oacc[j][r];
  }
#pragma unroll
  for (int g = 0; g < GG; ++g)
    if (lane == g) {
      red_m[wid * GG + g] = m_run[g];
      red_l[wid * GG + g] = l_w[g];
    }
  __syncthreads();
  for (int idx = tid; idx < GG * D; idx += kThreads) {
    const int g = idx / D, dc = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, red_m[w2 * GG + g]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) {
        const float wt = fast_exp2(red_m[w2 * GG + g] - M);
        num += wt * red[(w2 * GG + g) * D + dc];
        den += wt * red_l[w2 * GG + g];
      }
    }
    const size_t row = (size_t)u.b * p.Hq + u.h0 + g;
    if (p.n_splits == 1) {
      const float o = den > 0.0f ? num / den : 0.0f;
      if (p.out_f16) reinterpret_cast<_Float16*>(p.out)[row * D + dc] = (_Float16)o;
      else reinterpret_cast<float*>(p.out)[row * D + dc] = o;
    } else {
      float* dst = p.ws + (row * p.n_splits + split) * (D + kRecPad);
      st_dev(dst + dc, num);
      if (dc == 0) {
        st_dev(dst + D, M);
        st_dev(dst + D + 1, den);
      }
    }
  }
  if (p.n_splits == 1) return;

  // ---- the last workgroup of this (b, kv head, head group) to arrive merges all splits
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const bool last = arrive(p.counters + blockIdx.y) == (unsigned)p.n_splits;
    if (last) __hip_atomic_store(p.counters + blockIdx.y, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  if (!*s_flag) return;
  const int S_ = p.n_splits;
  for (int idx = tid; idx < GG * D; idx += kThreads) {
    const int g = idx / D, dc = idx % D;
    const size_t row = (size_t)u.b * p.Hq + u.h0 + g;
    const float* base = p.ws + row * (size_t)S_ * (D + kRecPad);
    // online log-sum-exp merge over tiles of kMergeTile splits; each tile's loads are issued together
    float M = -INFINITY, num = 0.0f, den = 0.0f;
    for (int s0 = 0; s0 < S_; s0 += kMergeTile) {
      float mv[kMergeTile], dv[kMergeTile], nv[kMergeTile];
#pragma unroll
      for (int k = 0; k < kMergeTile; ++k) {
        mv[k] = -INFINITY;
        dv[k] = 0.0f;
        nv[k] = 0.0f;
        if (s0 + k < S_) {
          const float* rec = base + (size_t)(s0 + k) * (D + kRecPad);
          mv[k] = ld_dev(rec + D);
          dv[k] = ld_dev(rec + D + 1);
          nv[k] = ld_dev(rec + dc);
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
    const float o = den > 0.0f ? num / den : 0.0f;
    if (p.out_f16) reinterpret_cast<_Float16*>(p.out)[row * D + dc] = (_Float16)o;
    else reinterpret_cast<float*>(p.out)[row * D + dc] = o;
  }
}

template <class S, int GG>
__global__ __launch_bounds__(kThreads) void score_kernel(const AttnParams p) {
  using Plan = LdsPlan<S, GG>;
  constexpr int HW = Plan::HW;
  __shared__ __align__(16) unsigned char smem[Plan::pst_off];
  float* lv = reinterpret_cast<float*>(smem + Plan::consts_off);
  float* qs = reinterpret_cast<float*>(smem + Plan::qs_off);

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

  prologue<S, GG>(p, u, qs, lv, tid, [] {});
  S::template build<GG, HW>(p, qs, lv, reinterpret_cast<float*>(smem), u.kvh, tid);
  lds_barrier();

  for (int c = wid * kChunk; c < n_stop; c += kWaves * kChunk) {
    uint32_t w[S::NW];
    float nrm = 1.0f;
    load_code_row_buf<S::BPK>(rc, lane * S::BPK, c * S::BPK, w);
    if constexpr (S::kNorm) nrm = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rn, lane * 4, c * 4, 0));
    float acc[GG];
    lut_scores<S, GG>(smem, w, acc);
    const int t = c + lane;
    if (t < n_stop) {
      const bool valid = t < n_valid;
#pragma unroll
      for (int g = 0; g < GG; ++g) {
        const float s = S::kNorm ? nrm * acc[g] : acc[g];
        p.scores[((size_t)u.b * p.Hq + u.h0 + g) * p.T_cap + t_begin + t] = valid ? s : -INFINITY;
      }
    }
  }
}

// The kernels' LDS is static (sized per instantiation), so nothing is requested at launch.
template <class Kern>
hipError_t launch_attn(Kern kernel, size_t lds, dim3 grid, hipStream_t s, const AttnParams& p) {
  if (lds > 160 * 1024) return hipErrorNotSupported;
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <class S, int GG>
hipError_t run_decode_gg(bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
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
    case 1: return launch_attn(score_kernel<S, 1>, LdsPlan<S, 1>::pst_off, grid, s, p);
    case 2: return launch_attn(score_kernel<S, 2>, LdsPlan<S, 2>::pst_off, grid, s, p);
    case 4: return launch_attn(score_kernel<S, 4>, LdsPlan<S, 4>::pst_off, grid, s, p);
    case 8: return launch_attn(score_kernel<S, 8>, LdsPlan<S, 8>::pst_off, grid, s, p);
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

}  // namespace kvq
