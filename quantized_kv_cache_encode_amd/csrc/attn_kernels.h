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
// Work decomposition (one workgroup = 4 waves of 64 lanes):
//   workgroup <- (batch b, kv head, group of GG query heads, split of T);
//   prologue: the GG queries are loaded into LDS, sign-flipped and put
//   through an in-LDS fast Walsh-Hadamard transform (Hadamard codec), then
//   the table for all GG heads is written to LDS as [GG/HW][rows][cols] of
//   HW-wide float vectors (HW = min(GG, 4)), so one ds_read_b128 at
//   (row, code) returns the entries of four heads;
//   main loop: a wave takes 64 consecutive keys at a time, lane <-> key.
//   Every lane unpacks its key's codes from registers and gathers one vector
//   per (row, head quad); all lanes read the same row at once and a row
//   holds at most `cols` entries, so a wave's gather touches one contiguous
//   span of LDS (no bank conflicts for cols <= 16).  Scores feed an online
//   softmax whose running maximum is only raised when a score exceeds it by
//   more than 2^8 (so probabilities stay <= 256), and the probabilities are
//   staged through LDS as the B operand of MFMA 16x16x16 f16 (fp32 values:
//   16x16x4 f32) whose A operand is V^T, giving out^T[dim][head] in the
//   matrix-core accumulators.  The four waves merge their (max, sum, acc)
//   through LDS; splits are merged by a log-sum-exp combine kernel.
#pragma once

#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 64;
constexpr float kLazyHeadroom = 8.0f;  // log2 of the largest probability allowed before rescaling

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
  __device__ static __forceinline__ uint32_t code(const uint32_t (&w)[NW], int i) { return code_at<BITS, NW>(w, i); }
  // LUT[g][i][j] = q'_{g,i} * c_j with q' = H D q (qs holds the unnormalised transform).
  template <int GG, int HW>
  __device__ static void build(const AttnParams&, const float* qs, const float* lv, float* lut, int, int tid) {
    constexpr int total = GG * ROWS * COLS;
    const float rs = 1.0f / __builtin_sqrtf((float)D);
    for (int idx = tid; idx < total; idx += kThreads) {
      const int hh = idx % HW;
      const int j = (idx / HW) % COLS;
      const int i = (idx / (HW * COLS)) % ROWS;
      const int g = (idx / (HW * COLS * ROWS)) * HW + hh;
      lut[idx] = (qs[g * D + i] * rs) * lv[j];
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
  static constexpr size_t consts_off = region0;                   // 16 levels + 8 sign words
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

// Loads the GG queries into qs[g][i] (fp32), copies the codebook levels and
// sign words into LDS, and for the Hadamard codec applies D then an
// unnormalised fast Walsh-Hadamard transform (Sylvester order) in LDS.
template <class S, int GG>
__device__ void prologue(const AttnParams& p, const Unit& u, float* qs, float* lv, uint32_t* sg, int tid) {
  constexpr int D = S::D;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (tid == k) lv[k] = p.levels[k];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (tid == 16 + k) sg[k] = p.signs[k];
  __syncthreads();
  for (int idx = tid; idx < GG * D; idx += kThreads) {
    const int g = idx / D, i = idx % D;
    const size_t off = ((size_t)u.b * p.Hq + u.h0 + g) * D + i;
    float x = p.q_f16 ? (float)reinterpret_cast<const _Float16*>(p.q)[off] : reinterpret_cast<const float*>(p.q)[off];
    if (S::kRotate && ((sg[i >> 5] >> (i & 31)) & 1u)) x = -x;
    qs[idx] = x;
  }
  __syncthreads();
  if constexpr (S::kRotate) {
    for (int h = 1; h < D; h <<= 1) {
      for (int pidx = tid; pidx < GG * D / 2; pidx += kThreads) {
        const int g = pidx / (D / 2), r = pidx % (D / 2);
        const int i = (r / h) * 2 * h + (r % h);
        const float a = qs[g * D + i], c = qs[g * D + i + h];
        qs[g * D + i] = a + c;
        qs[g * D + i + h] = a - c;
      }
      __syncthreads();
    }
  }
}

// DPL consecutive V elements of token ts (zeros past t_end, where the cache
// may hold anything): the slice this lane contributes to the MFMA A operand.
template <typename PT, int DPL, typename VR>
__device__ __forceinline__ VR load_vrow(const void* v, int64_t row0, int64_t ts, int64_t t_end, int D, int r16) {
  VR r = VR{};
  if (ts < t_end) {
    const PT* src = reinterpret_cast<const PT*>(v) + (size_t)(row0 + ts) * D + DPL * r16;
    if constexpr (DPL == 1) {
      r[0] = src[0];
    } else {
      r = *reinterpret_cast<const VR*>(src);
    }
  }
  return r;
}

// Scores of the key held by this lane for all GG heads (before the norm).
template <class S, int GG>
__device__ __forceinline__ void lut_scores(const typename VecF<(GG < 4 ? GG : 4)>::type* __restrict__ lut,
                                           const uint32_t (&w)[S::NW], float (&acc)[GG]) {
  constexpr int HW = GG < 4 ? GG : 4;
  constexpr int NQ = GG / HW;
#pragma unroll
  for (int g = 0; g < GG; ++g) acc[g] = 0.0f;
#pragma unroll
  for (int i = 0; i < S::ROWS; ++i) {
    const uint32_t c = S::code(w, i);
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) add_into(acc + qq * HW, lut[(qq * S::ROWS + i) * S::COLS + c]);
  }
}

template <class S, int GG, bool VF16>
__global__ __launch_bounds__(kThreads) void decode_kernel(const AttnParams p) {
  constexpr int D = S::D;
  constexpr int DPL = D / 16;  // V columns per lane per MFMA tile set
  using Plan = LdsPlan<S, GG>;
  constexpr int HW = Plan::HW;
  using E = typename VecF<HW>::type;
  using PT = typename std::conditional<VF16, _Float16, float>::type;
  extern __shared__ __align__(16) unsigned char smem[];
  E* lut = reinterpret_cast<E*>(smem);
  float* lv = reinterpret_cast<float*>(smem + Plan::consts_off);
  uint32_t* sg = reinterpret_cast<uint32_t*>(smem + Plan::consts_off + 64);
  float* qs = reinterpret_cast<float*>(smem + Plan::qs_off);
  PT* pst = reinterpret_cast<PT*>(smem + Plan::pst_off);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const Unit u = decode_unit(p, GG);
  const int split = blockIdx.x;
  const int64_t t_begin = (int64_t)split * p.split_len;
  int64_t t_end = t_begin + p.split_len;
  if (t_end > u.len) t_end = u.len;

  prologue<S, GG>(p, u, qs, lv, sg, tid);
  S::template build<GG, HW>(p, qs, lv, reinterpret_cast<float*>(lut), u.kvh, tid);
  __syncthreads();

  const int64_t row0 = ((int64_t)u.b * p.Hkv + u.kvh) * p.T_cap;
  const uint8_t* __restrict__ codes = p.codes;
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

  for (int64_t cb = t_begin + (int64_t)wid * kChunk; cb < t_end; cb += (int64_t)kWaves * kChunk) {
    // ---- loads: this lane's key codes and norm, and its V^T operand slices
    const int64_t t = cb + lane;
    const bool valid = t < t_end;
    uint32_t w[S::NW];
    if (valid) {
      load_code_row<S::BPK>(codes + (size_t)(row0 + t) * S::BPK, w);
    } else {
#pragma unroll
      for (int k = 0; k < S::NW; ++k) w[k] = 0;
    }
    float nrm = 1.0f;
    if constexpr (S::kNorm) nrm = valid ? p.norms[row0 + t] : 0.0f;

    // fp16 V: fetch this lane's V^T operand slices for the whole chunk up front
    // (4 K-steps x 4 tokens x DPL columns) so they are in flight during the gathers.
    typedef PT vrow_t __attribute__((ext_vector_type(DPL < 2 ? 2 : DPL)));
    constexpr int KS16 = VF16 ? 4 : 1;
    vrow_t vr[KS16][4];
    if constexpr (VF16) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int s = 0; s < 4; ++s) vr[ks][s] = load_vrow<PT, DPL, vrow_t>(p.v, row0, cb + 16 * ks + 4 * kq + s, t_end, D, r16);
    }

    // ---- scores from the table
    float acc[GG];
    lut_scores<S, GG>(lut, w, acc);
    float z[GG];
    bool need = false;
#pragma unroll
    for (int g = 0; g < GG; ++g) {
      const float s = S::kNorm ? nrm * acc[g] : acc[g];
      z[g] = valid ? s * p.zscale : -INFINITY;
      need |= z[g] > m_run[g] + kLazyHeadroom;
    }
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
        const vrow_t a = load_vrow<PT, DPL, vrow_t>(p.v, row0, cb + 4 * ks + kq, t_end, D, r16);
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
      float* dst = p.ws + (row * p.n_splits + split) * (D + 2);
      dst[dc] = num;
      if (dc == 0) {
        dst[D] = M;
        dst[D + 1] = den;
      }
    }
  }
}

template <class S, int GG>
__global__ __launch_bounds__(kThreads) void score_kernel(const AttnParams p) {
  constexpr int D = S::D;
  using Plan = LdsPlan<S, GG>;
  constexpr int HW = Plan::HW;
  using E = typename VecF<HW>::type;
  extern __shared__ __align__(16) unsigned char smem[];
  E* lut = reinterpret_cast<E*>(smem);
  float* lv = reinterpret_cast<float*>(smem + Plan::consts_off);
  uint32_t* sg = reinterpret_cast<uint32_t*>(smem + Plan::consts_off + 64);
  float* qs = reinterpret_cast<float*>(smem + Plan::qs_off);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const Unit u = decode_unit(p, GG);
  const int64_t t_begin = (int64_t)blockIdx.x * p.split_len;
  int64_t t_stop = t_begin + p.split_len;
  if (t_stop > p.T_cap) t_stop = p.T_cap;

  prologue<S, GG>(p, u, qs, lv, sg, tid);
  S::template build<GG, HW>(p, qs, lv, reinterpret_cast<float*>(lut), u.kvh, tid);
  __syncthreads();

  const int64_t row0 = ((int64_t)u.b * p.Hkv + u.kvh) * p.T_cap;
  for (int64_t cb = t_begin + (int64_t)wid * kChunk; cb < t_stop; cb += (int64_t)kWaves * kChunk) {
    const int64_t t = cb + lane;
    const bool inside = t < t_stop;
    const bool valid = t < u.len;
    uint32_t w[S::NW];
    if (valid) {
      load_code_row<S::BPK>(p.codes + (size_t)(row0 + t) * S::BPK, w);
    } else {
#pragma unroll
      for (int k = 0; k < S::NW; ++k) w[k] = 0;
    }
    float nrm = 1.0f;
    if constexpr (S::kNorm) nrm = valid ? p.norms[row0 + t] : 0.0f;
    float acc[GG];
    lut_scores<S, GG>(lut, w, acc);
    if (inside) {
#pragma unroll
      for (int g = 0; g < GG; ++g) {
        const float s = S::kNorm ? nrm * acc[g] : acc[g];
        p.scores[((size_t)u.b * p.Hq + u.h0 + g) * p.T_cap + t] = valid ? s : -INFINITY;
      }
    }
  }
}

template <class Kern>
hipError_t launch_attn(Kern kernel, size_t lds, dim3 grid, hipStream_t s, const AttnParams& p) {
  if (lds > 160 * 1024) return hipErrorNotSupported;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), lds, s, p);
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
