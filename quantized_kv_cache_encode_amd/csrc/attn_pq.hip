// Product-quantization read path (table of query-subvector x centroid inner
// products, "LOOKAT" summary page, AI Summary / Abstract) and PQ encode
// (nearest centroid per subspace).
#include "attn_kernels.h"

namespace kvq {

template <int D, int CB>
static hipError_t pq_decode_m(int M, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (M) {
    case 4: return run_decode<PqScorer<D, 4, CB>>(gg, v_f16, p, grid, s);
    case 8: return run_decode<PqScorer<D, 8, CB>>(gg, v_f16, p, grid, s);
    case 16: return run_decode<PqScorer<D, 16, CB>>(gg, v_f16, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

template <int D, int CB>
static hipError_t pq_score_m(int M, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (M) {
    case 4: return run_score<PqScorer<D, 4, CB>>(gg, p, grid, s);
    case 8: return run_score<PqScorer<D, 8, CB>>(gg, p, grid, s);
    case 16: return run_score<PqScorer<D, 16, CB>>(gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

template <int D>
static hipError_t pq_decode_d(int M, int cb, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  if (cb == 4) return pq_decode_m<D, 4>(M, gg, v_f16, p, grid, s);
  if (cb == 8) return pq_decode_m<D, 8>(M, gg, v_f16, p, grid, s);
  return hipErrorNotSupported;
}

template <int D>
static hipError_t pq_score_d(int M, int cb, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  if (cb == 4) return pq_score_m<D, 4>(M, gg, p, grid, s);
  if (cb == 8) return pq_score_m<D, 8>(M, gg, p, grid, s);
  return hipErrorNotSupported;
}

hipError_t launch_pq_decode(int D, int M, int cb, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  if (!v_f16) return hipErrorNotSupported;
  switch (D) {
    case 64: return pq_decode_d<64>(M, cb, gg, true, p, grid, s);
    case 128: return pq_decode_d<128>(M, cb, gg, true, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_pq_score(int D, int M, int cb, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 64: return pq_score_d<64>(M, cb, gg, p, grid, s);
    case 128: return pq_score_d<128>(M, cb, gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

// Squared distance of x to centroid c, coordinates in order; cent(c, k) is coordinate k of centroid c.
template <int DS, class CentAt>
__device__ __forceinline__ float pq_dist(const float (&x)[DS], int c, const CentAt& cent) {
  float dist = 0.0f;
#pragma unroll
  for (int k = 0; k < DS; ++k) {
    const float e = x[k] - cent(c, k);
    dist = __builtin_fmaf(e, e, dist);
  }
  return dist;
}

// The scan over centroids c0, c0 + step, ... < K: the first of the smallest distances, as (bd, best);
// (INFINITY, 0) when none is finite.
template <int DS, class CentAt>
__device__ __forceinline__ void pq_scan(const float (&x)[DS], const CentAt& cent, int K, int c0, int step, float& bd,
                                        int& best) {
  best = 0;
  bd = INFINITY;
#pragma unroll 4
  for (int c = c0; c < K; c += step) {
    const float dist = pq_dist<DS>(x, c, cent);
    if (dist < bd) {
      bd = dist;
      best = c;
    }
  }
}

// Nearest centroid (squared L2 in fp32, coordinates summed in order, ties keep the lowest index) of the
// DS-element sub-vector x among the K centroids [K][DS] at cent (LDS: all lanes read the same centroid at
// once, a broadcast).
template <int DS>
__device__ __forceinline__ int pq_nearest(const float (&x)[DS], const float* cent, int K) {
  float bd;
  int best;
  pq_scan<DS>(x, [&](int c, int k) { return cent[(size_t)c * DS + k]; }, K, 0, 1, bd, best);
  return best;
}

// One workgroup = 256 keys of one (batch, kv head) and one group of SPB subspaces (one subspace for byte
// codes, a pair for 4-bit codes, which share a byte): their centroids are staged in LDS and every lane
// scans them for its key's sub-vectors, then writes the byte.  Parallel over (key, subspace group), so
// even a short cache fills the chip.
template <int D, int M, int CB, bool KF16>
__global__ __launch_bounds__(256) void pq_encode_kernel(const EncodeParams p) {
  constexpr int DS = D / M;
  constexpr int SPB = 8 / CB;  // subspaces per byte
  constexpr int BPK = M * CB / 8;
  extern __shared__ __align__(16) float cent_s[];
  const int K = p.pq_K;
  const int bh = blockIdx.y;
  const int s0 = blockIdx.z * SPB;
  const int h = bh % p.Hkv, b = bh / p.Hkv;
  const float* cg = p.pq_cent + ((size_t)h * M + s0) * K * DS;
  {
    // 16-byte buffer loads, all issued before the first is used (SPB * K * DS <= 8192 floats: at most 8 per
    // thread; reads past the end return zero and are not stored)
    const int nv = SPB * K * DS / 4;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(cg, (int64_t)nv * 16);
    float4_t st[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      st[j] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, 16 * (threadIdx.x + 256 * j), 0, 0));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (threadIdx.x + 256 * j < nv) reinterpret_cast<float4_t*>(cent_s)[threadIdx.x + 256 * j] = st[j];
  }
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= p.T_new) return;
  const int64_t pos = (p.write_pos ? (int64_t)p.write_pos[b] : p.t0) + t;
  if (pos < 0 || pos >= p.T_cap) return;
  uint32_t byte = 0;
#pragma unroll
  for (int j = 0; j < SPB; ++j) {
    const size_t src = ((size_t)bh * p.T_new + t) * D + (size_t)(s0 + j) * DS;
    float x[DS];
#pragma unroll
    for (int k = 0; k < DS; ++k)
      x[k] = KF16 ? (float)reinterpret_cast<const _Float16*>(p.keys)[src + k] : reinterpret_cast<const float*>(p.keys)[src + k];
    byte |= (uint32_t)pq_nearest<DS>(x, cent_s + (size_t)j * K * DS, K) << (CB * j);
  }
  p.codes[((size_t)bh * p.T_cap + pos) * BPK + blockIdx.z] = (uint8_t)byte;
}

// Byte codes (up to 256 centroids) on the matrix cores.  The nearest centroid maximises
// s(c) = x.c - |c|^2/2, and the products x.c of 16 keys with 16 centroids at a time are one 16x16 fp32
// matrix product (the accumulators start at -|c|^2/2).  Each lane keeps the largest and the second largest
// of its values; the four lanes of a key then combine theirs.  The largest is taken where its lead over the
// second exceeds kPqMargin(DS) * (|x| + max|c|)^2, which covers the rounding of this form and of the plain
// fp32 distance form with room to spare (derived below); there the plain scan (pq_nearest) would pick the
// same centroid, unique.  Every other key (a near tie, a non-finite key or centroid, a tiny scale) runs the
// plain scan itself, so the code always equals what pq_nearest gives, ties to the lowest index included.
//
// The bound: with u = 2^-24 the matrix form errs by at most (DS + 2) u (|x||c| + |c|^2/2) (on gfx950 its
// fp32 products round like a chain of fused multiply-adds: measured against fp64, the worst error of 16x16x4
// steps at 4 to 32 dimensions equals the host chain's to within 10%), and the plain form by at most
// (DS + 3) u d with d <= (|x| + |c|)^2, i.e. half that in units of s.  Twice their sum is at most
// (3 DS + 7) u (|x| + max|c|)^2; the margin is twice that again.
template <int DS>
constexpr float kPqMargin = (6.0f * DS + 14.0f) * 0x1p-24f;

// Best and runner-up of one stream of values with the index of the best; merge() folds another stream in.
// Equal bests leave a zero lead, so which index is kept then does not matter (the lead decides).
struct PqTop2 {
  float m1, m2;
  int idx;
  __device__ __forceinline__ void merge(float o1, float o2, int oi) {
    const float r2 = fmaxf(fmaxf(m2, o2), fminf(m1, o1));
    if (o1 > m1 || (o1 == m1 && oi < idx)) idx = oi;
    m1 = fmaxf(m1, o1);
    m2 = r2;
  }
};

// The matrix operands' copy of one subspace's centroids in LDS: lane (n, kq) of a 16x16x4 step reads
// DQ = DS/4 consecutive coordinates kq*DQ .. of row n, so the coordinates are cut into quarters (kq), each
// quarter into slabs of W = min(DQ, 4) coordinates, and every slab holds its W coordinates of all KP rows
// contiguously.  A lane's read is then one W-dword vector at slab + row * W, and each slab's stride is padded
// so that the lanes of one LDS pass (64 dwords wide) fall on 64 different banks: for W = 1 all 64 lanes
// read in one pass (stride = 16 mod 64), for W = 2 the two halves of the wave (stride = 32 mod 64), for
// W = 4 each quarter (any stride).
template <int DS>
struct PqSlabs {
  static constexpr int DQ = DS / 4;
  static constexpr int W = DQ < 4 ? DQ : 4;
  static constexpr int G = DQ / W;  // slabs per quarter
  __host__ __device__ static int stride(int KP) {
    if constexpr (W == 1) return KP + ((16 - KP) & 63);
    else if constexpr (W == 2) return 2 * KP + 32;
    else return 4 * KP;
  }
  // dword offset of coordinate dim of row r
  __host__ __device__ static int at(int KP, int r, int dim) {
    const int kq = dim / DQ, k = dim % DQ;
    return (kq * G + k / W) * stride(KP) + r * W + k % W;
  }
  __host__ __device__ static int words(int KP) { return 4 * G * stride(KP); }
};

template <int D, int M, bool KF16>
// amdgpu_waves_per_eu(4): at most 128 registers, so the matrix products write ordinary registers that the
// comparisons read directly
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void pq_encode_mfma_kernel(const EncodeParams p) {
  constexpr int DS = D / M;
  constexpr int DQ = DS / 4;  // dimensions per lane and matrix step (the four k rows of a 16x16x4 step)
  using SL = PqSlabs<DS>;
  extern __shared__ __align__(16) float slab[];  // the centroids in slabs, then the biases
  const int K = p.pq_K;
  const int KP = (K + 31) & ~31;  // centroid rows padded to whole pairs of tiles (zero rows, bias -inf)
  float* bias = slab + SL::words(KP);
  unsigned* cmax_bits = reinterpret_cast<unsigned*>(bias + KP);
  const int tid = threadIdx.x;
  const int bh = blockIdx.y, sub = blockIdx.z;
  const int h = bh % p.Hkv, b = bh / p.Hkv;
  const float* cg = p.pq_cent + ((size_t)h * M + sub) * K * DS;
  const int lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, kq = lane >> 4;  // the lane's key within the 16 and its quarter of the k rows

  // every load goes out first: the lane's key coordinates for its four groups of 16 keys, then the
  // centroids as 16-byte buffer loads (zero past the K rows, which pads the last tile)
  float x[4][DQ];
  size_t src[4];
  bool valid[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int64_t t = (int64_t)blockIdx.x * 256 + wid * 64 + kt * 16 + n;
    valid[kt] = t < p.T_new;
    src[kt] = ((size_t)bh * p.T_new + (valid[kt] ? t : 0)) * D + (size_t)sub * DS;
#pragma unroll
    for (int k = 0; k < DQ; ++k) {
      const size_t e = src[kt] + kq * DQ + k;
      x[kt][k] = !valid[kt] ? 0.0f
                            : KF16 ? (float)reinterpret_cast<const _Float16*>(p.keys)[e]
                                   : reinterpret_cast<const float*>(p.keys)[e];
    }
  }
  {
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(cg, (int64_t)K * DS * 4);
    float4_t st[DS / 4];  // KP * DS / 4 <= 64 * DS vectors: DS / 4 per thread
#pragma unroll
    for (int j = 0; j < DS / 4; ++j)
      st[j] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, 16 * (tid + 256 * j), 0, 0));
    if (tid == 0) *cmax_bits = 0u;
#pragma unroll
    for (int j = 0; j < DS / 4; ++j) {
      const int v = tid + 256 * j;  // coordinates 4v .. 4v + 3: row 4v / DS
      if (v >= KP * DS / 4) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) slab[SL::at(KP, 4 * v / DS, (4 * v + e) % DS)] = st[j][e];
    }
  }
  __syncthreads();
  auto cent = [&](int c, int k) { return slab[SL::at(KP, c, k)]; };
  for (int c = tid; c < KP; c += 256) {
    float n2 = 0.0f;
#pragma unroll
    for (int k = 0; k < DS; ++k) n2 = __builtin_fmaf(cent(c, k), cent(c, k), n2);
    bias[c] = c < K ? -0.5f * n2 : -INFINITY;
    if (c < K) atomicMax(cmax_bits, __builtin_bit_cast(unsigned, n2));  // n2 >= 0 orders as its bits
  }
  __syncthreads();
  const float cmax = __builtin_sqrtf(__builtin_bit_cast(float, *cmax_bits));  // NaN if a centroid is NaN

  const int64_t pos0 = p.write_pos ? (int64_t)p.write_pos[b] : p.t0;
  const float* arow = slab + kq * SL::G * SL::stride(KP) + n * SL::W;  // + g * stride + row * W + k % W
  float xx[4];  // |x|^2 of the lane's key in each group of 16
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    xx[kt] = 0.0f;
#pragma unroll
    for (int k = 0; k < DQ; ++k) xx[kt] = __builtin_fmaf(x[kt][k], x[kt][k], xx[kt]);
    xx[kt] += __shfl_xor(xx[kt], 16, 64);
    xx[kt] += __shfl_xor(xx[kt], 32, 64);
  }
  // two groups of 16 keys per pass over the centroids, which then share each centroid read
#pragma unroll
  for (int kp = 0; kp < 4; kp += 2) {
    // one stream per group and accumulator slot r (centroid rows 4 kq + r of every tile), so that a tile's
    // four values share the one tile index they may record
    float m1[2][4], m2[2][4];
    int it[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        m1[j][r] = m2[j][r] = -INFINITY;
        it[j][r] = 0;
      }
    auto take = [&](int j, const float4_t& acc, int base) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[r];
        const bool up = v > m1[j][r];
        m2[j][r] = __builtin_amdgcn_fmed3f(m2[j][r], m1[j][r], v);  // m2 <= m1: the new runner-up
        m1[j][r] = up ? v : m1[j][r];
        it[j][r] = up ? base : it[j][r];
      }
    };
    for (int ct = 0; ct < KP; ct += 32) {
      float c0[DQ], c1[DQ];
#pragma unroll
      for (int k = 0; k < DQ; ++k) {
        c0[k] = arow[(k / SL::W) * SL::stride(KP) + ct * SL::W + k % SL::W];
        c1[k] = arow[(k / SL::W) * SL::stride(KP) + (ct + 16) * SL::W + k % SL::W];
      }
      const float4_t b0 = *reinterpret_cast<const float4_t*>(bias + ct + 4 * kq);
      const float4_t b1 = *reinterpret_cast<const float4_t*>(bias + ct + 16 + 4 * kq);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float4_t a0 = b0, a1 = b1;
#pragma unroll
        for (int k = 0; k < DQ; ++k) a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(c0[k], x[kp + j][k], a0, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < DQ; ++k) a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(c1[k], x[kp + j][k], a1, 0, 0, 0);
        take(j, a0, ct);
        take(j, a1, ct + 16);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kt = kp + j;
      const int64_t t = (int64_t)blockIdx.x * 256 + wid * 64 + kt * 16 + n;
      PqTop2 best{m1[j][0], m2[j][0], it[j][0] + 4 * kq};
#pragma unroll
      for (int r = 1; r < 4; ++r) best.merge(m1[j][r], m2[j][r], it[j][r] + 4 * kq + r);
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1)
        best.merge(__shfl_xor(best.m1, off, 64), __shfl_xor(best.m2, off, 64), __shfl_xor(best.idx, off, 64));
      const float sx = __builtin_sqrtf(xx[kt]) + cmax;
      const float marg = kPqMargin<DS> * sx * sx + 0x1p-100f;
      const bool certain = marg <= 0x1.fffffep127f && best.m1 - best.m2 >= marg;  // false for NaN anywhere
      // the rest, one key at a time (a wave-uniform loop over the uncertain keys of the 16): the plain scan
      // with the centroids dealt over the 64 lanes (c = lane mod 64), then the first of the smallest
      // distances over the lanes, which is what one scan in order gives
      int code = best.idx;
      for (uint64_t todo = __ballot(!certain && kq == 0 && valid[kt]); todo != 0; todo &= todo - 1) {
        const int kl = __builtin_ctzll(todo);  // the key's lane (n = kl, kq = 0); its quarters: lanes kl + 16 q
        float xf[DS];
#pragma unroll
        for (int k = 0; k < DS; ++k)
          xf[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x[kt][k % DQ]),
                                                                      kl + 16 * (k / DQ)));
        float bd;
        int bi;
        pq_scan<DS>(xf, cent, K, lane, 64, bd, bi);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float od = __shfl_xor(bd, off, 64);
          const int oi = __shfl_xor(bi, off, 64);
          if (od < bd || (od == bd && oi < bi)) {
            bd = od;
            bi = oi;
          }
        }
        if (lane == kl) code = bi;
      }
      if (kq != 0 || !valid[kt]) continue;
      const int64_t pos = pos0 + t;
      if (pos < 0 || pos >= p.T_cap) continue;
      p.codes[((size_t)bh * p.T_cap + pos) * M + sub] = (uint8_t)code;
    }
  }
}

template <int D, int M, int CB, bool KF16>
static hipError_t pq_encode_launch(const EncodeParams& p, hipStream_t s) {
  constexpr int SPB = 8 / CB;
  dim3 grid((unsigned)((p.T_new + 255) / 256), (unsigned)(p.B * p.Hkv), (unsigned)(M / SPB));
  // the matrix-core kernel where it measured faster than the plain scan: sub-vectors of 8 or more
  // coordinates and more than 128 centroids
  if constexpr (CB == 8 && D / M >= 8) {
    if (p.pq_K > 128) {
      const int kp = (p.pq_K + 31) / 32 * 32;
      const size_t lds = ((size_t)PqSlabs<D / M>::words(kp) + kp + 1) * 4;
      if (lds > 64 * 1024) return hipErrorNotSupported;
      hipLaunchKernelGGL((pq_encode_mfma_kernel<D, M, KF16>), grid, dim3(256), lds, s, p);
      return hipGetLastError();
    }
  }
  const size_t lds = (size_t)SPB * (D / M) * p.pq_K * 4;
  if (lds > 64 * 1024) return hipErrorNotSupported;
  hipLaunchKernelGGL((pq_encode_kernel<D, M, CB, KF16>), grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

template <int D, int CB>
static hipError_t pq_encode_m(int M, bool kf16, const EncodeParams& p, hipStream_t s) {
  switch (M) {
    case 4: return kf16 ? pq_encode_launch<D, 4, CB, true>(p, s) : pq_encode_launch<D, 4, CB, false>(p, s);
    case 8: return kf16 ? pq_encode_launch<D, 8, CB, true>(p, s) : pq_encode_launch<D, 8, CB, false>(p, s);
    case 16: return kf16 ? pq_encode_launch<D, 16, CB, true>(p, s) : pq_encode_launch<D, 16, CB, false>(p, s);
    default: return hipErrorNotSupported;
  }
}

template <int D>
static hipError_t pq_encode_d(int M, int cb, bool kf16, const EncodeParams& p, hipStream_t s) {
  if (cb == 4) return pq_encode_m<D, 4>(M, kf16, p, s);
  if (cb == 8) return pq_encode_m<D, 8>(M, kf16, p, s);
  return hipErrorNotSupported;
}

hipError_t launch_pq_encode(int D, int M, int cb, bool k_f16, const EncodeParams& p, hipStream_t s) {
  switch (D) {
    case 64: return pq_encode_d<64>(M, cb, k_f16, p, s);
    case 128: return pq_encode_d<128>(M, cb, k_f16, p, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace kvq
