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

// Nearest centroid (squared L2 in fp32, coordinates summed in order, ties keep the lowest index) of the
// DS-element sub-vector x among the K centroids [K][DS] at cent (LDS: all lanes read the same centroid at
// once, a broadcast).
template <int DS>
__device__ __forceinline__ int pq_nearest(const float (&x)[DS], const float* cent, int K) {
  int best = 0;
  float bd = INFINITY;
#pragma unroll 4
  for (int c = 0; c < K; ++c) {
    const float* cc = cent + (size_t)c * DS;
    float dist = 0.0f;
#pragma unroll
    for (int k = 0; k < DS; ++k) {
      const float e = x[k] - cc[k];
      dist = __builtin_fmaf(e, e, dist);
    }
    if (dist < bd) {
      bd = dist;
      best = c;
    }
  }
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
  for (int x = threadIdx.x; x < SPB * K * DS; x += 256) cent_s[x] = cg[x];
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

template <int D, int M, int CB, bool KF16>
static hipError_t pq_encode_launch(const EncodeParams& p, hipStream_t s) {
  constexpr int SPB = 8 / CB;
  const size_t lds = (size_t)SPB * (D / M) * p.pq_K * 4;
  if (lds > 64 * 1024) return hipErrorNotSupported;
  dim3 grid((unsigned)((p.T_new + 255) / 256), (unsigned)(p.B * p.Hkv), (unsigned)(M / SPB));
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
