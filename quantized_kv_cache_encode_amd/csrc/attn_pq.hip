// Product-quantization read path (table of query-subvector x centroid inner
// products, "LOOKAT" summary page, AI Summary / Abstract) and PQ encode
// (nearest centroid per subspace).
#include "attn_kernels.h"

namespace kvq {

template <int D>
static hipError_t pq_decode_d(int M, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (M) {
    case 4: return run_decode<PqScorer<D, 4>>(gg, v_f16, p, grid, s);
    case 8: return run_decode<PqScorer<D, 8>>(gg, v_f16, p, grid, s);
    case 16: return run_decode<PqScorer<D, 16>>(gg, v_f16, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

template <int D>
static hipError_t pq_score_d(int M, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (M) {
    case 4: return run_score<PqScorer<D, 4>>(gg, p, grid, s);
    case 8: return run_score<PqScorer<D, 8>>(gg, p, grid, s);
    case 16: return run_score<PqScorer<D, 16>>(gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_pq_decode(int D, int M, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  if (!v_f16) return hipErrorNotSupported;
  switch (D) {
    case 64: return pq_decode_d<64>(M, gg, true, p, grid, s);
    case 128: return pq_decode_d<128>(M, gg, true, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_pq_score(int D, int M, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 64: return pq_score_d<64>(M, gg, p, grid, s);
    case 128: return pq_score_d<128>(M, gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

// One workgroup = 256 keys of one (batch, kv head) and one subspace s: that subspace's centroids [K][D/M]
// are staged in LDS and every lane scans them for its key's sub-vector (all lanes read the same centroid at
// once: an LDS broadcast).  Squared distances sum (x_k - c_k)^2 in fp32 in coordinate order; ties keep the
// lowest index.  Parallel over (key, subspace), so even a short cache fills the chip.
template <int D, int M, bool KF16>
__global__ __launch_bounds__(256) void pq_encode_kernel(const EncodeParams p) {
  constexpr int DS = D / M;
  extern __shared__ __align__(16) float cent_s[];
  const int K = p.pq_K;
  const int bh = blockIdx.y;
  const int s = blockIdx.z;
  const int h = bh % p.Hkv, b = bh / p.Hkv;
  const float* cg = p.pq_cent + ((size_t)h * M + s) * K * DS;
  for (int x = threadIdx.x; x < K * DS; x += 256) cent_s[x] = cg[x];
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= p.T_new) return;
  const int64_t pos = (p.write_pos ? (int64_t)p.write_pos[b] : p.t0) + t;
  if (pos < 0 || pos >= p.T_cap) return;
  const size_t src = ((size_t)bh * p.T_new + t) * D + (size_t)s * DS;
  float x[DS];
#pragma unroll
  for (int k = 0; k < DS; ++k)
    x[k] = KF16 ? (float)reinterpret_cast<const _Float16*>(p.keys)[src + k] : reinterpret_cast<const float*>(p.keys)[src + k];
  int best = 0;
  float bd = INFINITY;
#pragma unroll 4
  for (int c = 0; c < K; ++c) {
    const float* cc = cent_s + (size_t)c * DS;
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
  p.codes[((size_t)bh * p.T_cap + pos) * M + s] = (uint8_t)best;
}

template <int D, int M, bool KF16>
static hipError_t pq_encode_launch(const EncodeParams& p, hipStream_t s) {
  const size_t lds = (size_t)(D / M) * p.pq_K * 4;
  if (lds > 64 * 1024) return hipErrorNotSupported;
  dim3 grid((unsigned)((p.T_new + 255) / 256), (unsigned)(p.B * p.Hkv), (unsigned)M);
  hipLaunchKernelGGL((pq_encode_kernel<D, M, KF16>), grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

template <int D>
static hipError_t pq_encode_d(int M, bool kf16, const EncodeParams& p, hipStream_t s) {
  switch (M) {
    case 4: return kf16 ? pq_encode_launch<D, 4, true>(p, s) : pq_encode_launch<D, 4, false>(p, s);
    case 8: return kf16 ? pq_encode_launch<D, 8, true>(p, s) : pq_encode_launch<D, 8, false>(p, s);
    case 16: return kf16 ? pq_encode_launch<D, 16, true>(p, s) : pq_encode_launch<D, 16, false>(p, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_pq_encode(int D, int M, bool k_f16, const EncodeParams& p, hipStream_t s) {
  switch (D) {
    case 64: return pq_encode_d<64>(M, k_f16, p, s);
    case 128: return pq_encode_d<128>(M, k_f16, p, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace kvq
