// Dispatch of the read-path kernels by head dimension, and the kernel that
// merges split-T partial results.
#include "attn_kernels.h"

namespace kvq {

extern template hipError_t run_hlm_decode<16>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_decode<32>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_decode<64>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_decode<128>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_decode<256>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<16>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<32>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<64>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<128>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<256>(int, int, const AttnParams&, dim3, hipStream_t);

hipError_t launch_hlm_decode(int D, int bits, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 16: return run_hlm_decode<16>(bits, gg, v_f16, p, grid, s);
    case 32: return run_hlm_decode<32>(bits, gg, v_f16, p, grid, s);
    case 64: return run_hlm_decode<64>(bits, gg, v_f16, p, grid, s);
    case 128: return run_hlm_decode<128>(bits, gg, v_f16, p, grid, s);
    case 256: return run_hlm_decode<256>(bits, gg, v_f16, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_hlm_score(int D, int bits, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 16: return run_hlm_score<16>(bits, gg, p, grid, s);
    case 32: return run_hlm_score<32>(bits, gg, p, grid, s);
    case 64: return run_hlm_score<64>(bits, gg, p, grid, s);
    case 128: return run_hlm_score<128>(bits, gg, p, grid, s);
    case 256: return run_hlm_score<256>(bits, gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

// Log-sum-exp merge of the split partials (num[D], max, den) of one
// (batch, query head) row: out = sum_s 2^(m_s - M) num_s / sum_s 2^(m_s - M) den_s,
// with the maxima in the log2 domain of the decode kernel.  Rows whose splits
// saw no key at all (empty sequence) give zeros.
__global__ __launch_bounds__(256) void combine_kernel(const AttnParams p, int D) {
  const size_t row = blockIdx.x;
  const int S = p.n_splits;
  const float* base = p.ws + row * (size_t)S * (D + 2);
  for (int dc = threadIdx.x; dc < D; dc += blockDim.x) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, base[(size_t)s * (D + 2) + D]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
      for (int s = 0; s < S; ++s) {
        const float* part = base + (size_t)s * (D + 2);
        const float wt = fast_exp2(part[D] - M);
        num += wt * part[dc];
        den += wt * part[D + 1];
      }
    }
    const float o = den > 0.0f ? num / den : 0.0f;
    if (p.out_f16) reinterpret_cast<_Float16*>(p.out)[row * D + dc] = (_Float16)o;
    else reinterpret_cast<float*>(p.out)[row * D + dc] = o;
  }
}

hipError_t launch_combine(const AttnParams& p, int D, hipStream_t s) {
  const int threads = D < 64 ? 64 : D;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(p.B * p.Hq)), dim3(threads), 0, s, p, D);
  return hipGetLastError();
}

}  // namespace kvq
