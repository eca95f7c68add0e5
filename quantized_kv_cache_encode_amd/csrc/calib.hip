// One-time sign-pattern selection ("AXELRAM: Quantize Once, Never Dequantize", Key Points / Abstract: the
// sign pattern is chosen once, without gradients, among candidates evaluated on a few calibration samples).
// A candidate is ranked by the error it causes in the attention output; the kernels here supply the two
// pieces the encode and decode kernels do not: exact (unquantized) attention over the calibration keys, and
// the relative squared error of a decode output against it.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kCalibThreads = 256;

__device__ __forceinline__ float load_elem(const void* p, size_t i, bool f16) {
  return f16 ? (float)reinterpret_cast<const _Float16*>(p)[i] : reinterpret_cast<const float*>(p)[i];
}

// Sum over the workgroup (deterministic order: waves in index order).
__device__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kCalibThreads / 64; ++k) s += red[k];
  return s;
}

__device__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int k = 1; k < kCalibThreads / 64; ++k) m = fmaxf(m, red[k]);
  return m;
}

// out[n][h][:] = softmax(scale * q.k_t) V over all T keys of kv head h / G; one workgroup per (n, h).
// Scores are held in LDS (T <= kCalibMaxT).  fp32 throughout.
template <int D>
__global__ __launch_bounds__(kCalibThreads) void exact_attn_kernel(const CalibParams p) {
  __shared__ float qs[D];
  __shared__ float sc[kCalibMaxT];
  __shared__ float red[kCalibThreads / 64];
  __shared__ float part[kCalibThreads];
  const int n = blockIdx.y, h = blockIdx.x;
  const int kvh = h / (p.Hq / p.Hkv);
  const size_t qoff = ((size_t)n * p.Hq + h) * D;
  const size_t kvoff = ((size_t)n * p.Hkv + kvh) * p.T * D;
  for (int i = threadIdx.x; i < D; i += kCalibThreads) qs[i] = load_elem(p.q, qoff + i, p.q_f16);
  __syncthreads();
  float mloc = -INFINITY;
  for (int t = threadIdx.x; t < p.T; t += kCalibThreads) {
    float s = 0.0f;
    for (int i = 0; i < D; ++i) s = __builtin_fmaf(qs[i], load_elem(p.keys, kvoff + (size_t)t * D + i, p.k_f16), s);
    s *= p.scale;
    sc[t] = s;
    mloc = fmaxf(mloc, s);
  }
  const float m = block_max(mloc, red);
  float lloc = 0.0f;
  for (int t = threadIdx.x; t < p.T; t += kCalibThreads) {
    const float e = expf(sc[t] - m);
    sc[t] = e;
    lloc += e;
  }
  const float l = block_sum(lloc, red);  // its barriers also order the probabilities written above
  // out: thread (group g, dim i) sums the probabilities of keys g, g + NG, ... times V
  constexpr int NG = kCalibThreads / D > 0 ? kCalibThreads / D : 1;
  for (int i0 = 0; i0 < D; i0 += kCalibThreads) {
    const int i = i0 + (int)threadIdx.x % (D < kCalibThreads ? D : kCalibThreads);
    const int g = (int)threadIdx.x / (D < kCalibThreads ? D : kCalibThreads);
    float acc = 0.0f;
    if (i < D)
      for (int t = g; t < p.T; t += NG) acc = __builtin_fmaf(sc[t], load_elem(p.v, kvoff + (size_t)t * D + i, p.v_f16), acc);
    part[threadIdx.x] = acc;
    __syncthreads();
    if ((int)threadIdx.x < (D < kCalibThreads ? D : kCalibThreads) && i < D) {
      float s = 0.0f;
      for (int gg = 0; gg < NG; ++gg) s += part[gg * (D < kCalibThreads ? D : kCalibThreads) + threadIdx.x];
      p.out[qoff + i] = s / l;
    }
    __syncthreads();
  }
}

// errors[c] = sum (oh - o)^2 / sum o^2 over n elements (0 when o is all zero); one workgroup.
__global__ __launch_bounds__(kCalibThreads) void rel_err_kernel(const float* oh, const float* o, int64_t n,
                                                                 float* errors, int c) {
  __shared__ float red[kCalibThreads / 64];
  float num = 0.0f, den = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += kCalibThreads) {
    const float e = oh[i] - o[i];
    num = __builtin_fmaf(e, e, num);
    den = __builtin_fmaf(o[i], o[i], den);
  }
  num = block_sum(num, red);
  den = block_sum(den, red);
  if (threadIdx.x == 0) errors[c] = den > 0.0f ? num / den : 0.0f;
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, size_t n_words, hipStream_t s) {
  if (n_words == 0) return hipSuccess;
  const size_t blocks = (n_words + 255) / 256;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s, p, n_words);
  return hipGetLastError();
}

hipError_t launch_exact_attn(int D, const CalibParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.Hq, (unsigned)p.n);
  switch (D) {
    case 16: hipLaunchKernelGGL(exact_attn_kernel<16>, grid, dim3(kCalibThreads), 0, s, p); break;
    case 32: hipLaunchKernelGGL(exact_attn_kernel<32>, grid, dim3(kCalibThreads), 0, s, p); break;
    case 64: hipLaunchKernelGGL(exact_attn_kernel<64>, grid, dim3(kCalibThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL(exact_attn_kernel<128>, grid, dim3(kCalibThreads), 0, s, p); break;
    case 256: hipLaunchKernelGGL(exact_attn_kernel<256>, grid, dim3(kCalibThreads), 0, s, p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_rel_err(const float* oh, const float* o, int64_t n, float* errors, int c, hipStream_t s) {
  hipLaunchKernelGGL(rel_err_kernel, dim3(1), dim3(kCalibThreads), 0, s, oh, o, n, errors, c);
  return hipGetLastError();
}

}  // namespace kvq
