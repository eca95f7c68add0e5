// Write path of the Hadamard/Lloyd-Max codec ("AXELRAM: Quantize Once, Never
// Dequantize", Key Points / Abstract: transform on write, store indices of a
// codebook fixed by d and b).
//
// For every key k: n = ||k||, y = H D k / n with H the normalised Sylvester
// Walsh-Hadamard matrix and D the sign pattern, code_i = #{ j : t_j <= y_i },
// codes packed LSB-first (b bits per coordinate) next to the fp32 norm.
//
// Layout: 8 coordinates per lane, D/8 lanes per key, so a wave holds 64/(D/8)
// keys.  The key is read with one 16-byte load per lane (fp16) and fully
// coalesced across the wave.  The transform is an in-register radix-2 fast
// Walsh-Hadamard transform for the lane's 8 coordinates followed by
// log2(D/8) cross-lane butterfly stages; ||k||^2 is reduced across the same
// lanes.  Each lane then compares its 8 coordinates with the thresholds,
// packs 8*b bits and stores them at its own byte offset of the key's row.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

template <int D, int BITS, bool KF16>
__global__ __launch_bounds__(256) void hlm_encode_kernel(const EncodeParams p) {
  constexpr int LPK = D / 8;           // lanes per key
  constexpr int KPB = 256 / LPK;       // keys per workgroup
  constexpr int L = 1 << BITS;
  constexpr int BPK = D * BITS / 8;    // code bytes per key
  const int tid = threadIdx.x;
  const int lk = tid & (LPK - 1);
  const int64_t key = (int64_t)blockIdx.x * KPB + tid / LPK;
  const int64_t n_keys = (int64_t)p.B * p.Hkv * p.T_new;
  const bool valid = key < n_keys;

  float x[8];
  if (valid) {
    if constexpr (KF16) {
      const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(p.keys) + key * D + lk * 8);
      const uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = h2f((uint16_t)(r[j] & 0xffffu));
        x[2 * j + 1] = h2f((uint16_t)(r[j] >> 16));
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.keys) + key * D + lk * 8);
      const float4 a = src[0], c = src[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.0f;
  }

  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
#pragma unroll
  for (int o = 1; o < LPK; o <<= 1) ss += __shfl_xor(ss, o, 64);

  // sign pattern D for coordinates lk*8 .. lk*8+7
  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < (D + 31) / 32; ++k)
    if (((lk * 8) >> 5) == k) word = p.signs[k];
  const uint32_t sb = (word >> ((lk * 8) & 31)) & 0xffu;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if ((sb >> j) & 1u) x[j] = -x[j];

  // in-register butterflies (distances 1, 2, 4)
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0) {
        const float a = x[i], c = x[i + h];
        x[i] = a + c;
        x[i + h] = a - c;
      }
  // cross-lane butterflies (distances 8, 16, ... = lane distances 1, 2, ...)
#pragma unroll
  for (int dl = 1; dl < LPK; dl <<= 1) {
    const bool upper = (lk & dl) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float o = __shfl_xor(x[j], dl, 64);
      x[j] = upper ? (o - x[j]) : (x[j] + o);
    }
  }

  const float nrm = __builtin_sqrtf(ss);
  const float inv = nrm > 0.0f ? 1.0f / (nrm * __builtin_sqrtf((float)D)) : 0.0f;
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float y = x[j] * inv;
    uint32_t c = 0;
#pragma unroll
    for (int t = 0; t < L - 1; ++t) c += (y >= p.thresholds[t]) ? 1u : 0u;
    packed |= c << (BITS * j);
  }

  if (!valid) return;
  const int64_t bh = key / p.T_new;
  const int64_t t = key - bh * p.T_new;
  const int b = (int)(bh / p.Hkv);
  const int64_t pos = (p.write_pos ? (int64_t)p.write_pos[b] : p.t0) + t;
  if (pos < 0 || pos >= p.T_cap) return;
  const int64_t row = bh * p.T_cap + pos;
  uint8_t* dst = p.codes + row * BPK + lk * BITS;
  if constexpr (BITS == 4) {
    *reinterpret_cast<uint32_t*>(dst) = packed;
  } else if constexpr (BITS == 2) {
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
  } else if constexpr (BITS == 1) {
    *dst = (uint8_t)packed;
  } else {
    dst[0] = (uint8_t)packed;
    dst[1] = (uint8_t)(packed >> 8);
    dst[2] = (uint8_t)(packed >> 16);
  }
  if (lk == 0) p.norms[row] = nrm;
}

template <int D, int BITS>
static hipError_t encode_launch(bool kf16, const EncodeParams& p, hipStream_t s) {
  constexpr int KPB = 256 / (D / 8);
  const int64_t n_keys = (int64_t)p.B * p.Hkv * p.T_new;
  const dim3 grid((unsigned)((n_keys + KPB - 1) / KPB));
  if (kf16) hipLaunchKernelGGL((hlm_encode_kernel<D, BITS, true>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((hlm_encode_kernel<D, BITS, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
static hipError_t encode_d(int bits, bool kf16, const EncodeParams& p, hipStream_t s) {
  switch (bits) {
    case 1: return encode_launch<D, 1>(kf16, p, s);
    case 2: return encode_launch<D, 2>(kf16, p, s);
    case 3: return encode_launch<D, 3>(kf16, p, s);
    case 4: return encode_launch<D, 4>(kf16, p, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_hlm_encode(int D, int bits, bool k_f16, const EncodeParams& p, hipStream_t s) {
  switch (D) {
    case 16: return encode_d<16>(bits, k_f16, p, s);
    case 32: return encode_d<32>(bits, k_f16, p, s);
    case 64: return encode_d<64>(bits, k_f16, p, s);
    case 128: return encode_d<128>(bits, k_f16, p, s);
    case 256: return encode_d<256>(bits, k_f16, p, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace kvq
