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
#include "encode_dev.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

template <int D, int BITS, bool KF16>
__global__ __launch_bounds__(256) void hlm_encode_kernel(const EncodeParams p) {
  constexpr int LPK = D / 8;           // lanes per key
  constexpr int KPB = 256 / LPK;       // keys per workgroup
  constexpr int BPK = D * BITS / 8;    // code bytes per key
  const int tid = threadIdx.x;
  const int lk = tid & (LPK - 1);
  const int64_t key = (int64_t)blockIdx.x * KPB + tid / LPK;
  const int64_t n_keys = (int64_t)p.B * p.Hkv * p.T_new;
  const bool valid = key < n_keys;

  float x[8];
  if (valid) {
    load_key_lane<D, KF16>(p.keys, key, lk, x);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.0f;
  }
  float nrm;
  const uint32_t packed = encode_key_lane<D, BITS>(x, lk, p.signs, p.thresholds, nrm);

  if (!valid) return;
  const int64_t bh = key / p.T_new;
  const int64_t t = key - bh * p.T_new;
  const int b = (int)(bh / p.Hkv);
  const int64_t pos = (p.write_pos ? (int64_t)p.write_pos[b] : p.t0) + t;
  if (pos < 0 || pos >= p.T_cap) return;
  const int64_t row = bh * p.T_cap + pos;
  store_code_bits<BITS>(p.codes + row * BPK, lk, packed);
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
