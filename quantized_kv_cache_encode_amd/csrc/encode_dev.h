// Per-key arithmetic of the Hadamard/Lloyd-Max write path, shared by the encode kernel and the fused
// append-and-attend path so that both produce identical codes.
//
// "AXELRAM: Quantize Once, Never Dequantize" (Key Points / Abstract): the key is rotated on write and
// each coordinate of the rotated unit vector is replaced by the index of its codebook cell.  Here
// y = H D k / ||k|| with H the normalised Sylvester Walsh-Hadamard matrix and D the sign pattern, and
// code_i = #{ j : t_j <= y_i } for the Lloyd-Max thresholds t of N(0, 1/d).
#pragma once

#include "kvq_device.h"

namespace kvq {

// One key is held by LPK = D/8 consecutive lanes (a power of two), 8 coordinates per lane: lane lk holds
// coordinates 8*lk .. 8*lk+7 in x.  All LPK lanes must call this together.  Returns the lane's 8*BITS code
// bits (coordinate 8*lk+j at bits [BITS*j, BITS*j+BITS)) and sets nrm = ||k|| in every lane of the key.
// `signs` is the bit mask of D (bit i set: coordinate i negated), `thresholds` the L-1 ascending cell
// boundaries of the codebook.
template <int D, int BITS>
__device__ __forceinline__ uint32_t encode_key_lane(float (&x)[8], int lk, const uint32_t* signs,
                                                    const float* thresholds, float& nrm) {
  constexpr int LPK = D / 8;
  constexpr int L = 1 << BITS;
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
#pragma unroll
  for (int o = 1; o < LPK; o <<= 1) ss += __shfl_xor(ss, o, 64);

  // sign pattern D for coordinates lk*8 .. lk*8+7
  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < (D + 31) / 32; ++k)
    if (((lk * 8) >> 5) == k) word = signs[k];
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

  nrm = __builtin_sqrtf(ss);
  const float inv = nrm > 0.0f ? 1.0f / (nrm * __builtin_sqrtf((float)D)) : 0.0f;
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float y = x[j] * inv;
    uint32_t c = 0;
#pragma unroll
    for (int t = 0; t < L - 1; ++t) c += (y >= thresholds[t]) ? 1u : 0u;
    packed |= c << (BITS * j);
  }
  return packed;
}

// Loads the 8 coordinates 8*lk .. 8*lk+7 of the key at `key` (fp16 or fp32, 16-byte aligned rows).
template <int D, bool KF16>
__device__ __forceinline__ void load_key_lane(const void* keys, int64_t key, int lk, float (&x)[8]) {
  if constexpr (KF16) {
    const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(keys) + key * D + lk * 8);
    const uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = h2f((uint16_t)(r[j] & 0xffffu));
      x[2 * j + 1] = h2f((uint16_t)(r[j] >> 16));
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(keys) + key * D + lk * 8);
    const float4 a = src[0], c = src[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
  }
}

// Stores a lane's 8*BITS code bits at its byte offset lk*BITS of the key's code row.
template <int BITS>
__device__ __forceinline__ void store_code_bits(uint8_t* row, int lk, uint32_t packed) {
  uint8_t* dst = row + lk * BITS;
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
}

}  // namespace kvq
