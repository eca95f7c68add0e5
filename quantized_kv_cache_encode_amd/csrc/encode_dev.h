// Per-key arithmetic of the Hadamard/Lloyd-Max write path, shared by the encode kernel and the fused
// append-and-attend path so that both produce identical codes.
//
// "AXELRAM: Quantize Once, Never Dequantize" (Key Points / Abstract): the key is rotated on write and
// each coordinate of the rotated unit vector is replaced by the index of its codebook cell.  Here
// y = H D k / ||k|| with H the normalised Sylvester Walsh-Hadamard matrix and D the sign pattern, and
// code_i = #{ j : t_j <= y_i } for the Lloyd-Max thresholds t of N(0, 1/d).
#pragma once

#include <type_traits>

#include "kvq_device.h"

namespace kvq {

// x from the lane lk ^ DL of the same key (lanes of a key are consecutive, start at a multiple of their
// count and stay within one half of the wave).  ds_swizzle in bit-mask mode (and 0x1f, or 0, xor DL)
// permutes within each group of 32 lanes through the LDS crossbar without touching LDS memory, which keeps
// the permutation off the vector ALU that the rest of the encode keeps busy.
template <int DL>
__device__ __forceinline__ float xor_lane(float x) {
  static_assert(DL >= 1 && DL <= 16, "lane distance within 32 lanes");
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), (DL << 10) | 0x1f));
}

// Coordinates per lane of the write path: a key of D coordinates is held by D/16 consecutive lanes (one
// lane for D = 16), so the per-key work that every lane repeats (norm, scale, addresses) is shared by 16
// coordinates and four of the transform's stages stay in registers.
constexpr int kEncCpl = 16;

template <int D>
struct EncLanes {
  static_assert(D % kEncCpl == 0 && D / kEncCpl <= 16, "16 <= D <= 256");
  static constexpr int LPK = D / kEncCpl;  // lanes per key (a power of two)
};

// Sum of v over the LPK lanes of the key (the same value in all of them).
template <int LPK>
__device__ __forceinline__ float key_lanes_sum(float v) {
  if constexpr (LPK >= 2) v += xor_lane<1>(v);
  if constexpr (LPK >= 4) v += xor_lane<2>(v);
  if constexpr (LPK >= 8) v += xor_lane<4>(v);
  if constexpr (LPK >= 16) v += xor_lane<8>(v);
  return v;
}

// Maximum of v over the LPK lanes of the key (the same value in all of them).
template <int LPK>
__device__ __forceinline__ float key_lanes_max(float v) {
  if constexpr (LPK >= 2) v = fmaxf(v, xor_lane<1>(v));
  if constexpr (LPK >= 4) v = fmaxf(v, xor_lane<2>(v));
  if constexpr (LPK >= 8) v = fmaxf(v, xor_lane<4>(v));
  if constexpr (LPK >= 16) v = fmaxf(v, xor_lane<8>(v));
  return v;
}

// Sign of coordinate 16*lk + j under the pattern D (bit i of `signs` set: coordinate i negated), as +-1.
template <int D>
__device__ __forceinline__ void lane_signs(const uint32_t* signs, int lk, float (&sg)[kEncCpl]) {
  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < (D + 31) / 32; ++k)
    if (((lk * kEncCpl) >> 5) == k) word = signs[k];
  const uint32_t sb = (word >> ((lk * kEncCpl) & 31)) & 0xffffu;
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) sg[j] = ((sb >> j) & 1u) ? -1.0f : 1.0f;
}

// One key is held by LPK = D/16 consecutive lanes, 16 coordinates per lane: lane lk holds coordinates
// 16*lk .. 16*lk+15 in x.  All LPK lanes must run this together.  On return x holds those coordinates of
// H' D k, where H' is the unnormalised Sylvester Walsh-Hadamard matrix, and the result is ||k|| (the same
// in every lane of the key).  sg are the lane's signs from lane_signs.
template <int D>
__device__ __forceinline__ float rotate_key_lane(float (&x)[kEncCpl], int lk, const float (&sg)[kEncCpl]) {
  constexpr int LPK = EncLanes<D>::LPK;
  // explicit fused multiply-adds: the sum is the same wherever this is inlined (a plain x*x + ss would
  // leave the compiler free to fuse differently in different callers)
  float ss = x[0] * x[0];
#pragma unroll
  for (int j = 1; j < kEncCpl; ++j) ss = __builtin_fmaf(x[j], x[j], ss);
  ss = key_lanes_sum<LPK>(ss);
  // signs folded into the first butterflies: (s0 a + s1 c, s0 a - s1 c), each product exact
#pragma unroll
  for (int i = 0; i < kEncCpl; i += 2) {
    const float c = x[i + 1] * sg[i + 1];
    const float a = x[i];
    x[i] = __builtin_fmaf(a, sg[i], c);
    x[i + 1] = __builtin_fmaf(a, sg[i], -c);
  }
  // remaining in-register butterflies (coordinate distances 2, 4, 8)
#pragma unroll
  for (int h = 2; h < kEncCpl; h <<= 1)
#pragma unroll
    for (int i = 0; i < kEncCpl; ++i)
      if ((i & h) == 0) {
        const float a = x[i], c = x[i + h];
        x[i] = a + c;
        x[i + h] = a - c;
      }
  // cross-lane butterflies (coordinate distances 16, 32, ... = lane distances 1, 2, ...): the lower lane
  // of a pair keeps x + partner, the upper one partner - x, both as one fused multiply-add with +-1 (the
  // same sums and differences as the in-register stages)
  auto stage = [&](auto dl_tag) {
    constexpr int DL = decltype(dl_tag)::value;
    const float s = (lk & DL) ? -1.0f : 1.0f;
#pragma unroll
    for (int j = 0; j < kEncCpl; ++j) x[j] = __builtin_fmaf(x[j], s, xor_lane<DL>(x[j]));
  };
  if constexpr (LPK >= 2) stage(std::integral_constant<int, 1>{});
  if constexpr (LPK >= 4) stage(std::integral_constant<int, 2>{});
  if constexpr (LPK >= 8) stage(std::integral_constant<int, 4>{});
  if constexpr (LPK >= 16) stage(std::integral_constant<int, 8>{});
  return __builtin_sqrtf(ss);
}

// 1 / (||k|| sqrt(d)): scales H' D k to the rotated unit vector y; 0 for a zero key.
template <int D>
__device__ __forceinline__ float unit_scale(float nrm) {
  return nrm > 0.0f ? 1.0f / (nrm * __builtin_sqrtf((float)D)) : 0.0f;
}

// code = #{ j : t_j <= y } by comparing with every threshold.
template <int BITS>
__device__ __forceinline__ uint32_t code_by_count(float y, const float* thresholds) {
  uint32_t c = 0;
#pragma unroll
  for (int t = 0; t < (1 << BITS) - 1; ++t) c += (y >= thresholds[t]) ? 1u : 0u;
  return c;
}

// The lane's 16*BITS code bits: coordinate 16*lk+j at bits [BITS*j, BITS*j+BITS), y_j = x_j * inv.
template <int BITS, class Q>
__device__ __forceinline__ uint64_t pack_lane_codes(const float (&x)[kEncCpl], float inv, Q&& code_of) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) {
    const uint32_t c = code_of(x[j] * inv);
    const int bit = BITS * j;
    if (bit < 32) lo |= c << bit;
    if (bit + BITS > 32) hi |= bit >= 32 ? c << (bit - 32) : c >> (32 - bit);
  }
  return ((uint64_t)hi << 32) | lo;
}

// Encode of one key with the per-threshold comparison (used where a single key is encoded).  Same lane
// layout and arithmetic as the encode kernel, whose table-driven cell search returns the same count.
template <int D, int BITS>
__device__ __forceinline__ uint64_t encode_key_lane(float (&x)[kEncCpl], int lk, const uint32_t* signs,
                                                    const float* thresholds, float& nrm) {
  float sg[kEncCpl];
  lane_signs<D>(signs, lk, sg);
  nrm = rotate_key_lane<D>(x, lk, sg);
  const float inv = unit_scale<D>(nrm);
  return pack_lane_codes<BITS>(x, inv, [&](float y) { return code_by_count<BITS>(y, thresholds); });
}

// Power-of-two codec (shift-accumulate attention page, English abstract): the lane's 16 elements of one key
// held on LPK = D/16 lanes (all of them must run this together).  alpha = max_i |k_i| over the whole key;
// element j gets the index of the magnitude nearest to |k_j| / alpha, counted as the midpoints m with
// |k_j| < t_m * alpha (a value on a midpoint takes the larger magnitude), and the sign bit k_j < 0 above
// it.  Returns the lane's 16*BITS packed bits (element 16*lk+j at bits [BITS*j, BITS*j+BITS)).  For fp16
// keys every comparison is exact in fp32 (alpha has 11 significant bits and a midpoint at most 3).
template <int D, int BITS>
__device__ __forceinline__ uint64_t pot_encode_lane(const float (&x)[kEncCpl], const float* thresholds, float& alpha) {
  constexpr int NM = 1 << (BITS - 1);  // magnitudes
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) amax = fmaxf(amax, fabsf(x[j]));
  alpha = key_lanes_max<EncLanes<D>::LPK>(amax);
  float lim[NM - 1];
#pragma unroll
  for (int m = 0; m < NM - 1; ++m) lim[m] = thresholds[m] * alpha;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) {
    const float a = fabsf(x[j]);
    uint32_t c = 0;
#pragma unroll
    for (int m = 0; m < NM - 1; ++m) c += a < lim[m] ? 1u : 0u;
    if (x[j] < 0.0f) c |= 1u << (BITS - 1);
    const int bit = BITS * j;
    if (bit < 32) lo |= c << bit;
    if (bit + BITS > 32) hi |= bit >= 32 ? c << (bit - 32) : c >> (32 - bit);
  }
  return ((uint64_t)hi << 32) | lo;
}

// Loads the 16 coordinates 16*lk .. 16*lk+15 of the key at `key` (fp16 or fp32, 16-byte aligned rows).
template <int D, bool KF16>
__device__ __forceinline__ void load_key_lane(const void* keys, int64_t key, int lk, float (&x)[kEncCpl]) {
  if constexpr (KF16) {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(keys) + key * D + lk * kEncCpl);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 raw = src[h];
      const uint32_t r[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * h + 2 * j] = h2f((uint16_t)(r[j] & 0xffffu));
        x[8 * h + 2 * j + 1] = h2f((uint16_t)(r[j] >> 16));
      }
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(keys) + key * D + lk * kEncCpl);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 a = src[h];
      x[4 * h] = a.x; x[4 * h + 1] = a.y; x[4 * h + 2] = a.z; x[4 * h + 3] = a.w;
    }
  }
}

// Stores a lane's 16*BITS code bits at its byte offset lk*2*BITS of the key's code row (code rows are
// whole multiples of 2*BITS bytes, so every store is naturally aligned).
template <int BITS>
__device__ __forceinline__ void store_code_bits(uint8_t* row, int lk, uint64_t packed) {
  uint8_t* dst = row + lk * 2 * BITS;
  if constexpr (BITS == 4) {
    *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)packed, (uint32_t)(packed >> 32));
  } else if constexpr (BITS == 2) {
    *reinterpret_cast<uint32_t*>(dst) = (uint32_t)packed;
  } else if constexpr (BITS == 1) {
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
  } else {
    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
    d16[0] = (uint16_t)packed;
    d16[1] = (uint16_t)(packed >> 16);
    d16[2] = (uint16_t)(packed >> 32);
  }
}

}  // namespace kvq
