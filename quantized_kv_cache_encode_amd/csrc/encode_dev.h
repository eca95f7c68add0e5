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
// 16*lk .. 16*lk+15.  All LPK lanes must run the rotation together.  It leaves in x those coordinates of
// H' D k, where H' is the unnormalised Sylvester Walsh-Hadamard matrix, and returns ||k||^2 (the same in
// every lane of the key).  x holds the lane's coordinates on entry; sg are the lane's signs from lane_signs.
template <int D>
__device__ __forceinline__ float rotate_key_lane(float (&x)[kEncCpl], int lk, const float (&sg)[kEncCpl]) {
  // explicit fused multiply-adds: the sum is the same wherever this is inlined (a plain x*x + ss would
  // leave the compiler free to fuse differently in different callers)
  float ss = x[0] * x[0];
#pragma unroll
  for (int j = 1; j < kEncCpl; ++j) ss = __builtin_fmaf(x[j], x[j], ss);
  ss = key_lanes_sum<EncLanes<D>::LPK>(ss);
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
  constexpr int LPK = EncLanes<D>::LPK;
  if constexpr (LPK >= 2) stage(std::integral_constant<int, 1>{});
  if constexpr (LPK >= 4) stage(std::integral_constant<int, 2>{});
  if constexpr (LPK >= 8) stage(std::integral_constant<int, 4>{});
  if constexpr (LPK >= 16) stage(std::integral_constant<int, 8>{});
  return ss;
}

// The packed bits of 16 codes of value 2^(BITS-1), the code of y = 0: what a key with an infinite or NaN
// coordinate is given.
template <int BITS>
__device__ __forceinline__ uint64_t middle_codes() {
  uint64_t v = 0;
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) v |= (uint64_t)(1u << (BITS - 1)) << (BITS * j);
  return v;
}

// The lane's 16 coordinates as floats from their raw bits: packed fp16 halves in raw[0..7] (coordinate 2j
// in the low half of raw[j]), else fp32.
template <bool KF16>
__device__ __forceinline__ void key_lane_floats(const uint32_t (&raw)[kEncCpl], float (&x)[kEncCpl]) {
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j)
    x[j] = KF16 ? h2f((uint16_t)(raw[j / 2] >> (16 * (j % 2)))) : __builtin_bit_cast(float, raw[j]);
}

// From ||k||^2: the norm ||k|| (stored with the codes) and the factor 1 / (||k|| sqrt(d)) that scales H' D k
// to the rotated unit vector y.  Within [2^-100, 2^100] the hardware square root and reciprocal square root
// (within about one ulp) serve; outside it (a zero, tiny, huge or non-finite sum) the correctly rounded
// operations.  The factor is 0 for a zero or non-finite norm.
template <int D>
__device__ __forceinline__ float unit_scale_ss(float ss, float& nrm) {
  if (ss >= 0x1p-100f && ss <= 0x1p100f) {
    nrm = __builtin_amdgcn_sqrtf(ss);
    return __builtin_amdgcn_rsqf(ss * (float)D);
  }
  nrm = __builtin_sqrtf(ss);
  const float inv = 1.0f / (nrm * __builtin_sqrtf((float)D));
  return (nrm > 0.0f && inv > 0.0f && inv < INFINITY) ? inv : 0.0f;
}

// y = x * inv for the lane's coordinates.  For a key with a finite sum of squares every y is then finite with
// |y| <= 1 up to rounding (0 for a zero key).
__device__ __forceinline__ void unit_vector(float (&x)[kEncCpl], float inv) {
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) x[j] *= inv;
}

// code = #{ j : t_j <= y } by comparing with every threshold.
template <int BITS>
__device__ __forceinline__ uint32_t code_by_count(float y, const float* thresholds) {
  uint32_t c = 0;
#pragma unroll
  for (int t = 0; t < (1 << BITS) - 1; ++t) c += (y >= thresholds[t]) ? 1u : 0u;
  return c;
}

// The lane's 16*BITS code bits: coordinate 16*lk+j at bits [BITS*j, BITS*j+BITS), from y_j = y[j].
template <int BITS, class Q>
__device__ __forceinline__ uint64_t pack_lane_codes(const float (&y)[kEncCpl], Q&& code_of) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) {
    const uint32_t c = code_of(y[j]);
    const int bit = BITS * j;
    if (bit < 32) lo |= c << bit;
    if (bit + BITS > 32) hi |= bit >= 32 ? c << (bit - 32) : c >> (32 - bit);
  }
  return ((uint64_t)hi << 32) | lo;
}

// The rare keys whose fp32 sum of squares is not finite.  x holds the lane's coordinates as loaded (not
// rotated), ss the key's sum of squares, and all LPK lanes of the key call this together (their ss is the
// same).  A key with an infinite or NaN coordinate has no unit vector: it gets the code of y = 0 in every
// coordinate and the norm sqrt(ss), +inf or NaN.  Every other such key is finite and only its sum
// overflowed: it is rotated again from x scaled by 2^-100 (exact for every coordinate above 2^-26 of the
// largest, and the sum then lies well inside [2^-100, 2^100]); the norm is scaled back, which rounds to
// +inf where ||k|| itself exceeds the fp32 range.
template <int D, int BITS, class Q>
__device__ __forceinline__ uint64_t encode_beyond_range(float (&x)[kEncCpl], int lk, const float (&sg)[kEncCpl],
                                                        float ss, float& nrm, Q&& code_of) {
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) amax = fmaxf(amax, fabsf(x[j]));
  amax = key_lanes_max<EncLanes<D>::LPK>(amax);
  if (__builtin_isnan(ss) || !(amax <= 0x1.fffffep127f)) {
    nrm = __builtin_sqrtf(ss);
    return middle_codes<BITS>();
  }
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) x[j] *= 0x1p-100f;
  const float ss2 = rotate_key_lane<D>(x, lk, sg);
  float n2;
  const float inv = unit_scale_ss<D>(ss2, n2);
  nrm = n2 * 0x1p100f;
  unit_vector(x, inv);
  return pack_lane_codes<BITS>(x, code_of);
}

// Encode of one key with the per-threshold comparison (used where a single key is encoded).  Same lane
// layout and arithmetic as the encode kernel, whose table-driven cell search returns the same count.  raw
// holds the lane's 16 coordinates: packed fp16 halves in raw[0..7] (kf16), else fp32 bits.
template <int D, int BITS>
__device__ __forceinline__ uint64_t encode_key_lane(const uint32_t (&raw)[kEncCpl], bool kf16, int lk,
                                                    const uint32_t* signs, const float* thresholds, float& nrm) {
  float x[kEncCpl];
  if (kf16) key_lane_floats<true>(raw, x);
  else key_lane_floats<false>(raw, x);
  float sg[kEncCpl];
  lane_signs<D>(signs, lk, sg);
  const float ss = rotate_key_lane<D>(x, lk, sg);
  const float inv = unit_scale_ss<D>(ss, nrm);
  auto code_of = [&](float y) { return code_by_count<BITS>(y, thresholds); };
  if (!(ss <= 0x1.fffffep127f)) {  // an overflowed or non-finite sum: start again from the loaded coordinates
    if (kf16) key_lane_floats<true>(raw, x);
    else key_lane_floats<false>(raw, x);
    return encode_beyond_range<D, BITS>(x, lk, sg, ss, nrm, code_of);
  }
  unit_vector(x, inv);
  return pack_lane_codes<BITS>(x, code_of);
}

__device__ __forceinline__ int clamp_int(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Power-of-two codec (shift-accumulate attention page, English abstract): the lane's 16 elements of one key
// held on LPK = D/16 lanes (all of them must run this together).  alpha = max_i |k_i| over the whole key;
// element j gets the index of the magnitude nearest to |k_j| / alpha, counted as the midpoints m with
// |k_j| < t_m * alpha (a value on a midpoint takes the larger magnitude), and the sign bit k_j < 0 above
// it.  Returns the lane's 16*BITS packed bits (element 16*lk+j at bits [BITS*j, BITS*j+BITS)).  For fp16
// keys every comparison is exact in fp32 (alpha has 11 significant bits and a midpoint at most 3).
//
// The midpoints are canonical (the host checks): t_m = (3/4) 2^-m, or with the mantissa term (MANT)
// (7/8) 2^-i for m = 2i and (5/8) 2^-i for m = 2i+1.  So the limits are L 2^-k for L = fl(tau * alpha),
// tau = t_0 or t_1; for alpha in [2^-100, 2^100] every L 2^-k used is a normal float whose bit pattern is
// bits(L) - k 2^23, and a non-negative float (a NaN counting as above everything, as in a comparison) lies
// below a positive normal one exactly when its bit pattern does.  Hence #{k < K : a < L 2^-k} =
// clamp(ceil((bits(L) - bits(a)) / 2^23), 0, K): one subtraction, shift and clamp per family instead of
// one comparison per midpoint.  Other scales take the comparisons.
template <int D, int BITS, bool MANT>
__device__ __forceinline__ uint64_t pot_encode_lane(const float (&x)[kEncCpl], const float* thresholds, float& alpha) {
  constexpr int NM = 1 << (BITS - 1);  // magnitudes
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kEncCpl; ++j) amax = fmaxf(amax, fabsf(x[j]));
  alpha = key_lanes_max<EncLanes<D>::LPK>(amax);
  uint32_t lo = 0, hi = 0;
  auto put = [&](int j, uint32_t c) {
    const int bit = BITS * j;
    if (bit < 32) lo |= c << bit;
    if (bit + BITS > 32) hi |= bit >= 32 ? c << (bit - 32) : c >> (32 - bit);
  };
  if (alpha >= 0x1p-100f && alpha <= 0x1p100f) {
    constexpr int k1 = MANT ? NM / 2 : NM - 1;  // midpoints of the first family (t_0 2^-k), and of the second
    constexpr int k2 = MANT ? NM / 2 - 1 : 0;
    const int r1 = __builtin_bit_cast(int, thresholds[0] * alpha) + 0x7fffff;
    const int r2 = k2 > 0 ? __builtin_bit_cast(int, thresholds[k2 > 0 ? 1 : 0] * alpha) + 0x7fffff : 0;
#pragma unroll
    for (int j = 0; j < kEncCpl; ++j) {
      const int ba = __builtin_bit_cast(int, fabsf(x[j]));
      uint32_t c = (uint32_t)clamp_int((r1 - ba) >> 23, 0, k1);
      if constexpr (k2 > 0) c += (uint32_t)clamp_int((r2 - ba) >> 23, 0, k2);
      if (x[j] < 0.0f) c |= 1u << (BITS - 1);
      put(j, c);
    }
  } else {
    float lim[NM - 1];
#pragma unroll
    for (int m = 0; m < NM - 1; ++m) lim[m] = thresholds[m] * alpha;
#pragma unroll
    for (int j = 0; j < kEncCpl; ++j) {
      const float a = fabsf(x[j]);
      uint32_t c = 0;
#pragma unroll
      for (int m = 0; m < NM - 1; ++m) c += a < lim[m] ? 1u : 0u;
      if (x[j] < 0.0f) c |= 1u << (BITS - 1);
      put(j, c);
    }
  }
  return ((uint64_t)hi << 32) | lo;
}

// The keys [begin, end) of a launch's key array that one workgroup of 256 lanes encodes, KPB = 256/LPK per
// pass: the LPK lanes tid/LPK take key begin + pass*KPB + tid/LPK.  Each lane reads its 16 coordinates (32 or
// 64 contiguous bytes) through a buffer resource over the workgroup's own range, two passes ahead in two
// register sets, so two fetches stay in flight while a pass computes; a fetch past `end` reads zeros.
// step(k, raw, refill) gets the key index k and the lane's coordinates as raw bits (packed fp16 halves in
// raw[0..7], or fp32), and calls refill() once it no longer needs raw (which then starts the fetch two
// passes ahead into it).  In the last pair of passes some keys may be at or past `end` (their coordinates
// read as zeros): step must store nothing for k >= end.  Every lane of a key takes the same trip count, so
// cross-lane steps see all of them.
template <int D, bool KF16, class Step>
__device__ __forceinline__ void walk_keys(const void* keys, int64_t begin, int64_t end, int tid, Step&& step) {
  constexpr int LPK = EncLanes<D>::LPK;
  constexpr int KPB = 256 / LPK;
  constexpr int ESZ = KF16 ? 2 : 4;
  constexpr int NV = kEncCpl * ESZ / 16;  // 16-byte loads per lane and key
  const int lk = tid & (LPK - 1);
  const int n = (int)(end - begin);  // the host keeps n * D * ESZ below 2^31
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(keys) + begin * D * ESZ), 0, n * D * ESZ, 0x00020000);
  // The two register sets are kept as 16-byte vectors, the loads' own type, and the passes come in pairs
  // with no exit between them, so that each refill lands in the registers the next pass reads: as 32-bit
  // words, or with an exit between the passes, the compiler swapped the sets through register copies at
  // the loop's back edge, and a copy has to wait for every load in flight.
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  auto fetch = [&](int rel, u4 (&r)[NV]) {
    const int off = rel * D * ESZ + lk * kEncCpl * ESZ;
#pragma unroll
    for (int h = 0; h < NV; ++h) r[h] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + 16 * h, 0, 0);
  };
  u4 ra[NV], rb[NV];
  int rel = tid / LPK;
  fetch(rel, ra);
  __builtin_amdgcn_sched_barrier(0);  // ra's loads first: the loop's waits count on that order
  fetch(rel + KPB, rb);
  auto pass = [&](int r, u4 (&buf)[NV]) {
    uint32_t raw[kEncCpl];
#pragma unroll
    for (int j = 0; j < kEncCpl; ++j) raw[j] = j < 4 * NV ? buf[j / 4 < NV ? j / 4 : 0][j % 4] : 0u;
    step(begin + r, raw, [&] { fetch(r + 2 * KPB, buf); });
  };
  for (; rel < n; rel += 2 * KPB) {
    pass(rel, ra);
    pass(rel + KPB, rb);
  }
}

// The cache row of key gk (an index into [B*Hkv*T_new], below 2^31) of an encode launch with parameters p,
// or -1 where its position falls outside [0, T_cap): row = (b*Hkv + h)*T_cap + pos, with pos = t +
// write_pos[b] or t + t0.  Where the new keys fill whole rows the row is gk itself.
template <class P>
__device__ __forceinline__ int64_t encode_row(const P& p, uint32_t gk) {
  if (p.rows_whole) return gk;
  auto fdiv = [](uint32_t n, uint32_t magic, int shift) -> uint32_t { return (__umulhi(n, magic) + n) >> shift; };
  const uint32_t bh = fdiv(gk, p.tnew_magic, p.tnew_shift);
  const uint32_t t = gk - bh * (uint32_t)p.T_new;
  int64_t pos = (int64_t)t;
  if (p.write_pos) pos += p.write_pos[fdiv(bh, p.hkv_magic, p.hkv_shift)];
  else pos += p.t0;
  if (pos < 0 || pos >= p.T_cap) return -1;
  return (int64_t)bh * p.T_cap + pos;
}

// Keys per workgroup of the encode kernels: contiguous ranges of whole pairs of passes (walk_keys runs its
// passes in pairs, so a block of one pass would spend a second one on keys past its end), about 8192
// workgroups for large launches (a workgroup that streams its own range keeps the mix of key reads and code
// writes cheaper for the memory than passes strided over the whole array) and one pair each for small ones.
inline int64_t encode_keys_per_block(int64_t n_keys, int kpb) {
  const int64_t per = (n_keys + 8191) / 8192;
  return (per + 2 * kpb - 1) / (2 * kpb) * (2 * kpb);
}

// Stores a lane's 16*BITS code bits at its byte offset lk*2*BITS of the key's code row (code rows are
// whole multiples of 2*BITS bytes, so every store is naturally aligned).  NT: non-temporal stores, for the
// encode kernels' global code rows, which nothing reads back during the call (measured: the power-of-two
// encode 4 % faster at the batch-64 sweep shape, the Hadamard encode unchanged within noise).
template <int BITS, bool NT = false>
__device__ __forceinline__ void store_code_bits(uint8_t* row, int lk, uint64_t packed) {
  uint8_t* dst = row + lk * 2 * BITS;
  auto put = [](auto* ptr, auto v) {
    if constexpr (NT) __builtin_nontemporal_store(v, ptr);
    else *ptr = v;
  };
  if constexpr (BITS == 4) {
    typedef unsigned u2v __attribute__((ext_vector_type(2)));
    put(reinterpret_cast<u2v*>(dst), u2v{(uint32_t)packed, (uint32_t)(packed >> 32)});
  } else if constexpr (BITS == 2) {
    put(reinterpret_cast<uint32_t*>(dst), (uint32_t)packed);
  } else if constexpr (BITS == 1) {
    put(reinterpret_cast<uint16_t*>(dst), (uint16_t)packed);
  } else {
    uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
    put(d16, (uint16_t)packed);
    put(d16 + 1, (uint16_t)(packed >> 16));
    put(d16 + 2, (uint16_t)(packed >> 32));
  }
}

}  // namespace kvq
