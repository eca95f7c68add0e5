// Device-side helpers for libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kvq {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Non-temporal cache policy for buffer loads (the aux operand of the raw buffer-load builtins).  The decode
// kernels use it for the cache they stream, where each byte is read once per call by a single load: the
// long-context decode step runs 6-9 % faster with it.  Loads whose windows overlap, the scores-only kernel,
// the small product-quantization launches and the encode keep the default policy (0), which measured as
// fast or faster there.
constexpr int kStreamLoad = 2;

template <int N> struct VecF;
template <> struct VecF<1> { typedef float type; };
template <> struct VecF<2> { typedef float2 type; };
template <> struct VecF<4> { typedef float4 type; };

template <int N> struct VecI;
template <> struct VecI<1> { typedef int type; };
template <> struct VecI<2> { typedef int2 type; };
template <> struct VecI<4> { typedef int4 type; };

__device__ __forceinline__ void set_from(float* acc, float e) { acc[0] = e; }
__device__ __forceinline__ void set_from(float* acc, float2 e) { acc[0] = e.x; acc[1] = e.y; }
__device__ __forceinline__ void set_from(float* acc, float4 e) { acc[0] = e.x; acc[1] = e.y; acc[2] = e.z; acc[3] = e.w; }
__device__ __forceinline__ void add_into(float* acc, float e) { acc[0] += e; }
__device__ __forceinline__ void add_into(float* acc, float2 e) { acc[0] += e.x; acc[1] += e.y; }
__device__ __forceinline__ void add_into(float* acc, float4 e) {
  acc[0] += e.x; acc[1] += e.y; acc[2] += e.z; acc[3] += e.w;
}

// Integer sums of table entries wrap modulo 2^32 (unsigned); the tables are scaled so that they never do.
__device__ __forceinline__ void set_from(uint32_t* acc, int e) { acc[0] = (uint32_t)e; }
__device__ __forceinline__ void set_from(uint32_t* acc, int2 e) { acc[0] = (uint32_t)e.x; acc[1] = (uint32_t)e.y; }
__device__ __forceinline__ void set_from(uint32_t* acc, int4 e) {
  acc[0] = (uint32_t)e.x; acc[1] = (uint32_t)e.y; acc[2] = (uint32_t)e.z; acc[3] = (uint32_t)e.w;
}
__device__ __forceinline__ void add_into(uint32_t* acc, int e) { acc[0] += (uint32_t)e; }
__device__ __forceinline__ void add_into(uint32_t* acc, int2 e) { acc[0] += (uint32_t)e.x; acc[1] += (uint32_t)e.y; }
__device__ __forceinline__ void add_into(uint32_t* acc, int4 e) {
  acc[0] += (uint32_t)e.x; acc[1] += (uint32_t)e.y; acc[2] += (uint32_t)e.z; acc[3] += (uint32_t)e.w;
}

// 2^e as a float, for -126 <= e <= 126 (exact).
__device__ __forceinline__ float pow2f(int e) { return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23); }

// Exponent of the fixed-point scale of one head's score table.  With A = sum_i |q'_i| and cmax the largest
// level magnitude, any sum of one entry per table row is at most A * cmax in magnitude; the scale 2^e with
// e = 29 - floor(log2(A * cmax)) keeps that below 2^30.  An entry is its fp32 value (relative error
// ~2^-23 per product and sum) rounded to an integer (at most 2^-(e+1) <= A * cmax * 2^-30 more), so a
// score's error stays orders of magnitude below 1e-4 |q| |k|.  For A * cmax = 0 or below the normal
// range e is clamped to 126 (the entries are then 0 or rounded to 0); for infinite or NaN A the table is
// meaningless, as the query is.
__device__ __forceinline__ int fix_exp(float a, float cmax) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, a * cmax);
  const int k = (int)((bits >> 23) & 0xffu) - 127;
  const int e = 29 - k;
  return e < -126 ? -126 : (e > 126 ? 126 : e);
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not wait for this wave's outstanding global-memory loads, so prefetches
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's LDS writes before its later LDS reads (data exchanged
// between lanes of one wave through LDS).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Value of x in another lane of the same row of 16, selected by a DPP control word.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMir = 0x141;  // row_half_mirror: lane i <- 7-i within 8
constexpr int kDppMirror = 0x140;   // row_mirror: lane i <- 15-i within 16

// Wave-wide reductions: within each row of 16 lanes through DPP moves, then across the four rows through
// lanes 0, 16, 32, 48.  The result is the same in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppSwap1>(x));
  x = fmaxf(x, dpp_f<kDppSwap2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMir>(x));
  x = fmaxf(x, dpp_f<kDppMirror>(x));
  const int xi = __builtin_bit_cast(int, x);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<kDppSwap1>(x);
  x += dpp_f<kDppSwap2>(x);
  x += dpp_f<kDppHalfMir>(x);
  x += dpp_f<kDppMirror>(x);
  const int xi = __builtin_bit_cast(int, x);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return (a + b) + (c + d);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Load the N-byte code row at p (p aligned to the largest power of two <= 16
// dividing N) into 32-bit words, little-endian.
template <int N>
__device__ __forceinline__ void load_code_row(const uint8_t* __restrict__ p, uint32_t (&w)[(N + 3) / 4]) {
  if constexpr (N % 16 == 0) {
#pragma unroll
    for (int k = 0; k < N / 16; ++k) {
      uint4 x = reinterpret_cast<const uint4*>(p)[k];
      w[4 * k + 0] = x.x; w[4 * k + 1] = x.y; w[4 * k + 2] = x.z; w[4 * k + 3] = x.w;
    }
  } else if constexpr (N % 8 == 0) {
#pragma unroll
    for (int k = 0; k < N / 8; ++k) {
      uint2 x = reinterpret_cast<const uint2*>(p)[k];
      w[2 * k + 0] = x.x; w[2 * k + 1] = x.y;
    }
  } else if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k) w[k] = reinterpret_cast<const uint32_t*>(p)[k];
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int k = 0; k < (N + 3) / 4; ++k) w[k] = 0;
#pragma unroll
    for (int k = 0; k < N / 2; ++k) w[k / 2] |= (uint32_t)reinterpret_cast<const uint16_t*>(p)[k] << (16 * (k % 2));
  } else {
#pragma unroll
    for (int k = 0; k < (N + 3) / 4; ++k) w[k] = 0;
#pragma unroll
    for (int k = 0; k < N; ++k) w[k / 4] |= (uint32_t)p[k] << (8 * (k % 4));
  }
}

// Bits [I*B, I*B+B) of a little-endian word array (I, B compile-time).
template <int I, int B, int NW>
__device__ __forceinline__ uint32_t bit_field(const uint32_t (&w)[NW]) {
  constexpr int bit = I * B;
  constexpr int word = bit / 32;
  constexpr int off = bit % 32;
  constexpr uint32_t mask = (1u << B) - 1u;
  if constexpr (off + B <= 32) {
    return (w[word] >> off) & mask;
  } else {
    return ((w[word] >> off) | (w[word + 1] << (32 - off))) & mask;
  }
}

// fp16 <-> fp32 helpers on raw bits.
__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

}  // namespace kvq
