// Write path of the Hadamard/Lloyd-Max codec ("AXELRAM: Quantize Once, Never
// Dequantize", Key Points / Abstract: transform on write, store indices of a
// codebook fixed by d and b).
//
// For every key k: n = ||k||, y = H D k / n with H the normalised Sylvester
// Walsh-Hadamard matrix and D the sign pattern, code_i = #{ j : t_j <= y_i },
// codes packed LSB-first (b bits per coordinate) next to the fp32 norm.
//
// Layout: 16 coordinates per lane, D/16 lanes per key, so a wave holds
// 64/(D/16) keys.  The key is read with two 16-byte loads per lane (fp16) and
// fully coalesced across the wave; each workgroup streams a contiguous range
// of keys.  The transform is an in-register radix-2 fast Walsh-Hadamard
// transform for the lane's 16 coordinates followed by log2(D/16) cross-lane
// butterfly stages; ||k||^2 is reduced across the same lanes.  Each lane then finds the codes
// of its 16 coordinates in a cell table, packs 16*b bits and stores them at
// its own byte offset of the key's row.
#include "encode_dev.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// WHOLE: the new keys fill whole cache rows (p.rows_whole), so key i of the launch goes to row i.
template <int D, int BITS, bool KF16, bool WHOLE>
// amdgpu_waves_per_eu(5): at most 96 registers, five waves per SIMD (the kernel needs no more; with 97 the
// compiler's own choice left four per SIMD, measured 4 % slower).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void hlm_encode_kernel(const EncodeParams p) {
  constexpr int LPK = EncLanes<D>::LPK;  // lanes per key
  constexpr int BPK = D * BITS / 8;    // code bytes per key
  constexpr int L = 1 << BITS;
  constexpr int ESZ = KF16 ? 2 : 4;
  // per cell, 8 bytes apart: the threshold inside the cell (or +inf) and the count of thresholds below it
  __shared__ float2 cells[kEncodeMaxCells];

  // cell table: the count of thresholds in lower cells and the one threshold (if any) inside the cell
  for (int c = threadIdx.x; c < p.n_cells; c += 256) {
    int below = 0;
    float inside = INFINITY;
#pragma unroll
    for (int j = 0; j < L - 1; ++j) {
      const int cj = (int)floorf(__builtin_fmaf(p.thresholds[j], p.cell_inv, p.cell_shift));
      below += cj < c ? 1 : 0;
      if (cj == c) inside = p.thresholds[j];
    }
    cells[c] = make_float2(inside, __builtin_bit_cast(float, below));
  }
  __syncthreads();

  const int tid = threadIdx.x;
  const int lk = tid & (LPK - 1);
  float sg[kEncCpl];
  lane_signs<D>(p.signs, lk, sg);
  // The cell's byte offset in the table comes straight from the bits of v = y * cell_inv + cell_shift + 2^20.
  // In [2^20, 2^21) the spacing of floats is 1/8, so the mantissa holds 8 v rounded to the nearest eighth,
  // and masking off its low three bits leaves 8 * cell.  The rounding moves v by at most 1/16 of a cell, and
  // every threshold sits at least 7% of a cell inside its cell (choose_encode_cells), so where it moves v
  // into the neighbouring cell no threshold lies in between and the count is the same.  The shift is a
  // multiple of 1/8 below 2^18, so cell_shift + 2^20 is exact and the fma's single rounding is the only
  // one.  y is finite with |y| <= 1 up to rounding (keys with a non-finite coordinate do not get here), and
  // the cells span |y| <= 1.0001 with a spare cell at either end, so v is positive and the cell is in range
  // without a clamp.
  const float shift20 = p.cell_shift + 0x1p20f;
  auto code_of = [&](float y) -> uint32_t {
    const uint32_t off = __builtin_bit_cast(uint32_t, __builtin_fmaf(y, p.cell_inv, shift20)) & 0x7ffff8u;
    const float2 e = *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(cells) + off);
    return (uint32_t)__builtin_bit_cast(int, e.y) + (y >= e.x ? 1u : 0u);
  };
  const int64_t n_keys = p.key_end - p.key_begin;
  const int64_t kb = (int64_t)blockIdx.x * p.keys_per_block;
  const int64_t ke = kb + p.keys_per_block < n_keys ? kb + p.keys_per_block : n_keys;
  const void* keys = reinterpret_cast<const char*>(p.keys) + p.key_begin * D * ESZ;
  walk_keys<D, KF16>(keys, kb, ke, tid, [&](int64_t k, uint32_t (&raw)[kEncCpl], auto&& refill) {
    float x[kEncCpl];
    key_lane_floats<KF16>(raw, x);
    // the coordinates are converted here, so that raw is free and the loads two passes ahead go out now (left
    // alone, the compiler reads raw's fp16 halves in later mixed-precision FMAs, and the later refill measured
    // slower)
#pragma unroll
    for (int j = 0; j < kEncCpl; ++j) asm volatile("" : "+v"(x[j]));
    refill();
    const float ss = rotate_key_lane<D>(x, lk, sg);
    float nrm;
    const float inv = unit_scale_ss<D>(ss, nrm);
    uint64_t packed;
    if (ss <= 0x1.fffffep127f) {  // every finite key whose sum of squares stays in range
      unit_vector(x, inv);
      packed = pack_lane_codes<BITS>(x, code_of);
    } else {  // rare: the sum overflowed, or a coordinate is infinite or NaN; the key is read again
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(keys) +
                                                        (k * D + lk * kEncCpl) * ESZ);
      uint32_t r2[kEncCpl];
#pragma unroll
      for (int h = 0; h < kEncCpl * ESZ / 16; ++h) {
        const uint4 v = src[h];
        r2[4 * h + 0] = v.x; r2[4 * h + 1] = v.y; r2[4 * h + 2] = v.z; r2[4 * h + 3] = v.w;
      }
      key_lane_floats<KF16>(r2, x);
      packed = encode_beyond_range<D, BITS>(x, lk, sg, ss, nrm, code_of);
    }

    if (k >= ke) return;  // past the workgroup's keys (the last pair of passes)
    const int64_t row = WHOLE ? p.key_begin + k : encode_row(p, (uint32_t)(p.key_begin + k));
    if (row < 0) return;
    store_code_bits<BITS, true>(p.codes + row * BPK, lk, packed);
    if (lk == 0) p.norms[row] = nrm;
  });
}

template <int D, int BITS>
static hipError_t encode_launch(bool kf16, const EncodeParams& p0, hipStream_t s) {
  constexpr int KPB = 256 / EncLanes<D>::LPK;
  const int64_t n_keys = (int64_t)p0.B * p0.Hkv * p0.T_new;
  // launches of at most 2^30 key bytes each (key indices stay below 2^31); each workgroup encodes a
  // contiguous range of keys
  const int64_t per_launch = ((int64_t)1 << 30) / (D * (kf16 ? 2 : 4));
  for (int64_t k0 = 0; k0 < n_keys; k0 += per_launch) {
    EncodeParams p = p0;
    p.key_begin = k0;
    p.key_end = k0 + per_launch < n_keys ? k0 + per_launch : n_keys;
    p.keys_per_block = encode_keys_per_block(p.key_end - p.key_begin, KPB);
    const dim3 grid((unsigned)((p.key_end - p.key_begin + p.keys_per_block - 1) / p.keys_per_block));
    if (p.rows_whole) {
      if (kf16) hipLaunchKernelGGL((hlm_encode_kernel<D, BITS, true, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((hlm_encode_kernel<D, BITS, false, true>), grid, dim3(256), 0, s, p);
    } else {
      if (kf16) hipLaunchKernelGGL((hlm_encode_kernel<D, BITS, true, false>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((hlm_encode_kernel<D, BITS, false, false>), grid, dim3(256), 0, s, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
