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
// fully coalesced across the wave.  The transform is an in-register radix-2
// fast Walsh-Hadamard transform for the lane's 16 coordinates followed by
// log2(D/16) cross-lane butterfly stages; ||k||^2 is reduced across the same
// lanes.  Each lane then finds the codes of its 16 coordinates, packs 16*b
// bits and stores them at its own byte offset of the key's row.
#include "encode_dev.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

template <int D, int BITS, bool KF16>
__global__ __launch_bounds__(256) void hlm_encode_kernel(const EncodeParams p) {
  constexpr int LPK = EncLanes<D>::LPK;  // lanes per key
  constexpr int KPB = 256 / LPK;       // keys per workgroup per pass
  constexpr int BPK = D * BITS / 8;    // code bytes per key
  constexpr int L = 1 << BITS;
  constexpr int ESZ = KF16 ? 2 : 4;
  __shared__ float2 cells[kEncodeMaxCells];  // (threshold inside the cell or +inf, count below the cell)

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
  const int64_t n_keys = p.key_end - p.key_begin;
  const int64_t stride = (int64_t)gridDim.x * KPB;
  // keys through a buffer resource (byte offsets < 2^31, which the host ensures per launch): a fetch past
  // the launch's last key reads zeros, so the two-deep prefetch needs no guard
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(reinterpret_cast<const char*>(p.keys) + p.key_begin * D * ESZ),
                                        0, (int)(n_keys * D * ESZ), 0x00020000);
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  constexpr int NV = kEncCpl * ESZ / 16;  // 16-byte loads per lane and key
  struct Raw { u4 v[NV]; };
  auto fetch = [&](int64_t key) {
    Raw r;
    const int off = (int)(key < n_keys ? key : n_keys) * D * ESZ + lk * kEncCpl * ESZ;
#pragma unroll
    for (int h = 0; h < NV; ++h) r.v[h] = __builtin_amdgcn_raw_buffer_load_b128(rk, off + 16 * h, 0, 0);
    return r;
  };
  const float cell_max = (float)(p.n_cells - 1);
  auto code_of = [&](float y) -> uint32_t {
    // cell_shift keeps the argument positive for |y| <= 1, so truncation is the floor; the clamp guards
    // the table against anything else (a NaN lands in cell 0)
    const int c = (int)__builtin_amdgcn_fmed3f(__builtin_fmaf(y, p.cell_inv, p.cell_shift), 0.0f, cell_max);
    const float2 e = cells[c];
    return (uint32_t)__builtin_bit_cast(int, e.y) + (y >= e.x ? 1u : 0u);
  };

  auto fdiv = [](uint32_t n, uint32_t magic, int shift) -> uint32_t {
    return (__umulhi(n, magic) + n) >> shift;
  };
  // One key: convert its coordinates, put the fetch two passes ahead into the registers just freed (so two
  // fetches stay in flight), transform, quantize, store.  The loop alternates two register sets.
  auto step = [&](int64_t k, Raw& r) {
    float x[kEncCpl];
#pragma unroll
    for (int h = 0; h < NV; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // the vector elements go through named scalars: bit-casting an element expression directly
        // read element 0 for every j with this compiler
        const uint32_t w = r.v[h][j];
        if constexpr (KF16) {
          x[8 * h + 2 * j] = h2f((uint16_t)(w & 0xffffu));
          x[8 * h + 2 * j + 1] = h2f((uint16_t)(w >> 16));
        } else {
          x[4 * h + j] = __builtin_bit_cast(float, w);
        }
      }
    r = fetch(k + 2 * stride);
    const float nrm = rotate_key_lane<D>(x, lk, sg);
    const uint64_t packed = pack_lane_codes<BITS>(x, unit_scale<D>(nrm), code_of);

    const uint32_t gk = (uint32_t)(p.key_begin + k);  // key index in [B*Hkv*T_new] (< 2^31)
    const uint32_t bh = fdiv(gk, p.tnew_magic, p.tnew_shift);
    const uint32_t t = gk - bh * (uint32_t)p.T_new;
    int64_t pos = (int64_t)t;
    if (p.write_pos) pos += p.write_pos[fdiv(bh, p.hkv_magic, p.hkv_shift)];
    else pos += p.t0;
    if (pos < 0 || pos >= p.T_cap) return;
    const int64_t row = (int64_t)bh * p.T_cap + pos;
    store_code_bits<BITS>(p.codes + row * BPK, lk, packed);
    if (lk == 0) p.norms[row] = nrm;
  };

  int64_t key = (int64_t)blockIdx.x * KPB + tid / LPK;
  Raw ra = fetch(key), rb = fetch(key + stride);
  for (; key < n_keys; key += 2 * stride) {
    step(key, ra);
    if (key + stride >= n_keys) break;
    step(key + stride, rb);
  }
}

template <int D, int BITS>
static hipError_t encode_launch(bool kf16, const EncodeParams& p0, hipStream_t s) {
  constexpr int KPB = 256 / EncLanes<D>::LPK;
  const int64_t n_keys = (int64_t)p0.B * p0.Hkv * p0.T_new;
  // launches of at most 2^30 key bytes each (32-bit buffer offsets); a persistent grid of at most 2048
  // workgroups (eight per compute unit) walks the keys of a launch
  const int64_t per_launch = ((int64_t)1 << 30) / (D * (kf16 ? 2 : 4));
  for (int64_t k0 = 0; k0 < n_keys; k0 += per_launch) {
    EncodeParams p = p0;
    p.key_begin = k0;
    p.key_end = k0 + per_launch < n_keys ? k0 + per_launch : n_keys;
    const int64_t blocks = (p.key_end - p.key_begin + KPB - 1) / KPB;
    const dim3 grid((unsigned)(blocks < 2048 ? blocks : 2048));
    if (kf16) hipLaunchKernelGGL((hlm_encode_kernel<D, BITS, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((hlm_encode_kernel<D, BITS, false>), grid, dim3(256), 0, s, p);
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
