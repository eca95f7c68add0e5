// Write path of the power-of-two codec (shift-accumulate attention page, English abstract: the key cache
// holds a signed power-of-two code per element, so that every product in q.k becomes a sign flip and a
// shift, with an optional sub-power mantissa term).
//
// For every key k: alpha = max_i |k_i|; element i gets the index j of the magnitude nearest to |k_i| / alpha
// in the codebook's descending set (|k_i| < t_m * alpha for exactly j of the midpoints t_m; a value on a
// midpoint takes the larger magnitude) and the sign bit k_i < 0 above it; codes are packed LSB-first next
// to alpha in the norms buffer.  No rotation.
//
// Layout: 16 elements per lane, D/16 lanes per key (a wave holds 64/(D/16) keys), and each workgroup
// streams a contiguous range of keys; alpha is reduced across
// the key's lanes; each lane packs its 16*b bits and stores them at its own byte offset of the key's row.  For
// fp16 keys every comparison is exact in fp32 (alpha has 11 significant bits and a midpoint at most 3).
#include "encode_dev.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

template <int D, int BITS, bool KF16, bool MANT>
__global__ __launch_bounds__(256) void pot_encode_kernel(const EncodeParams p) {
  constexpr int LPK = EncLanes<D>::LPK;  // lanes per key
  constexpr int BPK = D * BITS / 8;
  const int lk = threadIdx.x & (LPK - 1);
  const int64_t n_keys = p.key_end - p.key_begin;
  const int64_t kb = (int64_t)blockIdx.x * p.keys_per_block;
  const int64_t ke = kb + p.keys_per_block < n_keys ? kb + p.keys_per_block : n_keys;
  const void* keys = reinterpret_cast<const char*>(p.keys) + p.key_begin * D * (KF16 ? 2 : 4);
  walk_keys<D, KF16>(keys, kb, ke, threadIdx.x, [&](int64_t k, uint32_t (&raw)[kEncCpl], auto&& refill) {
    float x[kEncCpl];
    key_lane_floats<KF16>(raw, x);
    refill();
    float alpha;
    const uint64_t packed = pot_encode_lane<D, BITS, MANT>(x, p.thresholds, alpha);
    if (k >= ke) return;  // past the workgroup's keys (the last pair of passes)
    const int64_t row = encode_row(p, (uint32_t)(p.key_begin + k));
    if (row < 0) return;
    store_code_bits<BITS, true>(p.codes + row * BPK, lk, packed);
    if (lk == 0) p.norms[row] = alpha;
  });
}

template <int D, int BITS>
static hipError_t pot_launch(bool kf16, const EncodeParams& p0, hipStream_t s) {
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
    if (kf16 && p.pot_mant) hipLaunchKernelGGL((pot_encode_kernel<D, BITS, true, true>), grid, dim3(256), 0, s, p);
    else if (kf16) hipLaunchKernelGGL((pot_encode_kernel<D, BITS, true, false>), grid, dim3(256), 0, s, p);
    else if (p.pot_mant) hipLaunchKernelGGL((pot_encode_kernel<D, BITS, false, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((pot_encode_kernel<D, BITS, false, false>), grid, dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
static hipError_t pot_d(int bits, bool kf16, const EncodeParams& p, hipStream_t s) {
  switch (bits) {
    case 2: return pot_launch<D, 2>(kf16, p, s);
    case 3: return pot_launch<D, 3>(kf16, p, s);
    case 4: return pot_launch<D, 4>(kf16, p, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_pot_encode(int D, int bits, bool k_f16, const EncodeParams& p, hipStream_t s) {
  switch (D) {
    case 16: return pot_d<16>(bits, k_f16, p, s);
    case 32: return pot_d<32>(bits, k_f16, p, s);
    case 64: return pot_d<64>(bits, k_f16, p, s);
    case 128: return pot_d<128>(bits, k_f16, p, s);
    case 256: return pot_d<256>(bits, k_f16, p, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace kvq
