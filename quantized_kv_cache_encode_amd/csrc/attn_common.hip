// Dispatch of the read-path kernels by head dimension.
#include "attn_qv.h"

namespace kvq {

extern template hipError_t run_hlm_decode<16>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_decode<32>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_decode<64>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_decode<128>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_decode<256>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_qv_decode<16>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_qv_decode<32>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_qv_decode<64>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_qv_decode<128>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_qv_decode<256>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<16>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<32>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<64>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<128>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_hlm_score<256>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_decode<16>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_decode<32>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_decode<64>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_decode<128>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_decode<256>(int, int, bool, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_score<16>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_score<32>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_score<64>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_score<128>(int, int, const AttnParams&, dim3, hipStream_t);
extern template hipError_t run_pot_score<256>(int, int, const AttnParams&, dim3, hipStream_t);

hipError_t launch_hlm_decode(int D, int bits, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 16: return run_hlm_decode<16>(bits, gg, v_f16, p, grid, s);
    case 32: return run_hlm_decode<32>(bits, gg, v_f16, p, grid, s);
    case 64: return run_hlm_decode<64>(bits, gg, v_f16, p, grid, s);
    case 128: return run_hlm_decode<128>(bits, gg, v_f16, p, grid, s);
    case 256: return run_hlm_decode<256>(bits, gg, v_f16, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_hlm_score(int D, int bits, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 16: return run_hlm_score<16>(bits, gg, p, grid, s);
    case 32: return run_hlm_score<32>(bits, gg, p, grid, s);
    case 64: return run_hlm_score<64>(bits, gg, p, grid, s);
    case 128: return run_hlm_score<128>(bits, gg, p, grid, s);
    case 256: return run_hlm_score<256>(bits, gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_hlm_decode_qv(int D, int bits, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 16: return run_qv_decode<16>(bits, gg, p, grid, s);
    case 32: return run_qv_decode<32>(bits, gg, p, grid, s);
    case 64: return run_qv_decode<64>(bits, gg, p, grid, s);
    case 128: return run_qv_decode<128>(bits, gg, p, grid, s);
    case 256: return run_qv_decode<256>(bits, gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_pot_decode(int D, int bits, int gg, bool v_f16, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 16: return run_pot_decode<16>(bits, gg, v_f16, p, grid, s);
    case 32: return run_pot_decode<32>(bits, gg, v_f16, p, grid, s);
    case 64: return run_pot_decode<64>(bits, gg, v_f16, p, grid, s);
    case 128: return run_pot_decode<128>(bits, gg, v_f16, p, grid, s);
    case 256: return run_pot_decode<256>(bits, gg, v_f16, p, grid, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_pot_score(int D, int bits, int gg, const AttnParams& p, dim3 grid, hipStream_t s) {
  switch (D) {
    case 16: return run_pot_score<16>(bits, gg, p, grid, s);
    case 32: return run_pot_score<32>(bits, gg, p, grid, s);
    case 64: return run_pot_score<64>(bits, gg, p, grid, s);
    case 128: return run_pot_score<128>(bits, gg, p, grid, s);
    case 256: return run_pot_score<256>(bits, gg, p, grid, s);
    default: return hipErrorNotSupported;
  }
}
}  // namespace kvq
