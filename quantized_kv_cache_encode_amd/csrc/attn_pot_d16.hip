// Read-path kernels of the power-of-two codec for head dimension 16.
#include "attn_kernels.h"

namespace kvq {
template hipError_t run_pot_decode<16>(int, int, bool, const AttnParams&, dim3, hipStream_t);
template hipError_t run_pot_score<16>(int, int, const AttnParams&, dim3, hipStream_t);
}  // namespace kvq
