// Read-path kernels of the power-of-two codec for head dimension 256.
#include "attn_kernels.h"

namespace kvq {
template hipError_t run_pot_decode<256>(int, int, bool, const AttnParams&, dim3, hipStream_t);
template hipError_t run_pot_score<256>(int, int, const AttnParams&, dim3, hipStream_t);
}  // namespace kvq
