// Decode attention over quantized keys and values, head dimension 16.
#include "attn_qv.h"

namespace kvq {
template hipError_t run_qv_decode<16>(int, int, const AttnParams&, dim3, hipStream_t);
}  // namespace kvq
