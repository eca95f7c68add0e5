// Decode attention over quantized keys and values, head dimension 64.
#include "attn_qv.h"

namespace kvq {
template hipError_t run_qv_decode<64>(int, int, const AttnParams&, dim3, hipStream_t);
}  // namespace kvq
