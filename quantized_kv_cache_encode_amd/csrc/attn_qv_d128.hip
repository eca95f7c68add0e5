// Decode attention over quantized keys and values, head dimension 128.
#include "attn_qv.h"

namespace kvq {
template hipError_t run_qv_decode<128>(int, int, const AttnParams&, dim3, hipStream_t);
}  // namespace kvq
