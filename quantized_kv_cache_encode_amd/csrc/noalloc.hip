// Decode attention that allocates nothing: the split partials and arrival counters that
// kvq_decode_attn keeps in a caller workspace live here in one library-owned device array.
#include <cstdio>
#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

constexpr size_t kScratchBytes = KVQ_NOALLOC_SCRATCH_BYTES;  // 4 MiB

// One copy per device, zero at load (static storage); each device holds it until the process ends.  Host
// code never passes this name to a kernel: there it names a host-side shadow, not the device address.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // per device: the address of its copy of `scratch`, once set up

// Set-up on first use of a device (that device current): look up the array's device address and clear
// it, on the caller's stream, with the fill kernel.  Every completed decode leaves its arrival counters
// at zero again, so later calls need no clearing.
kvq_status scratch_of_current_device(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return (kvq_status)kvq::set_error(KVQ_ERR_DEVICE, "kvq_decode_attn_noalloc: no usable current device");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      char msg[256];
      snprintf(msg, sizeof msg, "kvq_decode_attn_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s",
               dev, hipGetErrorString(e));
      return (kvq_status)kvq::set_error(KVQ_ERR_DEVICE, msg);
    }
    const hipError_t z = kvq::launch_zero_words(static_cast<uint32_t*>(ptr), kScratchBytes / 4, s);
    if (z != hipSuccess) {
      char msg[256];
      snprintf(msg, sizeof msg, "kvq_decode_attn_noalloc: clearing the scratch array failed: %s", hipGetErrorString(z));
      return (kvq_status)kvq::set_error(KVQ_ERR_DEVICE, msg);
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return KVQ_OK;
}

}  // namespace

extern "C" kvq_status kvq_decode_attn_noalloc(const kvq_codebook* cb, const int8_t* signs, const void* q,
                                              kvq_dtype qdtype, const uint8_t* codes, const float* norms,
                                              const void* v, kvq_dtype vdtype, int B, int Hq, int Hkv,
                                              int64_t T_cap, const int32_t* seq_lens, float scale, void* out,
                                              kvq_dtype odtype, int n_splits, void* stream) {
  if (!cb) return (kvq_status)kvq::set_error(KVQ_ERR_INVALID_ARG, "codebook is NULL");
  const size_t need = kvq_decode_attn_workspace(cb, B, Hq, Hkv, T_cap, n_splits);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "kvq_decode_attn_noalloc: this shape needs %zu bytes of split partials, more than the library's "
             "%zu-byte scratch array (use kvq_decode_attn with a workspace, or fewer splits)",
             need, kScratchBytes);
    return (kvq_status)kvq::set_error(KVQ_ERR_WORKSPACE, msg);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const kvq_status st = scratch_of_current_device(s, &ws);
  if (st != KVQ_OK) return st;
  return kvq_decode_attn(cb, signs, q, qdtype, codes, norms, v, vdtype, B, Hq, Hkv, T_cap, seq_lens, scale, out,
                         odtype, ws, kScratchBytes, n_splits, stream);
}
