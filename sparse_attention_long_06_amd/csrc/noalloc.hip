// dsa_decode_noalloc: dsa_decode for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its workspace is a fixed static device array, one per
// GPU for the life of the process, instead of caller-provided memory.
//
// In host code `scratch` names a host-side stand-in of the array, not its
// device address: the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that pointer is
// handed to the kernels.
#include <mutex>

#include "dsa.h"
#include "dsa_kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;   // DSA_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

thread_local char g_msg[256];

// Device address of this device's `scratch`, looked up on the first call made
// with the device current.  Returns nullptr and fills g_msg on failure.
void* scratch_ptr() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    snprintf(g_msg, sizeof g_msg, "dsa_decode_noalloc: no usable current device (%s, device %d)",
             hipGetErrorString(e), dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(g_msg, sizeof g_msg, "dsa_decode_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
               hipGetErrorString(e));
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

// Set by api.hip: records a message for dsa_last_error() and returns the status.
dsa_status dsa_record_error(dsa_status s, const char* msg);

extern "C" size_t dsa_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" dsa_status dsa_decode_noalloc(const dsa_batch* batch, const uint8_t* q8, const float* q_scale,
                                         const float* w, const dsa_cache* kidx, const dsa_cache* kscale, int H_I,
                                         int d_I, int k, const uint16_t* q, const dsa_cache* kv,
                                         const dsa_cache* v, int H, int D, int D_v, float scale, uint16_t* out,
                                         float* lse, int32_t* idx_out, void* stream) {
  const size_t need = dsa_workspace_size(DSA_WS_DECODE, batch, k, H, D_v);
  if (need == (size_t)-1) {
    // invalid geometry or sizes: dsa_decode reports which
    return dsa_decode(batch, q8, q_scale, w, kidx, kscale, H_I, d_I, k, q, kv, v, H, D, D_v, scale, out, lse,
                      idx_out, nullptr, 0, stream);
  }
  if (need > kScratchBytes) {
    snprintf(g_msg, sizeof g_msg,
             "dsa_decode_noalloc: this batch needs %zu workspace bytes, more than the %zu-byte static scratch "
             "(use dsa_decode with a caller-provided workspace)", need, kScratchBytes);
    return dsa_record_error(DSA_ERR_WORKSPACE, g_msg);
  }
  void* ws = scratch_ptr();
  if (!ws) return dsa_record_error(DSA_ERR_HIP, g_msg);
  return dsa_decode(batch, q8, q_scale, w, kidx, kscale, H_I, d_I, k, q, kv, v, H, D, D_v, scale, out, lse,
                    idx_out, ws, kScratchBytes, stream);
}
