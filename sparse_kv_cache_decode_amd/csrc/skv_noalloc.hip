// The decode step for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
// kernels as skv_decode_step, with the step's transient scratch (logits, LSE
// partials, selection lists, attention partials) in this file's static device
// array instead of the handle's own region.
//
// The array's address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept; host code only ever passes that address to the
// kernels, never the array's name, which in host code is a stand-in and not a
// device address.  Every call on one device shares that device's array and
// nothing in it has to start at zero (each step writes every part it reads), so
// calls that overlap on one device race on it.
#include <mutex>
#include <vector>

#include "skv_internal.h"

namespace {

__device__ __align__(256) char scratch[SKV_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
std::vector<char*> g_addr;   // by device ordinal; nullptr until looked up

// The device address of this device's copy of `scratch` (looked up on first use).
hipError_t scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_addr.size() <= dev) g_addr.resize(dev + 1, nullptr);
  if (!g_addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = static_cast<char*>(ptr);
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" skv_status skv_decode_step_noalloc(skv_layer* h, const uint16_t* q, float* out, int32_t* chunk_ids,
                                              void* stream) {
  if (!h) return SKV_ERR_INVALID_ARG;
  if (skv::transient_bytes(h) > (size_t)SKV_NOALLOC_SCRATCH_BYTES) return SKV_ERR_SCRATCH;
  char* xs = nullptr;
  if (scratch_address(&xs) != hipSuccess) {
    (void)hipGetLastError();
    return SKV_ERR_HIP;
  }
  return skv::decode_enqueue(h, q, out, chunk_ids, stream, xs);
}
