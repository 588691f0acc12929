// noalloc.hip - fa_decode_noalloc: fa_decode with its workspace in a static
// device array, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable of the library's code object:
// every GPU the library runs on holds its own copy, at its own address, until
// the process ends.  Host code never passes the array's name to a kernel (in
// host code that name is a host-side stand-in, not a device address): the
// device address is looked up once per device with hipGetSymbolAddress and
// kept here, and only that address is used.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "fa.h"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(FA_NOALLOC_SCRATCH_MIB) << 20;
constexpr int kMaxDevices = 64;

}  // namespace

// The scratch array (one copy per GPU).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device).  Returns FA_OK and sets *out, or an error with fa_last_error text
// set by the caller's path.
fa_status_t scratch_ptr(void** out, char* why, size_t why_len) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(why, why_len, "hipGetDevice: %s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(why, why_len, "device %d outside [0, %d)", dev, kMaxDevices);
    return FA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(why, why_len, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
               hipGetErrorString(e));
      return FA_ERR_HIP;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return FA_OK;
}

}  // namespace

// Defined in fa_api.cpp (not exported): sets the calling thread's
// fa_last_error text.
extern "C" __attribute__((visibility("hidden"))) void fa_set_last_error(const char* text);

extern "C" {

fa_status_t fa_decode_noalloc(const fa_desc_t* desc, const void* q, const void* kx, const void* vx,
                              const void* ke, const void* ve, const float* ck, const float* cv,
                              float scale, float* out, void* stream) {
  size_t need = 0;
  fa_status_t st = fa_decode_workspace_size(desc, &need);
  if (st != FA_OK) return st;
  char why[256];
  if (need > kScratchBytes) {
    snprintf(why, sizeof why,
             "fa_decode_noalloc: this shape needs %zu workspace bytes, more than the %zu of the "
             "static scratch buffer (use fa_decode with a workspace)",
             need, kScratchBytes);
    fa_set_last_error(why);
    return FA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws, why, sizeof why)) != FA_OK) {
    fa_set_last_error(why);
    return st;
  }
  return fa_decode(desc, q, kx, vx, ke, ve, ck, cv, scale, out, ws, kScratchBytes, stream);
}

}  // extern "C"
