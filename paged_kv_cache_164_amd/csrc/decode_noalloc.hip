// The static device scratch of pkv_paged_attention_decode_noalloc (pkv_abi.cpp), the decode call
// for callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array is this file's `scratch`.  Its host-side name is only a stand-in for the symbol: the
// device address comes from hipGetSymbolAddress, once per device (each device holds its own copy
// of the array, at its own address), and only that address is handed to the kernels.  The decode
// kernels need no initial contents in their workspace (the plan kernel writes the item count, the
// work items and the per-sequence counts before anything reads them), so nothing is cleared.
// Every call on a device shares that device's array: calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (looked up on the first call on the device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return pkv::record_error(PKV_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return pkv::record_error(PKV_ERR_UNSUPPORTED, "device index >= 64");
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return pkv::record_error(PKV_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                                hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return PKV_OK;
}

}  // namespace

namespace pkv {

// This device's copy of the scratch array (looked up on the first call on the device).
int noalloc_scratch_address(void** out) { return scratch_address(out); }

}  // namespace pkv
