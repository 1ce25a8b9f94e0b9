// The allocation-free vocabulary argmax: dflash_lm_head_argmax with its per-work-group
// (value, index) keys in a fixed device array of this library instead of the context's
// workspace, for callers that cannot allocate device memory at the call (code under HIP
// graph capture, tight serving loops, harnesses that forbid it).
//
// The array is a file-scope __device__ variable. In host code its name stands for a host
// shadow, not a device address, so host code never passes it to a kernel: at context
// creation, with the context's device current, the runtime asks for the device address of
// that device's copy (hipGetSymbolAddress) once per device and keeps it, and the entry point
// hands that address to the argmax launches. Each GPU holds its own copy of the array until
// the process ends, and every call on one GPU shares it: calls that overlap on one GPU
// (two streams, two host threads) race on its contents. Nothing in it needs clearing: every
// launch writes each key it later reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dflash.h"
#include "kernels.h"
#include "noalloc.h"

namespace {

static __device__ __align__(256) unsigned long long scratch[dflash::NOALLOC_KEY_BYTES / sizeof(unsigned long long)];

std::mutex g_mu;
void* g_addr[dflash::MAX_DEVICES];  // device address of each device's copy, once looked up

}  // namespace

namespace dflash {

hipError_t noalloc_scratch_address(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[device] = p;
  }
  *out = g_addr[device];
  return hipSuccess;
}

}  // namespace dflash

extern "C" dflash_status dflash_lm_head_argmax_noalloc(dflash_ctx* ctx, const void* rows, int32_t n, int32_t* d_idx,
                                                       void* stream) {
  if (!ctx) return DFLASH_E_ARG;
  unsigned long long* keys = nullptr;
  const dflash_status s = dflash::noalloc_keys_for_call(ctx, &keys);
  if (s != DFLASH_OK) return s;
  return dflash::lm_head_argmax_into(ctx, rows, n, d_idx, keys, dflash::NOALLOC_KEY_BYTES, (hipStream_t)stream);
}
