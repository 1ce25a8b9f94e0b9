// Runtime internals shared by dflash.cpp and noalloc.hip (the allocation-free argmax).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

// Bytes of the fixed argmax key array per device: 8-byte keys of a launch's rows from its
// work-groups: up to 16 rows from 16384 work-groups, 32 or 48 rows from 8192 (rows past 16
// take four 16-column tiles per work-group), which covers every vocabulary up to 524288 rows
// (the bound is computed per call and checked against this size).
constexpr size_t NOALLOC_KEY_BYTES = (size_t)4 << 20;

// Device address of `device`'s copy of the array (looked up once per device; that device
// must be current on the first call for it). Defined in noalloc.hip.
hipError_t noalloc_scratch_address(int device, void** out);

// The array of the context's device, checking that this device is current (dflash.cpp).
dflash_status noalloc_keys_for_call(dflash_ctx* ctx, unsigned long long** out);

// dflash_lm_head_argmax with the per-work-group keys in `keys` (keys_bytes long); returns
// DFLASH_E_SHAPE with nothing enqueued if a launch would need more (dflash.cpp).
dflash_status lm_head_argmax_into(dflash_ctx* ctx, const void* rows, int32_t n, int32_t* d_idx,
                                  unsigned long long* keys, size_t keys_bytes, hipStream_t st);

}  // namespace dflash
