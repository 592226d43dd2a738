// lt_store.h -- device-scope stores for a kernel's last writes.
//
// A store marked sc1 (device coherent) is a plain vector store whose write
// goes through to the device-wide cache level at once.  For the last writes
// of a short kernel (the weight-streaming kernel's `out` update, the norm
// kernel's latent) this measured 0.2-0.3 us less per call back to back than
// the default-scope store of the same bits: the call ends when its writes
// are done, and these are done sooner.
#pragma once

#include "lt_device.h"

// Cache-policy bit of buffer instructions: device (agent) coherent, sc1.
constexpr int LT_SC1 = 16;

__device__ __forceinline__ void lt_store8_dev(void *p, u32x2_t v)
{
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), __builtin_bit_cast(uint64_t, v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void lt_store2_dev(u16 *p, u16 v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
