// Launch helper shared by the GEMM and attention kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

namespace pipegemm {

// Raises `fn`'s dynamic LDS limit to the 160 KiB of a gfx950 CU on the current
// device, once per device: the attribute belongs to the function as loaded on
// one device.  `done` holds one bit per device id below 64 (higher ids set the
// attribute on every call).  Two first calls racing on one device both set the
// same value, which is harmless.
inline hipError_t allow_full_lds(const void *fn, std::atomic<uint64_t> &done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit))
        return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_release);
    return e;
}

}  // namespace pipegemm
