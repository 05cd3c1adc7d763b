// Fixed-size device scratch for mlora_linear_noalloc, the entry point for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own copy, at
// its own address, until the process ends.  In host code the array's name is only a host-side
// stand-in for the symbol; its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that address is what the kernels receive.
// Calls on one GPU share the array, so calls that overlap on one GPU race; the kernels of
// mlora_linear need no part of it to start at zero.
#include <mutex>

#include "kernels.h"
#include "mlora.h"

static __device__ __align__(256) uint8_t scratch[MLORA_NOALLOC_SCRATCH_BYTES];

namespace mlora {

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void **ptr)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess)
                e = e2;
        }
        if (e != hipSuccess)
            return e;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace mlora
