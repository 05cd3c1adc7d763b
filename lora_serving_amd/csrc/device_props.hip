// Per-device facts the launchers need, looked up once per device and cached under a lock:
// the CU count, each kernel's static LDS, how many of a kernel's workgroups a CU holds at once,
// and the dynamic-LDS limit already granted to a kernel (hipFuncSetAttribute is called again
// only when a launch needs more).
#include <map>
#include <mutex>
#include <utility>

#include "kernels.h"

namespace mlora {

namespace {
std::mutex g_mu;
std::map<int, int> g_cus;                                    // device -> CUs
std::map<std::pair<int, const void *>, size_t> g_lds_granted; // (device, kernel) -> bytes
std::map<std::pair<int, const void *>, size_t> g_lds_static;  // (device, kernel) -> bytes
std::map<std::pair<int, const void *>, int> g_resident;       // (device, kernel) -> workgroups

int current_device()
{
    int dev = 0;
    return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}
}  // namespace

int device_cu_count()
{
    const int dev = current_device();
    if (dev < 0)
        return MI355X_CUS;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_cus.find(dev);
    if (it != g_cus.end())
        return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = MI355X_CUS;
    g_cus[dev] = n;
    return n;
}

size_t kernel_static_lds(const void *fn)
{
    const int dev = current_device();
    std::lock_guard<std::mutex> lock(g_mu);
    auto key = std::make_pair(dev, fn);
    auto it = g_lds_static.find(key);
    if (it != g_lds_static.end())
        return it->second;
    hipFuncAttributes attr{};
    size_t s = 0;
    if (hipFuncGetAttributes(&attr, fn) == hipSuccess)
        s = attr.sharedSizeBytes;
    else
        s = 1024;   // unknown: assume a little, so that budgets stay on the safe side
    g_lds_static[key] = s;
    return s;
}

int kernel_resident_blocks(const void *fn, int threads, size_t dyn_lds)
{
    const int dev = current_device();
    std::lock_guard<std::mutex> lock(g_mu);
    auto key = std::make_pair(dev, fn);
    auto it = g_resident.find(key);
    if (it != g_resident.end())
        return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, dyn_lds) != hipSuccess ||
        n < 1)
        n = 1;
    g_resident[key] = n;
    return n;
}

hipError_t ensure_dynamic_lds(const void *fn, size_t bytes)
{
    if (bytes <= 64 * 1024)
        return hipSuccess;   // within the default limit
    const int dev = current_device();
    std::lock_guard<std::mutex> lock(g_mu);
    auto key = std::make_pair(dev, fn);
    auto it = g_lds_granted.find(key);
    if (it != g_lds_granted.end() && it->second >= bytes)
        return hipSuccess;
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess)
        g_lds_granted[key] = bytes;
    return e;
}

}  // namespace mlora
