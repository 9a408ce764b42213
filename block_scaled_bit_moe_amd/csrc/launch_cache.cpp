// launch_cache.cpp -- per-device answers to the runtime queries a launch
// needs (CU count, resident workgroups per CU, dynamic-LDS opt-in), computed
// once and then served from a table, so that a call makes no runtime query
// after its first on a device.  Safe to call from several threads at once.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>

#include "kernels.h"

namespace moeq {

namespace {
std::mutex g_mu;
std::map<int, int> g_cus;                                          // device -> CUs
std::map<std::tuple<const void *, int, int, size_t>, int> g_occ;   // (kernel, device, threads, lds) -> per CU
std::map<std::pair<const void *, int>, size_t> g_lds;              // (kernel, device) -> dynamic LDS allowed
}  // namespace

int current_device() {
    int dev = 0;
    (void)hipGetDevice(&dev);
    return dev;
}

int cached_cus() {
    const int dev = current_device();
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_cus.find(dev);
        if (it != g_cus.end()) return it->second;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 1;
    std::lock_guard<std::mutex> lk(g_mu);
    g_cus[dev] = cus;
    return cus;
}

int cached_occupancy(const void *kern, int threads, size_t dyn) {
    const auto key = std::make_tuple(kern, current_device(), threads, dyn);
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_occ.find(key);
        if (it != g_occ.end()) return it->second;
    }
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, threads, dyn) != hipSuccess || per < 0) per = 0;
    std::lock_guard<std::mutex> lk(g_mu);
    g_occ[key] = per;
    return per;
}

hipError_t ensure_dyn_lds(const void *kern, size_t dyn) {
    const auto key = std::make_pair(kern, current_device());
    std::lock_guard<std::mutex> lk(g_mu);   // held across the call: the attribute is raised once
    size_t &have = g_lds[key];
    if (dyn <= have) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e == hipSuccess) have = dyn;
    return e;
}

}  // namespace moeq
