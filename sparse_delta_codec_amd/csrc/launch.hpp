// launch.hpp -- host side of persistent launches: a grid of at most as many
// workgroups as fit on the device at once, launched cooperatively so that the
// runtime guarantees they are all resident together.  Kernels that pass
// results from tile to tile (decoupled look-back) then walk their tiles in a
// static order, blockIdx.x, blockIdx.x + gridDim.x, ..., and every tile a
// workgroup waits for belongs to a workgroup that is running.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <unordered_map>

namespace pulse {

// Workgroups of `kernel` (threads per group, dynamic LDS) resident at once on
// the current device; 0 on error.  Cached per (kernel, device).
inline int64_t resident_groups(const void *kernel, int threads, size_t lds) {
    static std::mutex mu;
    static std::unordered_map<uint64_t, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const uint64_t key = (uint64_t)reinterpret_cast<uintptr_t>(kernel) * 131 + (uint64_t)dev;
    {
        std::lock_guard<std::mutex> g(mu);
        const auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const int64_t n = (int64_t)per_cu * cus;
    std::lock_guard<std::mutex> g(mu);
    cache[key] = n;
    return n;
}

// Cooperative launch of `kernel(args)` over min(tiles, resident) workgroups.
template <typename Args>
inline int launch_persistent(const void *kernel, int64_t tiles, int threads, size_t lds, Args &args,
                             hipStream_t stream) {
    const int64_t res = resident_groups(kernel, threads, lds);
    if (res <= 0) return -5;
    const int64_t grid = tiles < res ? tiles : res;
    void *params[] = {&args};
    const hipError_t e = hipLaunchCooperativeKernel(kernel, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(threads),
                                                    params, (unsigned)lds, stream);
    return e == hipSuccess ? 0 : -5;
}

}  // namespace pulse
