// Dispatch of the split-KV decode kernels (bodies in ifa_split_impl.h).
#include <map>
#include <mutex>
#include <utility>

#include "internal.h"

namespace ifa {

hipError_t launch_split(const SplitParams &p, int kv, int D, int G, bool paged, int extra, hipStream_t s) {
    switch (kv) {
    case KV_F16: return launch_split_kv<KV_F16>(p, D, G, paged, extra, s);
    case KV_BF16: return launch_split_kv<KV_BF16>(p, D, G, paged, extra, s);
    case KV_I8: return launch_split_kv<KV_I8>(p, D, G, paged, extra, s);
    }
    return hipErrorInvalidValue;
}

// Resident waves of a kernel on the current device.  The occupancy query is
// made once per (device, kernel) and cached: it does not change while the
// process runs, and it would otherwise be a per-call host cost.
int split_resident_waves(int kv, int D, int G, bool paged, int extra) {
    const void *f = kv == KV_F16 ? split_kernel_ptr<KV_F16>(D, G, paged, extra)
                  : kv == KV_BF16 ? split_kernel_ptr<KV_BF16>(D, G, paged, extra)
                                  : split_kernel_ptr<KV_I8>(D, G, paged, extra);
    int dev = 0;
    if (!f || hipGetDevice(&dev) != hipSuccess) return 0;
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, int> cache;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find({dev, f});
        if (it != cache.end()) return it->second;
    }
    int blocks = 0, cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, f, 64 * kWavesPerBlock, 0) != hipSuccess) return 0;
    const int waves = blocks * kWavesPerBlock * cus;
    std::lock_guard<std::mutex> lock(mu);
    cache[{dev, f}] = waves;
    return waves;
}

}  // namespace ifa
