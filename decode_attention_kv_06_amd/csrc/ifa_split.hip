// Dispatch of the split-KV decode kernels (bodies in ifa_split_impl.h).
#include "internal.h"

namespace ifa {

hipError_t launch_split(const SplitParams &p, int kv, int D, int G, bool paged, bool masked, hipStream_t s) {
    switch (kv) {
    case KV_F16: return launch_split_kv<KV_F16>(p, D, G, paged, masked, s);
    case KV_BF16: return launch_split_kv<KV_BF16>(p, D, G, paged, masked, s);
    case KV_I8: return launch_split_kv<KV_I8>(p, D, G, paged, masked, s);
    }
    return hipErrorInvalidValue;
}

int split_resident_waves(int kv, int D, int G, bool paged, bool masked) {
    const void *f = kv == KV_F16 ? split_kernel_ptr<KV_F16>(D, G, paged, masked)
                  : kv == KV_BF16 ? split_kernel_ptr<KV_BF16>(D, G, paged, masked)
                                  : split_kernel_ptr<KV_I8>(D, G, paged, masked);
    int blocks = 0, dev = 0, cus = 0;
    if (!f || hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, f, 64 * kWavesPerBlock, 0) != hipSuccess) return 0;
    return blocks * kWavesPerBlock * cus;
}

}  // namespace ifa
