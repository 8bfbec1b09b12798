// Split-KV decode kernels for bf16 KV caches (instantiations of ifa_split_impl.h).
#include "ifa_split_impl.h"

namespace ifa {
template hipError_t launch_split_kv<KV_BF16>(const SplitParams &, int, int, bool, int, hipStream_t);
template const void *split_kernel_ptr<KV_BF16>(int, int, bool, int);
}  // namespace ifa
