// Split-combine kernel: merges the partial softmax states of one (b, h) row
// in a fixed order (deterministic: same inputs, same bits), divides by the
// softmax denominator, applies the V antiquant epilogue and rounds the fp32
// result to nearest-even into the query dtype.
//
//   M = max_i m_i,  out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i
//
// A row with no work item, or whose denominator is 0 (every position
// excluded), is written as zeros.  For int8 V the partial sums are over the
// integer values, so out = s_V * ratio + s_V * o_V (dequantised value
// (x + o) * s, index 1 of the antiquant parameters).
#include "internal.h"

namespace ifa {
namespace {

__device__ __forceinline__ float ld_param(const void *p, int64_t i, bool bf16) {
    const uint32_t bits = reinterpret_cast<const uint16_t *>(p)[i];
    return bf16 ? __builtin_bit_cast(float, bits << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__global__ __launch_bounds__(256) void combine_kernel(const CombineParams P) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= P.nb * P.N) return;
    const int bl = row / P.N, h = row % P.N;
    const int64_t b = P.b0 + bl;
    const int c0 = P.cum[bl], nch = P.cum[bl + 1] - c0;
    const int D = P.D;

    float M = -__builtin_huge_valf();
    for (int i = 0; i < nch; i++) M = fmaxf(M, P.part_ml[((int64_t)(c0 + i) * P.N + h) * 2]);
    float L = 0.f;
    for (int i = 0; i < nch; i++) {
        const float2 ml = *reinterpret_cast<const float2 *>(P.part_ml + ((int64_t)(c0 + i) * P.N + h) * 2);
        L += __builtin_amdgcn_exp2f(ml.x - M) * ml.y;
    }
    const bool bf = P.out_bf16 != 0;
    for (int d = lane; d < D; d += 64) {
        float o = 0.f;
        for (int i = 0; i < nch; i++) {
            const int64_t pr = (int64_t)(c0 + i) * P.N + h;
            o += __builtin_amdgcn_exp2f(P.part_ml[pr * 2] - M) * P.part_acc[pr * D + d];
        }
        float res = 0.f;
        if (nch > 0 && L > 0.f) {
            res = o / L;
            if (P.aq_mode) {
                const int j = h / P.g;
                const int64_t pi = (P.aq_mode == 1) ? 1 : ((int64_t)P.Nkv + j) * D + d;
                const float sv = ld_param(P.v_scale, pi, bf), ov = ld_param(P.v_offset, pi, bf);
                res = sv * res + sv * ov;
            }
        }
        const int64_t oi = (b * P.N + h) * D + d;
        if (bf)
            reinterpret_cast<__bf16 *>(P.out)[oi] = (__bf16)res;
        else
            reinterpret_cast<_Float16 *>(P.out)[oi] = (_Float16)res;
    }
}

}  // namespace

hipError_t launch_combine(const CombineParams &p, hipStream_t s) {
    const int rows = p.nb * p.N;
    const int blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, p);
    return hipGetLastError();
}

}  // namespace ifa
