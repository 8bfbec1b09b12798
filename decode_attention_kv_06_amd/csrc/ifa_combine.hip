// Split-combine kernel: merges the partial softmax states of one (b, h) row
// in a fixed order (deterministic: same inputs, same bits), divides by the
// softmax denominator, applies the V antiquant epilogue and rounds the fp32
// result to nearest-even into the query dtype, or quantises it to int8.
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

__device__ __forceinline__ float ld_q2(const void *p, int64_t i, int bf16) {
    if (bf16) return __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
    return reinterpret_cast<const float *>(p)[i];
}

// Maximum over the 64 lanes: DPP within each 16-lane row, then the four row
// results through readlane.
__device__ __forceinline__ float wave_max(float x) {
    auto dpp = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value,
                                                                  0xF, 0xF, true));
    };
    x = fmaxf(x, dpp(x, std::integral_constant<int, 0xB1>{}));
    x = fmaxf(x, dpp(x, std::integral_constant<int, 0x4E>{}));
    x = fmaxf(x, dpp(x, std::integral_constant<int, 0x141>{}));
    x = fmaxf(x, dpp(x, std::integral_constant<int, 0x140>{}));
    const int xi = __builtin_bit_cast(int, x);
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// One wave per (b, h) row.  The split states are read lane-parallel (lane i
// holds split i, 64 at a time); the weighted sum over splits runs in split
// order in every lane, so the result does not depend on timing.
// PL = D / 64 output elements per lane.
template <int PL>
__global__ __launch_bounds__(256) void combine_kernel(const CombineParams P) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= P.nb * P.N) return;
    const int bl = row / P.N, h = row % P.N;
    const int64_t b = P.b0 + bl;
    const int D = P.D;
    // the segments of row (b, j, hg) sit in consecutive slots, one per piece
    // that the row overlaps (the split kernel's slot rule)
    const int jj = h / P.g, hin = h - jj * P.g;
    const int hg = hin / P.G, hh = hin - hg * P.G;
    const int rj = jj * P.n_hg + hg;
    const int len = P.len[bl];
    int nch = 0;
    int64_t slot0 = 0;
    if (len > 0) {
        const int64_t start = row_cost(P, bl, rj);        // the row's first cost unit
        nch = (int)((start + len - 1) / P.piece - start / P.piece + 1);
        slot0 = P.sbase[bl] + (int64_t)rj * P.maxseg[bl];
    }
    // partial state i of this head lives at row (slot0 + i) * G + hh
    auto prow = [&](int i) -> int64_t { return (slot0 + i) * P.G + hh; };
    // (m, l) pairs read as 64-bit words through a global pointer (no flat loads)
    typedef __attribute__((address_space(1))) const uint64_t gu64;
    gu64 *mlw = (gu64 *)P.part_ml;
    auto ml = [&](int64_t r) { return __builtin_bit_cast(float2, (uint64_t)mlw[r]); };

    // (m, l) of up to 64 splits in one load round, lane i holding split i
    const bool bf = P.out_bf16 != 0;
    constexpr int kMaxPerLane = PL;
    constexpr int per_lane = PL;
    float o[kMaxPerLane];
#pragma unroll
    for (int e = 0; e < kMaxPerLane; e++) o[e] = 0.f;
    float L = 0.f;
    float M = -__builtin_huge_valf();
    // The accumulators of the first U splits are requested together with the
    // (m, l) pairs (one memory round trip for rows of up to U splits): 16 for
    // head dims up to 256, 8 for 512, in at most 64 registers.
    constexpr int U = PL >= 8 ? 8 : 16;
    float v[U][kMaxPerLane];
    auto load_acc = [&](int first, int cnt_total) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const float *acc = P.part_acc + prow(min(first + u, cnt_total - 1)) * D;
#pragma unroll
            for (int e = 0; e < kMaxPerLane; e++) v[u][e] = e < per_lane ? acc[lane + 64 * e] : 0.f;
        }
    };
    float2 ml0 = make_float2(-__builtin_huge_valf(), 0.f);
    if (lane < nch) ml0 = ml(prow(lane));
    if (nch > 0) load_acc(0, nch);
    M = ml0.x;
    for (int i0 = 64; i0 < nch; i0 += 64) {
        const int i = i0 + lane;
        if (i < nch) M = fmaxf(M, ml(prow(i)).x);
    }
    M = wave_max(M);
    for (int i0 = 0; i0 < nch; i0 += 64) {
        const int cnt = min(64, nch - i0);
        float w = 0.f, lw = 0.f;
        if (lane < cnt) {
            const float2 mv = i0 == 0 ? ml0 : ml(prow(i0 + lane));
            w = __builtin_amdgcn_exp2f(mv.x - M);
            lw = w * mv.y;
        }
        // Splits in order, U at a time: their loads are issued together
        // (indices past the last split re-read it and get weight 0), then
        // accumulated in split order with the weight broadcast by readlane.
        for (int i = 0; i < cnt; i += U) {
            if (i0 + i > 0) load_acc(i0 + i, nch);
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int iu = min(i + u, 63);
                float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), iu));
                float li = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lw), iu));
                if (i + u >= cnt) wi = li = 0.f;
                L += li;
#pragma unroll
                for (int e = 0; e < kMaxPerLane; e++) o[e] += wi * v[u][e];
            }
        }
    }
#pragma unroll
    for (int e = 0; e < kMaxPerLane; e++) {
        if (e >= per_lane) break;
        const int d = lane + 64 * e;
        if (d >= P.Dr) break;                    // past the call's head dim
        float res = 0.f;
        if (nch > 0 && L > 0.f) {
            res = o[e] / L;
            if (P.aq_mode) {
                const int j = h / P.g;
                const int64_t pi = (P.aq_mode == 1) ? 1 : ((int64_t)P.Nkv + j) * P.Dr + d;
                const float sv = ld_param(P.v_scale, pi, bf), ov = ld_param(P.v_offset, pi, bf);
                res = sv * res + sv * ov;
            }
        }
        const int64_t oi = (b * P.N + h) * P.Dr + d;
        if (P.out_i8) {
            // int8 output: y = res * s + t on the fp32 result, ties to even, saturated
            const int64_t ci = P.q2_per_channel ? (int64_t)h * P.Dr + d : 0;
            const float qs = ld_q2(P.q_scale2, ci, P.q2_bf16);
            const float qo = P.q_offset2 ? ld_q2(P.q_offset2, ci, P.q2_bf16) : 0.f;
            const float y = fminf(fmaxf(__builtin_rintf(fmaf(res, qs, qo)), -128.f), 127.f);
            reinterpret_cast<int8_t *>(P.out)[oi] = (int8_t)(int)y;
        } else if (bf) {
            reinterpret_cast<__bf16 *>(P.out)[oi] = (__bf16)res;
        } else {
            reinterpret_cast<_Float16 *>(P.out)[oi] = (_Float16)res;
        }
    }
}

}  // namespace

hipError_t launch_combine(const CombineParams &p, hipStream_t s) {
    const int rows = p.nb * p.N;
    const int blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    switch (p.D / 64) {
    case 1: hipLaunchKernelGGL(combine_kernel<1>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, p); break;
    case 2: hipLaunchKernelGGL(combine_kernel<2>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, p); break;
    case 4: hipLaunchKernelGGL(combine_kernel<4>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, p); break;
    default: hipLaunchKernelGGL(combine_kernel<8>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, p); break;
    }
    return hipGetLastError();
}

}  // namespace ifa
