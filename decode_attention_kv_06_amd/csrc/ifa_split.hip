// Split-KV decode kernel for IncreFlashAttention on gfx950.
//
// Computes, for one work item, the partial softmax state of
//     softmax(scale * q K^T) V                (IncreFlashAttention README, "Formula")
// over a contiguous range of KV positions: the running maximum m (log2
// domain), the running sum l of exp2(x - m) and the unnormalised sum of
// exp2(x - m) * v.  The split-combine kernel merges the work items of a row.
//
// Mapping to the hardware: one wave64 per work item, four independent waves
// per workgroup.  A KV row of D elements is read by D/8 consecutive lanes,
// 16 bytes each (8 bytes for int8), so one load instruction covers 64/(D/8)
// consecutive rows: fully used 128-byte lines, no LDS staging.  Each lane
// keeps the running softmax state of the rows it reads; the lanes of one row
// hold identical copies (their dot products are reduced with DPP inside the
// 16-lane DPP row), and the row groups are merged once per work item.  Dot
// products use v_dot2_f32_{f16,bf16} (two products per lane-op, fp32
// accumulation); int8 rows are widened exactly to fp16 with a byte permute.
// The next tile's K/V loads are in flight while the current tile computes.
#include "internal.h"

namespace ifa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxInit = -1.0e30f;   // finite start value of the running max

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                                                 false));
}

__device__ __forceinline__ float swz_xor16(float x) {
    // ds_swizzle bit mode: and 0x1f, or 0, xor 0x10 (within 32-lane halves).
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

// Sum over the LPR consecutive lanes that share one KV row; every lane of the
// group ends with the same bits (each step adds a symmetric pair).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    if constexpr (LPR >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    if constexpr (LPR >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) x += dpp<0x141>(x);   // row_half_mirror
    if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror
    if constexpr (LPR >= 32) x += swz_xor16(x);
    if constexpr (LPR >= 64) x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, std::integral_constant<int, KV_BF16>) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, std::integral_constant<int, KV_F16>) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

__device__ __forceinline__ uint32_t pack_p(float a, float b, std::integral_constant<int, KV_BF16>) {
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pack_p(float a, float b, std::integral_constant<int, KV_F16>) {
    f16x2 r;
    r[0] = (_Float16)a;
    r[1] = (_Float16)b;
    return __builtin_bit_cast(uint32_t, r);
}

// int8 -> fp16, exact: the byte b (two's complement) is xor'ed with 0x80 to
// u = b + 128, placed under the fp16 exponent of 1024 (0x64 high byte) to
// give 1024 + u, and 1152 is subtracted.  Values 1024..1279 are exact in fp16.
__device__ __forceinline__ uint32_t i8pair_to_f16x2(uint32_t biased_pair) {
    f16x2 h = __builtin_bit_cast(f16x2, biased_pair);
    const f16x2 c = {(_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(uint32_t, h - c);
}
constexpr uint32_t kF16Hi = 0x64646464u;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// s / block_size for 32-bit s (Granlund-Montgomery, "Division by invariant
// integers using multiplication", round-up multiplier, valid for divisors >= 2).
__device__ __forceinline__ uint32_t div_bs(uint32_t s, uint32_t magic, int shift) {
    uint32_t t1 = __umulhi(magic, s);
    return (t1 + ((s - t1) >> 1)) >> (shift - 1);
}

template <int KV, int D, int G>
struct Cfg {
    static constexpr int LPR = D / 8;                      // lanes per KV row
    static constexpr int RPI = 64 / LPR;                   // rows per load instruction
    static constexpr int W = (KV == KV_I8) ? 2 : 4;        // dwords per lane per row
    static constexpr int EB = (KV == KV_I8) ? 1 : 2;       // element bytes
    static constexpr int RT = (G >= 4) ? 4 : 8;            // row steps per tile
    static constexpr int TT = RT * RPI;                    // positions per tile
};

template <int KV, int D, int G, bool PAGED>
__global__ __launch_bounds__(256) void split_kernel(const SplitParams P) {
    using C = Cfg<KV, D, G>;
    constexpr int LPR = C::LPR, RPI = C::RPI, W = C::W, EB = C::EB, RT = C::RT, TT = C::TT;
    constexpr bool I8 = KV == KV_I8;
    using DotK = std::integral_constant<int, I8 ? KV_F16 : KV>;

    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= P.n_items) return;
    const int hg = item % P.n_hg;
    const int rest = item / P.n_hg;
    const int j = rest % P.Nkv;
    const int gc = rest / P.Nkv;

    // Batch of this chunk: the number of batches whose first chunk is <= gc.
    int cnt = 0;
    for (int e0 = 0; e0 < P.nb; e0 += 64) {
        const int e = e0 + lane;
        const bool le = e < P.nb && P.cum[e] <= gc;
        cnt += __popcll(__ballot(le));
    }
    const int bl = __builtin_amdgcn_readfirstlane(cnt - 1);
    const int lo = P.lo[bl] + (gc - P.cum[bl]) * P.chunk;
    const int hi = min(P.hi[bl], lo + P.chunk);
    const int64_t b = P.b0 + bl;

    const int r = lane / LPR;      // row group
    const int c = lane % LPR;      // 8-element slot within the row

    // ---------------------------------------------------------- query
    const int hbase = j * P.g + hg * G;
    uint32_t qv[G][4];
    float qmul = P.score_mul;
    if constexpr (!I8) {
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            const bool ok = hg * G + hh < P.g;
            const int64_t off = ((b * P.N + hbase + (ok ? hh : 0)) * D + 8 * c) * 2;
            uint4 x = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(P.q) + off);
            if (!ok) x = make_uint4(0, 0, 0, 0);
            qv[hh][0] = x.x; qv[hh][1] = x.y; qv[hh][2] = x.z; qv[hh][3] = x.w;
        }
    } else {
        // q' = q * s_K (K's antiquant scale) in fp16, multiplied by a power of
        // two so the largest |q'| of the wave sits just under 2^15; the score
        // multiplier takes the inverse power.  The K offset adds a constant
        // per row and drops out of the softmax.
        float qf[G][8];
        float amax = 0.f;
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            const bool ok = hg * G + hh < P.g;
            const int64_t off = ((b * P.N + hbase + (ok ? hh : 0)) * D + 8 * c) * 2;
            uint4 x = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(P.q) + off);
            uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFF;
                float qe = P.q_bf16 ? bf16_to_f32(bits) : f16_to_f32(bits);
                const int64_t si = (P.aq_mode == 1) ? 0 : (int64_t)j * D + 8 * c + e;
                const uint32_t sb = reinterpret_cast<const uint16_t *>(P.k_scale)[si];
                const float sc = P.q_bf16 ? bf16_to_f32(sb) : f16_to_f32(sb);
                qe = ok ? qe * sc : 0.f;
                qf[hh][e] = qe;
                amax = fmaxf(amax, fabsf(qe));
            }
        }
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        int ex = 0;
        if (amax > 0.f) (void)frexpf(amax, &ex);        // amax < 2^ex
        const float up = ldexpf(1.f, 15 - ex), down = ldexpf(1.f, ex - 15);
        qmul = P.score_mul * down;
#pragma unroll
        for (int hh = 0; hh < G; hh++)
#pragma unroll
            for (int w = 0; w < 4; w++) {
                f16x2 h2;
                h2[0] = (_Float16)(qf[hh][2 * w] * up);
                h2[1] = (_Float16)(qf[hh][2 * w + 1] * up);
                qv[hh][w] = __builtin_bit_cast(uint32_t, h2);
            }
    }

    // ---------------------------------------------------------- addressing
    const char *kb = reinterpret_cast<const char *>(P.k);
    const char *vb = reinterpret_cast<const char *>(P.v);
    const int64_t lane_byte = (int64_t)8 * c * EB;
    int64_t dense_base = 0;
    const int32_t *btab = nullptr;
    if constexpr (!PAGED) dense_base = b * P.sB + (int64_t)j * P.sN;
    else btab = P.block_table + b * P.max_blocks;
    const uint8_t *mrow = nullptr;
    if (P.mask_mode) mrow = P.mask + (P.mask_sB ? b * P.mask_sB : 0) + (int64_t)hbase * P.mask_sH;

    // Byte offset of position t's row for this lane; ok=false when the block
    // id is out of range (never dereferenced: offset 0 is read instead).
    auto row_off = [&](int t, bool &ok) -> int64_t {
        if constexpr (!PAGED) {
            ok = true;
            return (dense_base + (int64_t)t * P.sS) * EB + lane_byte;
        } else {
            const uint32_t q = div_bs((uint32_t)t, P.bs_magic, P.bs_shift);
            const int rr = t - (int)q * P.block_size;
            const int blk = btab[q];
            ok = (unsigned)blk < (unsigned)P.num_blocks;
            const int64_t e = (int64_t)blk * P.blk_stride + (int64_t)j * P.head_stride + (int64_t)rr * P.row_stride;
            return ok ? e * EB + lane_byte : 0;
        }
    };

    uint32_t kA[RT][W], vA[RT][W], kB[RT][W], vB[RT][W];
    bool okA[RT], okB[RT];

    auto load_tile = [&](int ts, uint32_t (&kr)[RT][W], uint32_t (&vr)[RT][W], bool (&okr)[RT]) {
        int64_t offs[RT];
#pragma unroll
        for (int i = 0; i < RT; i++) {
            const int t = min(ts + i * RPI + r, hi - 1);
            offs[i] = row_off(t, okr[i]);
        }
#pragma unroll
        for (int i = 0; i < RT; i++) {
            if constexpr (W == 4) {
                const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kb + offs[i]));
                kr[i][0] = x[0]; kr[i][1] = x[1]; kr[i][2] = x[2]; kr[i][3] = x[3];
            } else {
                const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(kb + offs[i]));
                kr[i][0] = x[0]; kr[i][1] = x[1];
            }
        }
#pragma unroll
        for (int i = 0; i < RT; i++) {
            if constexpr (W == 4) {
                const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vb + offs[i]));
                vr[i][0] = x[0]; vr[i][1] = x[1]; vr[i][2] = x[2]; vr[i][3] = x[3];
            } else {
                const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(vb + offs[i]));
                vr[i][0] = x[0]; vr[i][1] = x[1];
            }
        }
    };

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int hh = 0; hh < G; hh++) {
        m[hh] = kMaxInit;
        l[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) acc[hh][e] = 0.f;
    }

    auto compute_tile = [&](int ts, const uint32_t (&kr)[RT][W], const uint32_t (&vr)[RT][W],
                            const bool (&okr)[RT]) {
        float s[RT][G];
#pragma unroll
        for (int i = 0; i < RT; i++) {
            uint32_t kk[4];
            if constexpr (I8) {
                const uint32_t w0 = kr[i][0] ^ 0x80808080u, w1 = kr[i][1] ^ 0x80808080u;
                kk[0] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, w0, 0x04010400u));
                kk[1] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, w0, 0x04030402u));
                kk[2] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, w1, 0x04010400u));
                kk[3] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, w1, 0x04030402u));
            } else {
#pragma unroll
                for (int w = 0; w < 4; w++) kk[w] = kr[i][w];
            }
#pragma unroll
            for (int hh = 0; hh < G; hh++) {
                float a = 0.f;
#pragma unroll
                for (int w = 0; w < 4; w++) a = dot2(qv[hh][w], kk[w], a, DotK{});
                s[i][hh] = row_sum<LPR>(a);
            }
        }
        // validity: inside the chunk, block id in range, not masked
#pragma unroll
        for (int i = 0; i < RT; i++) {
            const int t = ts + i * RPI + r;
            const bool in = t < hi && okr[i];
            const int tl = min(t, hi - 1);
            bool shared_masked = false;
            if (P.mask_mode == 1) shared_masked = mrow[tl] != 0;
#pragma unroll
            for (int hh = 0; hh < G; hh++) {
                bool msk = shared_masked;
                // padded heads of the last group (hg*G + hh >= g) have no mask row
                if (P.mask_mode == 2) msk = (hg * G + hh < P.g) ? mrow[(int64_t)hh * P.mask_sH + tl] != 0 : true;
                s[i][hh] = (in && !msk) ? s[i][hh] * qmul : kNegInf;
            }
        }
        // online softmax (log2 domain)
        float p[RT][G];
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            float mt = s[0][hh];
#pragma unroll
            for (int i = 1; i < RT; i++) mt = fmaxf(mt, s[i][hh]);
            const float mn = fmaxf(m[hh], mt);
            const float alpha = __builtin_amdgcn_exp2f(m[hh] - mn);
            m[hh] = mn;
            float ls = 0.f;
#pragma unroll
            for (int i = 0; i < RT; i++) {
                p[i][hh] = __builtin_amdgcn_exp2f(s[i][hh] - mn);
                ls += p[i][hh];
            }
            l[hh] = l[hh] * alpha + ls;
#pragma unroll
            for (int e = 0; e < 8; e++) acc[hh][e] *= alpha;
        }
        // P.V over pairs of row steps (two positions per dot2)
#pragma unroll
        for (int i = 0; i < RT; i += 2) {
            uint32_t vp[8];     // vp[e] = {v_i[d_e], v_{i+1}[d_e]} as a 16-bit pair
            if constexpr (I8) {
#pragma unroll
                for (int w = 0; w < 2; w++) {
                    const uint32_t a = vr[i][w] ^ 0x80808080u, bq = vr[i + 1][w] ^ 0x80808080u;
                    const uint32_t x01 = __builtin_amdgcn_perm(bq, a, 0x05010400u);  // a0 b0 a1 b1
                    const uint32_t x23 = __builtin_amdgcn_perm(bq, a, 0x07030602u);  // a2 b2 a3 b3
                    vp[4 * w + 0] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, x01, 0x04010400u));
                    vp[4 * w + 1] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, x01, 0x04030402u));
                    vp[4 * w + 2] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, x23, 0x04010400u));
                    vp[4 * w + 3] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, x23, 0x04030402u));
                }
            } else {
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    vp[2 * w] = __builtin_amdgcn_perm(vr[i + 1][w], vr[i][w], 0x05040100u);
                    vp[2 * w + 1] = __builtin_amdgcn_perm(vr[i + 1][w], vr[i][w], 0x07060302u);
                }
            }
#pragma unroll
            for (int hh = 0; hh < G; hh++) {
                const uint32_t pp = pack_p(p[i][hh], p[i + 1][hh], DotK{});
#pragma unroll
                for (int e = 0; e < 8; e++) acc[hh][e] = dot2(pp, vp[e], acc[hh][e], DotK{});
            }
        }
    };

    // ---------------------------------------------------------- main loop
    int ts = lo;
    load_tile(ts, kA, vA, okA);
    while (true) {
        if (ts + TT < hi) load_tile(ts + TT, kB, vB, okB);
        compute_tile(ts, kA, vA, okA);
        ts += TT;
        if (ts >= hi) break;
        if (ts + TT < hi) load_tile(ts + TT, kA, vA, okA);
        compute_tile(ts, kB, vB, okB);
        ts += TT;
        if (ts >= hi) break;
    }

    // ---------------------------------------------------------- merge row groups
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            const float mo = __shfl_xor(m[hh], off);
            const float lo2 = __shfl_xor(l[hh], off);
            const float mn = fmaxf(m[hh], mo);
            const float a = __builtin_amdgcn_exp2f(m[hh] - mn), bb = __builtin_amdgcn_exp2f(mo - mn);
            l[hh] = l[hh] * a + lo2 * bb;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float ao = __shfl_xor(acc[hh][e], off);
                acc[hh][e] = acc[hh][e] * a + ao * bb;
            }
            m[hh] = mn;
        }
    }

    if (r == 0) {
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            if (hg * G + hh >= P.g) break;
            const int64_t row = (int64_t)gc * P.N + hbase + hh;
            float4 *dst = reinterpret_cast<float4 *>(P.part_acc + row * D + 8 * c);
            dst[0] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
            dst[1] = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
            if (c == 0) *reinterpret_cast<float2 *>(P.part_ml + row * 2) = make_float2(m[hh], l[hh]);
        }
    }
}

template <int KV, int D, int G, bool PAGED>
hipError_t launch_one(const SplitParams &p, hipStream_t s) {
    const int blocks = (p.n_items + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL((split_kernel<KV, D, G, PAGED>), dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, p);
    return hipGetLastError();
}

template <int KV, int D, int G>
const void *kernel_ptr(bool paged) {
    void (*fp)(const SplitParams) = paged ? split_kernel<KV, D, G, true> : split_kernel<KV, D, G, false>;
    return reinterpret_cast<const void *>(fp);
}

template <int KV, int D>
hipError_t dispatch_g(const SplitParams &p, int G, bool paged, hipStream_t s) {
    switch (G) {
    case 1: return paged ? launch_one<KV, D, 1, true>(p, s) : launch_one<KV, D, 1, false>(p, s);
    case 2: return paged ? launch_one<KV, D, 2, true>(p, s) : launch_one<KV, D, 2, false>(p, s);
    case 4: return paged ? launch_one<KV, D, 4, true>(p, s) : launch_one<KV, D, 4, false>(p, s);
    case 8: return paged ? launch_one<KV, D, 8, true>(p, s) : launch_one<KV, D, 8, false>(p, s);
    }
    return hipErrorInvalidValue;
}

template <int KV>
hipError_t dispatch_d(const SplitParams &p, int D, int G, bool paged, hipStream_t s) {
    switch (D) {
    case 64: return dispatch_g<KV, 64>(p, G, paged, s);
    case 128: return dispatch_g<KV, 128>(p, G, paged, s);
    case 256: return dispatch_g<KV, 256>(p, G, paged, s);
    case 512: return dispatch_g<KV, 512>(p, G, paged, s);
    }
    return hipErrorInvalidValue;
}

template <int KV, int D>
const void *ptr_g(int G, bool paged) {
    switch (G) {
    case 1: return kernel_ptr<KV, D, 1>(paged);
    case 2: return kernel_ptr<KV, D, 2>(paged);
    case 4: return kernel_ptr<KV, D, 4>(paged);
    case 8: return kernel_ptr<KV, D, 8>(paged);
    }
    return nullptr;
}

template <int KV>
const void *ptr_d(int D, int G, bool paged) {
    switch (D) {
    case 64: return ptr_g<KV, 64>(G, paged);
    case 128: return ptr_g<KV, 128>(G, paged);
    case 256: return ptr_g<KV, 256>(G, paged);
    case 512: return ptr_g<KV, 512>(G, paged);
    }
    return nullptr;
}

}  // namespace

hipError_t launch_split(const SplitParams &p, int kv, int D, int G, bool paged, hipStream_t s) {
    switch (kv) {
    case KV_F16: return dispatch_d<KV_F16>(p, D, G, paged, s);
    case KV_BF16: return dispatch_d<KV_BF16>(p, D, G, paged, s);
    case KV_I8: return dispatch_d<KV_I8>(p, D, G, paged, s);
    }
    return hipErrorInvalidValue;
}

int split_resident_waves(int kv, int D, int G, bool paged) {
    const void *f = kv == KV_F16 ? ptr_d<KV_F16>(D, G, paged)
                  : kv == KV_BF16 ? ptr_d<KV_BF16>(D, G, paged) : ptr_d<KV_I8>(D, G, paged);
    int blocks = 0, dev = 0, cus = 0;
    if (!f || hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, f, 64 * kWavesPerBlock, 0) != hipSuccess) return 0;
    return blocks * kWavesPerBlock * cus;
}

int split_tile_tokens(int kv, int D, int G) {
    const int lpr = D / 8, rpi = 64 / lpr;
    const int rt = (G >= 4) ? 4 : 8;
    (void)kv;
    return rt * rpi;
}

}  // namespace ifa
