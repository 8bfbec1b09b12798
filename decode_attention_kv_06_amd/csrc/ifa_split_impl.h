// Split-KV decode kernel for IncreFlashAttention on gfx950 (template body;
// instantiated per KV dtype in ifa_split_{f16,bf16,i8}.hip).
//
// Computes, for one segment of KV positions of one (batch, KV head, head
// group), the partial softmax state of
//     softmax(scale * q K^T) V                (IncreFlashAttention README, "Formula")
// as the running maximum m (log2 domain), the running sum l of exp2(x - m)
// and the unnormalised sum of exp2(x - m) * v.  The split-combine kernel
// merges the segments of a row.
//
// Mapping to the hardware: one wave64 per piece of work, four independent
// waves per workgroup.  A KV row of D elements is read by D/8 consecutive
// lanes, 16 bytes each (8 bytes for int8), so one load instruction covers
// 64/(D/8) consecutive rows: whole 128-byte lines, no LDS staging.  Each lane
// keeps the softmax state of the rows it reads; the lanes of one row hold
// identical copies (their partial dot products are reduced with DPP inside
// the 16-lane DPP row), and the row groups are merged once per segment.  Dot
// products use v_dot2_f32_{f16,bf16} (two products per lane-op, fp32
// accumulation); int8 rows are widened exactly to fp16 with byte permutes.
// The next tile's K/V loads are in flight while the current tile computes.
#pragma once

#include <type_traits>

#include "internal.h"

namespace ifa {
namespace split_detail {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x4 gu32x4;   // in global memory
typedef __attribute__((address_space(1))) u32x2 gu32x2;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxInit = -1.0e30f;   // finite start value of the running max
constexpr int kTblSlots = 256;        // staged block ids per wave (paged caches)
// The running max is raised only when a tile's max exceeds it by more than
// this many log2 units, so p = exp2(x - m) stays below 2^kLazy (exact: the
// same m scales both l and the accumulator).
constexpr float kLazy = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// A wave-uniform pointer, declared so (scalar registers).
__device__ __forceinline__ const char *uniform_ptr(const char *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo);
}

template <int CTRL>
__device__ __forceinline__ int dppi(int x) {
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ float swz_xor16(float x) {
    // ds_swizzle bit mode: and 0x1f, or 0, xor 0x10 (within 32-lane halves).
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

// Value of lane n of this lane's 16-lane DPP row (row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) { return dpp<0x150 + N>(x); }

// Reduce-scatter of G per-lane partial sums over the 16 lanes of a DPP row.
// Each level pairs every lane with the lane a DPP pattern names (row mirror:
// lane bits 0-3 flipped; half mirror: bits 0-2; quad swap: bit 1), adds the
// partner's upper half of the remaining registers to its own lower half, and
// so halves the heads a lane keeps.  No lane-dependent select is needed: the
// lanes hold their heads in a lane-dependent order, register p of lane l
// holding head p ^ head_code(l), with the code's bits (top first) b3, b2^b3,
// b1^b2 of the lane number.  Each pattern flips exactly the code bit of its
// level, so a lane's partner always holds the lane's kept heads in the
// registers it sends.  After log2(G) levels lane l holds head head_code(l);
// the remaining in-row levels (and the cross-row ones for rows longer than
// 16 lanes) are plain sums, which leave the code unchanged.
template <int G>
__host__ __device__ constexpr int head_code(int lane) {
    const int b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1, b3 = (lane >> 3) & 1;
    return G == 2 ? b3 : G == 4 ? (b3 << 1) | (b2 ^ b3) : G == 8 ? (b3 << 2) | ((b2 ^ b3) << 1) | (b1 ^ b2) : 0;
}
template <int CTRL, int N>
__device__ __forceinline__ void scatter_level(float (&v)[8]) {
#pragma unroll
    for (int j = 0; j < N / 2; j++) v[j] += dpp<CTRL>(v[j + N / 2]);
}
template <int G, int LPR>
__device__ __forceinline__ float scatter_reduce(const float (&s)[G]) {
    static_assert(G == 2 || G == 4 || G == 8, "head group");
    static_assert(LPR >= 16, "whole DPP rows");
    float v[8];
#pragma unroll
    for (int h = 0; h < G; h++) v[h] = s[h];
    scatter_level<0x140, G>(v);
    if constexpr (G >= 4) scatter_level<0x141, G / 2>(v);
    else v[0] += dpp<0x141>(v[0]);
    if constexpr (G >= 8) scatter_level<0x4E, G / 4>(v);
    else v[0] += dpp<0x4E>(v[0]);
    v[0] += dpp<0xB1>(v[0]);
    if constexpr (LPR >= 32) v[0] += swz_xor16(v[0]);
    if constexpr (LPR >= 64) v[0] += __shfl_xor(v[0], 32);
    return v[0];
}
template <int G>
__device__ __forceinline__ int head_of_lane(int lane) { return head_code<G>(lane); }
// a lane of a DPP row that holds head H after scatter_reduce (lane bit 0 clear)
template <int G, int H>
constexpr int lane_of_head() {
    constexpr int b3 = G == 2 ? H : G == 4 ? H >> 1 : H >> 2;
    constexpr int b2 = G == 4 ? (H & 1) ^ b3 : G == 8 ? ((H >> 1) & 1) ^ b3 : 0;
    constexpr int b1 = G == 8 ? (H & 1) ^ b2 : 0;
    static_assert(head_code<G>(8 * b3 + 4 * b2 + 2 * b1) == H, "head code inverse");
    return 8 * b3 + 4 * b2 + 2 * b1;
}
// every head's value from the lanes that hold them
template <int G, int H = 0>
__device__ __forceinline__ void gather_heads(float x, float (&out)[G]) {
    if constexpr (H < G) {
        out[H] = row_bcast<lane_of_head<G, H>()>(x);
        gather_heads<G, H + 1>(x, out);
    }
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, std::integral_constant<int, KV_BF16>) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, std::integral_constant<int, KV_F16>) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// The first product of a dot-product chain, written as the three-operand
// form with an inline 0 accumulator: the compiler otherwise picks the
// two-operand accumulate form and spends a v_mov per chain to zero it.
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b, std::integral_constant<int, KV_BF16>) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b, std::integral_constant<int, KV_F16>) {
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
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
    static constexpr int RT = (G >= 8) ? 4 : 8;                  // row steps per tile
    static constexpr int TT = RT * RPI;                    // positions per tile
};

// Waves per SIMD the register budget is sized for (G heads of state per lane
// and RT rows of K and V in flight): longer tiles at two waves per SIMD keep
// more bytes in flight than shorter ones at three.
template <int G>
constexpr int waves_per_eu() { return G == 1 ? 3 : 2; }

// One segment of a wave's piece: batch bl of the slice, row rj = j*n_hg + hg,
// window [lo, lo + nseg), partial slot.
struct SegDesc {
    int bl, rj, lo, nseg;
    int64_t slot;
};

// The position at cost c of the work sequence (a cost inside a row-start
// charge maps to the start of that row).  Wave-uniform: the batch is found
// with ballots over the slice's batches.
__device__ __forceinline__ int64_t cost_to_pos(const SplitParams &P, int64_t c, int lane) {
    const int64_t gap = (int64_t)P.seg_cost * P.Nkv * P.n_hg;   // row-start charges of one batch
    int cnt = 0;
    for (int e0 = 0; e0 < P.nb; e0 += 64) {
        const int e = e0 + lane;
        cnt += __popcll(__ballot(e < P.nb && P.pre[e] + gap * e <= c));
    }
    const int bl = __builtin_amdgcn_readfirstlane(cnt - 1);
    const int64_t within = c - (P.pre[bl] + gap * bl);
    const int64_t L = P.len[bl], per = L + P.seg_cost;
    if (per == 0) return P.pre[bl];
    const int64_t rj = within / per, t = within - rj * per;
    return P.pre[bl] + (t < L ? rj * L + t : (rj + 1) * L);
}

// Position range [f0, f1) of piece w.
__device__ __forceinline__ void piece_range(const SplitParams &P, int w, int lane, int64_t &f0, int64_t &f1) {
    const int64_t total_cost = P.total + (int64_t)P.seg_cost * P.Nkv * P.n_hg * P.nb;
    const int64_t c0 = (int64_t)w * P.piece, c1 = c0 + P.piece;
    f0 = c0 >= total_cost ? P.total : cost_to_pos(P, c0, lane);
    f1 = c1 >= total_cost ? P.total : cost_to_pos(P, c1, lane);
}

// EXTRA selects the optional score terms compiled in: EX_NONE, EX_MASK
// (attenMask), or EX_PSE (pseShift, with attenMask checked at run time).
template <int KV, int D, int G, bool PAGED, int EXTRA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_per_eu<G>(), 8)))
void split_kernel(const SplitParams P) {
    using C = Cfg<KV, D, G>;
    constexpr int LPR = C::LPR, RPI = C::RPI, W = C::W, EB = C::EB, RT = C::RT, TT = C::TT;
    constexpr bool I8 = KV == KV_I8;
    constexpr bool MASKED = EXTRA != EX_NONE;
    constexpr bool PSE = EXTRA == EX_PSE;
    using DotK = std::integral_constant<int, I8 ? KV_F16 : KV>;
    // heads reduced by reduce-scatter (one head per lane through the softmax)
    // when a KV row fills whole DPP rows and the group has several heads
    constexpr bool SCATTER = LPR >= 16 && G >= 2;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave_id = blockIdx.x * kWavesPerBlock + wave;
    if (wave_id >= P.n_pieces) return;
    const int hl = SCATTER ? head_of_lane<(G >= 2 ? G : 2)>(lane) : 0;   // scatter path: this lane's head
    const int r = lane / LPR;      // row group
    const int c = lane % LPR;      // 8-element slot within the row
    // A head dim below the compiled D: lanes past it re-read the row's last
    // 8-element chunk (every load stays inside the row) and hold a zero query,
    // so they add nothing to the scores; their output columns are never written.
    const int cq = min(c, P.Dr / 8 - 1);
    const bool col_ok = c < P.Dr / 8;
    const char *kb = reinterpret_cast<const char *>(P.k);
    const char *vb = reinterpret_cast<const char *>(P.v);
    const int64_t lane_byte = (int64_t)8 * cq * EB;
    __shared__ int32_t s_tbl[kWavesPerBlock][kTblSlots];
    int32_t *wtbl = s_tbl[wave];

    // This wave's piece of the flattened (batch, KV head, head group,
    // position) space; it is cut into segments at row boundaries, and every
    // segment leaves one partial softmax state.  In row mode workgroup
    // blockIdx.x takes row blockIdx.x of the slice, its waves a quarter of the
    // window each.
    // A row-mode wave knows its one segment from the workgroup id, so it
    // skips the piece lookup and the segment decode (each a dependent read of
    // the batch tables before the first query and K/V loads can issue).
    int64_t f0 = 0, f1 = 0;
    if (I8 || !P.row_mode) piece_range(P, wave_id, lane, f0, f1);
    __shared__ float2 s_ml[kWavesPerBlock][G];   // row mode: each wave's (m, l) per head
    if constexpr (!I8) {
        if (P.row_mode) {
            const int rpb = P.Nkv * P.n_hg;
            const int row = blockIdx.x;
            const int bl = row / rpb, rj = row - bl * rpb;
            const int len = (int)(P.row_win[row] >> 32);
            const int quarter = (len + kWavesPerBlock - 1) / kWavesPerBlock;
            // only the quarter's length matters here: the segment itself comes from row_desc
            f0 = min(len, wave * quarter);
            f1 = min(len, (wave + 1) * quarter);
            if (len == 0) {     // an empty window: zero rows (the whole workgroup returns)
                const int j = rj / P.n_hg, hg = rj - j * P.n_hg;
                using T = std::conditional_t<KV == KV_BF16, __bf16, _Float16>;
                T *o = reinterpret_cast<T *>(P.out) + ((P.b0 + bl) * P.N + j * P.g + hg * G) * (int64_t)P.Dr;
                const int nh = min(G, P.g - hg * G);
                for (int i = threadIdx.x; i < nh * P.Dr; i += 64 * kWavesPerBlock) o[i] = (T)0.f;
                return;
            }
        }
    }
    // Row mode: the wave's quarter of row blockIdx.x (no partial slot).
    auto row_desc = [&]() -> SegDesc {
        const int rpb = P.Nkv * P.n_hg;
        const int row = blockIdx.x;
        const int bl = row / rpb, rj = row - bl * rpb;
        const int64_t w = P.row_win[row];
        const int len = (int)(w >> 32), lo = (int)(uint32_t)w;
        const int quarter = (len + kWavesPerBlock - 1) / kWavesPerBlock;
        const int t0 = min(len, wave * quarter), t1 = min(len, (wave + 1) * quarter);
        return SegDesc{bl, rj, lo + t0, t1 - t0, 0};
    };
    // The segment that starts at position f: its batch is the number of
    // batches whose rows start at or before f.
    auto decode = [&](int64_t f) -> SegDesc {
        int cnt = 0;
        for (int e0 = 0; e0 < P.nb; e0 += 64) {
            const int e = e0 + lane;
            const bool le = e < P.nb && P.pre[e] <= f;
            cnt += __popcll(__ballot(le));
        }
        SegDesc d;
        d.bl = __builtin_amdgcn_readfirstlane(cnt - 1);
        const int len = P.len[d.bl];
        const int64_t within = f - P.pre[d.bl];
        d.rj = (int)(within / len);
        const int t0 = (int)(within - (int64_t)d.rj * len);
        d.nseg = (int)min((int64_t)(len - t0), f1 - f);
        d.lo = P.lo[d.bl] + t0;
        d.slot = P.sbase[d.bl] + (int64_t)d.rj * P.maxseg[d.bl] + (wave_id - row_cost(P, d.bl, d.rj) / P.piece);
        return d;
    };
    // 16-bit query of the head group (register hh holds head hh ^ hl on the
    // scatter path, the lane-dependent order its reduce-scatter needs; head hh
    // otherwise)
    auto load_q16 = [&](uint32_t (&qd)[G][4], int64_t bq, int hbq, int hgq) {
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            const int hq = SCATTER ? hh ^ hl : hh;
            const bool ok = hgq * G + hq < P.g;
            const int64_t off = ((bq * P.N + hbq + (ok ? hq : 0)) * P.Dr + 8 * cq) * 2;
            u32x4 x = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(P.q) + off);
#pragma unroll
            for (int w = 0; w < 4; w++) qd[hh][w] = ok && col_ok ? x[w] : 0u;
        }
    };
    // Dense caches: this lane's pointers into row lo + r of the segment's K and
    // V (tensor lists: batch b's own tensors, batch index 0).
    auto dense_rows = [&](const SegDesc &d, const char *&kq, const char *&vq) {
        const int64_t bq = P.b0 + d.bl;
        const int jq = d.rj / P.n_hg;
        const char *kb_ = kb, *vb_ = vb;
        int64_t boff = bq * P.sB, sN = P.sN;
        if (P.k_list) {
            kb_ = reinterpret_cast<const char *const *>(P.k_list)[bq];
            vb_ = reinterpret_cast<const char *const *>(P.v_list)[bq];
            boff = 0;
            if (P.list_bnsd) sN = (int64_t)P.list_seq[d.bl] * P.sS;
        }
        const int64_t base = (boff + (int64_t)jq * sN) * EB + lane_byte + (int64_t)(d.lo + r) * (P.sS * EB);
        kq = kb_ + base;
        vq = vb_ + base;
    };
    // Plain dense streams chain their segments: during the last tile of a
    // segment the wave requests the next segment's query and first K and V
    // rows, so a new segment starts with its operands already in flight.
    // (Not for D = 64 with head groups of 8: the extra live state would spill.)
    constexpr bool kChain = !PAGED && EXTRA == EX_NONE && !I8 && !(D == 64 && G == 8);
    bool pref = false;                  // the next segment's query and first tile are in flight
    SegDesc nx{0, 0, 0, 0, 0};
    uint32_t qv[G][4];
    uint32_t kr[RT][W], vr[RT][W];
    for (int64_t f = f0; f < f1;) {
        const bool chained = kChain && pref;
        pref = false;
        const SegDesc sg = chained ? nx : (!I8 && P.row_mode) ? row_desc() : decode(f);
        const int bl = sg.bl, rj = sg.rj, nseg = sg.nseg;   // row of the batch: j * n_hg + hg
        const int j = rj / P.n_hg, hg = rj - j * P.n_hg;
        const int lo = sg.lo;
        const int hi = lo + nseg;
        const int64_t b = P.b0 + bl;
        const int64_t slot = sg.slot;

        // ------------------------------------------------------ query
        const int hbase = j * P.g + hg * G;
        float qmul = P.score_mul;
        if constexpr (!I8) {
            if (!chained) load_q16(qv, b, hbase, hg);
        } else {
            // q' = q * s_K (K's antiquant scale) in fp16, multiplied by a power
            // of two so the largest |q'| of the wave sits just under 2^15; the
            // score multiplier takes the inverse power.  The K offset adds a
            // constant per row and drops out of the softmax.
            float qf[G][8];
            float amax = 0.f;
#pragma unroll
            for (int hh = 0; hh < G; hh++) {
                const int hq = SCATTER ? hh ^ hl : hh;
                const bool ok = hg * G + hq < P.g && col_ok;
                const int64_t off = ((b * P.N + hbase + (ok ? hq : 0)) * P.Dr + 8 * cq) * 2;
                const u32x4 x = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(P.q) + off);
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const uint32_t bits = (x[e >> 1] >> (16 * (e & 1))) & 0xFFFF;
                    float qe = P.q_bf16 ? bf16_to_f32(bits) : f16_to_f32(bits);
                    const int64_t si = (P.aq_mode == 1) ? 0 : (int64_t)j * P.Dr + 8 * cq + e;
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

        // ------------------------------------------------------ addressing
        // Dense: this lane's pointers to row (lo + r) of K and V; row i of the
        // tile at ts is (ts - lo + i*RPI) row strides further (a uniform offset).
        const char *kp = nullptr, *vp_ = nullptr;
        int64_t sS_b = 0;
        if constexpr (!PAGED) {
            sS_b = P.sS * EB;
            dense_rows(sg, kp, vp_);
        }
        const int lim = hi - 1 - lo - r;     // last valid row index relative to row lo + r
        // Paged: the block ids of the segment are staged into this wave's LDS
        // slots (one coalesced load), so finding a row costs an LDS read.
        const int32_t *btab = nullptr;
        int q_first = 0;
        bool tbl_in_lds = false;
        const bool two_blk = PAGED && P.block_size >= TT;   // a tile spans at most two blocks
        uint32_t blk_b = 0, head_b = 0, row_b = 0;
        if constexpr (PAGED) {
            btab = P.block_table + b * P.max_blocks;
            blk_b = (uint32_t)(P.blk_stride * EB);
            head_b = (uint32_t)(P.head_stride * EB) * (uint32_t)j;
            row_b = (uint32_t)(P.row_stride * EB);
            q_first = (int)div_bs((uint32_t)lo, P.bs_magic, P.bs_shift);
            const int q_last = (int)div_bs((uint32_t)(hi - 1), P.bs_magic, P.bs_shift);
            tbl_in_lds = q_last - q_first < kTblSlots;
            if (tbl_in_lds) {
                for (int e = lane; e <= q_last - q_first; e += 64) wtbl[e] = btab[q_first + e];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        }
        const uint8_t *mrow = nullptr;
        if constexpr (MASKED) {
            if (P.mask) mrow = P.mask + (P.mask_sB ? b * P.mask_sB : 0) + (int64_t)hbase * P.mask_sH;
        }
        // pseShift row(s) of this lane.  Scatter path: the lane's own head, at
        // the RT positions whose scores it holds.  Other path: every head of
        // the group at position ts + lane (a coalesced read), fetched from the
        // owning lane when the scores are scaled.  Heads past the group read
        // head 0 of it; their scores are never stored.
        constexpr int PH = PSE ? (SCATTER ? 1 : G) : 1;
        constexpr int PR = PSE && SCATTER ? RT : 1;
        const uint16_t *prow[PH];
        bool pse_bf16 = false;
        if constexpr (PSE) {
            pse_bf16 = I8 ? P.q_bf16 != 0 : KV == KV_BF16;
            const uint16_t *pb = reinterpret_cast<const uint16_t *>(P.pse) + (P.pse_sB ? b * P.pse_sB : 0);
#pragma unroll
            for (int hh = 0; hh < PH; hh++) {
                const int hq = SCATTER ? hl : hh;
                prow[hh] = pb + (int64_t)(hbase + (hg * G + hq < P.g ? hq : 0)) * P.pse_sH;
            }
        }

        // Rolling pipeline with one tile resident: the K rows of tile k+1 are
        // requested as soon as QK of tile k has consumed the K registers, and
        // its V rows as soon as PV of tile k has consumed the V registers.
        // With a mask, the mask bytes run one tile further ahead, so the rows
        // every head of the group excludes are never read: their registers
        // keep the previous tile's (finite) values, and their p is 0.
        constexpr int MB = MASKED ? G : 1;
        if (!chained) {
#pragma unroll
            for (int i = 0; i < RT; i++)
#pragma unroll
                for (int w = 0; w < W; w++) kr[i][w] = vr[i][w] = 0u;
        }
        bool okr[RT];
        uint32_t mbr[MB];       // mask byte of position ts + lane (per head for per-head masks), one tile ahead
        uint32_t pbr[PR][PH];   // pseShift bits: scatter path of ts + i*RPI + r, else of ts + lane
        int64_t offs[RT];       // paged: byte offsets of the tile's rows

        // The row pointers are global memory.  Saying so keeps the loads global
        // (vector memory counter only) where the compiler could not infer it
        // (bases read from memory or chosen at run time), instead of flat loads
        // that also count against the LDS counter: int8 kernels run 11 % faster.
        // The plain dense 16-bit kernels with head groups of 2 or 4 (one wave
        // per SIMD) are the exception: there the flat loads, waited for all at
        // once, measured 4-6 % faster on BSH caches and no slower on BNSD ones.
        constexpr bool kFlatRows = !PAGED && EXTRA == EX_NONE && !I8 && (G == 2 || G == 4);
        auto load_rows = [&](const char *const (&ptr)[RT], uint32_t (&dst)[RT][W], uint64_t skip) {
#pragma unroll
            for (int i = 0; i < RT; i++) {
                if constexpr (MASKED) {
                    if ((skip >> (i * RPI + r)) & 1) continue;     // excluded for every head: not read
                }
                if constexpr (W == 4) {
                    const u32x4 x = kFlatRows ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ptr[i]))
                                              : __builtin_nontemporal_load((const gu32x4 *)ptr[i]);
                    dst[i][0] = x[0]; dst[i][1] = x[1]; dst[i][2] = x[2]; dst[i][3] = x[3];
                } else {
                    const u32x2 x = __builtin_nontemporal_load((const gu32x2 *)ptr[i]);
                    dst[i][0] = x[0]; dst[i][1] = x[1];
                }
            }
        };
        auto row_ptrs = [&](int ts, const char *base, const char *(&ptr)[RT]) {
            if constexpr (!PAGED) {
                if (ts + TT <= hi) {
#pragma unroll
                    for (int i = 0; i < RT; i++) ptr[i] = base + (int64_t)(ts - lo + i * RPI) * sS_b;
                } else {
#pragma unroll
                    for (int i = 0; i < RT; i++) ptr[i] = base + (int64_t)min(ts - lo + i * RPI, lim) * sS_b;
                }
            } else {
#pragma unroll
                for (int i = 0; i < RT; i++) ptr[i] = base + offs[i];
            }
        };
        auto issue_k = [&](int ts, uint64_t skip) {
            if constexpr (PAGED) {
              if (two_blk) {
                // A tile spans at most two blocks, q0 and q1 (q1 = q0 or q0 + 1):
                // two uniform block-id reads, and per row a select between the
                // two block bases by the row's place in block q0.
                const int last = min(ts + TT, hi) - 1;
                const uint32_t q0 = div_bs((uint32_t)ts, P.bs_magic, P.bs_shift);
                const uint32_t q1 = div_bs((uint32_t)last, P.bs_magic, P.bs_shift);
                int b0, b1;
                if (tbl_in_lds) {
                    const __attribute__((address_space(3))) int32_t *lt = (const __attribute__((address_space(3))) int32_t *)wtbl;
                    b0 = lt[q0 - q_first];
                    b1 = lt[q1 - q_first];
                } else {
                    const __attribute__((address_space(1))) int32_t *gt = (const __attribute__((address_space(1))) int32_t *)btab;
                    b0 = gt[q0];
                    b1 = gt[q1];
                }
                b0 = __builtin_amdgcn_readfirstlane(b0);
                b1 = __builtin_amdgcn_readfirstlane(b1);
                const bool ok0 = (unsigned)b0 < (unsigned)P.num_blocks, ok1 = (unsigned)b1 < (unsigned)P.num_blocks;
                // row offset within block q0 of tile row 0, and of the last row
                const int rel0 = ts - (int)q0 * P.block_size, rel_last = last - (int)q0 * P.block_size;
                // base of block q0, and of block q1 shifted back by one block's rows
                const int64_t s0 = (int64_t)(uint32_t)b0 * blk_b + head_b;
                const int64_t s1 = (int64_t)(uint32_t)b1 * blk_b + head_b - (int64_t)P.block_size * row_b;
#pragma unroll
                for (int i = 0; i < RT; i++) {
                    const int rel = min(rel0 + i * RPI + r, rel_last);
                    const bool sel = rel >= P.block_size;
                    okr[i] = sel ? ok1 : ok0;
                    offs[i] = okr[i] ? (sel ? s1 : s0) + (int64_t)((uint32_t)rel * row_b) + lane_byte : 0;
                }
              } else {
#pragma unroll
                for (int i = 0; i < RT; i++) {
                    const int t = min(ts + i * RPI + r, hi - 1);
                    const uint32_t q = div_bs((uint32_t)t, P.bs_magic, P.bs_shift);
                    const uint32_t rr = (uint32_t)t - q * (uint32_t)P.block_size;
                    // two loads in their own address spaces (a pointer select would
                    // make one flat load that stalls on both memory counters)
                    int blk;
                    if (tbl_in_lds) blk = ((const __attribute__((address_space(3))) int32_t *)wtbl)[q - q_first];
                    else blk = ((const __attribute__((address_space(1))) int32_t *)btab)[q];
                    okr[i] = (unsigned)blk < (unsigned)P.num_blocks;
                    // never dereference an out-of-range block id: read block 0 instead
                    offs[i] = okr[i] ? (int64_t)(uint32_t)blk * blk_b + (head_b + rr * row_b) + lane_byte : 0;
                }
              }
            }
            const char *ptr[RT];
            row_ptrs(ts, PAGED ? kb : kp, ptr);
            load_rows(ptr, kr, skip);
        };
        // mask bytes of the tile at ts: position ts + lane, lanes < TT
        auto load_mask = [&](int ts) {
            if constexpr (MASKED) {
                const int tm = min(ts + lane, hi - 1);
#pragma unroll
                for (int hh = 0; hh < MB; hh++) {
                    // shared mask: only entry 0; per-head mask: one byte per real head
                    const bool want = lane < TT && (P.mask_mode == 2 ? hg * G + hh < P.g : P.mask_mode == 1 && hh == 0);
                    uint32_t v = 0;
                    if (want) v = mrow[(int64_t)hh * P.mask_sH + tm];
                    mbr[hh] = v;
                }
            }
        };
        // the loaded mask bytes as per-head bitmaps (bit = position in the tile),
        // and the positions that every real head of the group excludes
        auto mask_bits = [&](uint64_t (&bits)[MB]) -> uint64_t {
            uint64_t all = 0;
            if constexpr (MASKED) {
                if (P.mask_mode == 1) {
                    bits[0] = __ballot(mbr[0] != 0);
#pragma unroll
                    for (int hh = 1; hh < MB; hh++) bits[hh] = bits[0];
                    all = bits[0];
                } else {
                    all = ~0ull;
#pragma unroll
                    for (int hh = 0; hh < MB; hh++) {
                        bits[hh] = __ballot(mbr[hh] != 0);
                        if (hg * G + hh < P.g) all &= bits[hh];
                    }
                    if (P.mask_mode == 0) all = 0;
                }
            }
            return all;
        };
        auto issue_pse = [&](int ts) {
            if constexpr (PSE && SCATTER) {
#pragma unroll
                for (int i = 0; i < RT; i++) pbr[i][0] = prow[0][min(ts + i * RPI + r, hi - 1)];
            } else if constexpr (PSE) {
                const int t = min(ts + lane, hi - 1);
#pragma unroll
                for (int hh = 0; hh < PH; hh++) pbr[0][hh] = lane < TT ? prow[hh][t] : 0u;
            }
        };
        auto pse_log2 = [&](uint32_t bits) {
            return (pse_bf16 ? bf16_to_f32(bits) : f16_to_f32(bits)) * kLog2e;
        };
        auto issue_v = [&](int ts, uint64_t skip) {
            const char *ptr[RT];
            row_ptrs(ts, PAGED ? vb : vp_, ptr);
            load_rows(ptr, vr, skip);
        };

        float m[G], l[G], acc[G][8];
#pragma unroll
        for (int hh = 0; hh < G; hh++) {
            m[hh] = kMaxInit;
            l[hh] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) acc[hh][e] = 0.f;
        }
        float m1 = kMaxInit, l1 = 0.f;      // scatter path: state of this lane's head hl

        // -------------------------------------------------- main loop
        int ts = lo;
        uint64_t mcur[MB], mnext[MB];     // per-head mask bitmaps of this tile and the next
        uint64_t skip_cur = 0, skip_next = 0;
#pragma unroll
        for (int hh = 0; hh < MB; hh++) mcur[hh] = mnext[hh] = 0;
        if constexpr (MASKED) {
            load_mask(ts);
            skip_cur = mask_bits(mcur);
        }
        if (!chained) issue_k(ts, skip_cur);
        if constexpr (MASKED) {
            if (ts + TT < hi) load_mask(ts + TT);
        }
        if (!chained) issue_v(ts, skip_cur);
        issue_pse(ts);
        while (true) {
            // QK: partial dot products of the resident K rows, then the DPP
            // reductions one step at a time across all rows and heads
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
                    float a = dot2_first(qv[hh][0], kk[0], DotK{});
#pragma unroll
                    for (int w = 1; w < 4; w++) a = dot2(qv[hh][w], kk[w], a, DotK{});
                    s[i][hh] = a;
                }
            }
            float x[RT];        // scatter path: this lane's head, per row step
            if constexpr (SCATTER) {
#pragma unroll
                for (int i = 0; i < RT; i++) x[i] = scatter_reduce<G, LPR>(s[i]);
            }
            if constexpr (!SCATTER && LPR >= 2) {
#pragma unroll
                for (int i = 0; i < RT; i++)
#pragma unroll
                    for (int hh = 0; hh < G; hh++) s[i][hh] += dpp<0xB1>(s[i][hh]);   // quad_perm [1,0,3,2]
            }
            if constexpr (!SCATTER && LPR >= 4) {
#pragma unroll
                for (int i = 0; i < RT; i++)
#pragma unroll
                    for (int hh = 0; hh < G; hh++) s[i][hh] += dpp<0x4E>(s[i][hh]);   // quad_perm [2,3,0,1]
            }
            if constexpr (!SCATTER && LPR >= 8) {
#pragma unroll
                for (int i = 0; i < RT; i++)
#pragma unroll
                    for (int hh = 0; hh < G; hh++) s[i][hh] += dpp<0x141>(s[i][hh]);  // row_half_mirror
            }
            if constexpr (!SCATTER && LPR >= 16) {
#pragma unroll
                for (int i = 0; i < RT; i++)
#pragma unroll
                    for (int hh = 0; hh < G; hh++) s[i][hh] += dpp<0x140>(s[i][hh]);  // row_mirror
            }
            if constexpr (!SCATTER && LPR >= 32) {
#pragma unroll
                for (int i = 0; i < RT; i++)
#pragma unroll
                    for (int hh = 0; hh < G; hh++) s[i][hh] += swz_xor16(s[i][hh]);
            }
            if constexpr (!SCATTER && LPR >= 64) {
#pragma unroll
                for (int i = 0; i < RT; i++)
#pragma unroll
                    for (int hh = 0; hh < G; hh++) s[i][hh] += __shfl_xor(s[i][hh], 32);
            }

            // validity bitmaps of the tile, taken before the next tile's
            // loads reuse the registers
            uint64_t mbits[MB];
#pragma unroll
            for (int hh = 0; hh < MB; hh++) mbits[hh] = mcur[hh];
            bool okc[RT];
#pragma unroll
            for (int i = 0; i < RT; i++) okc[i] = PAGED ? okr[i] : true;

            const bool more = ts + TT < hi;
            if (more) {
                if constexpr (MASKED) {
                    skip_next = mask_bits(mnext);          // the mask loaded one tile ago
                    if (ts + 2 * TT < hi) load_mask(ts + 2 * TT);
                }
                issue_k(ts + TT, skip_next);
            }
            // last tile: the next segment's query and K rows, into the
            // registers this tile's scores have consumed
            const char *nvp = nullptr;
            int nlim = 0;
            if constexpr (kChain) {
                if (!more && f + nseg < f1) {
                    nx = decode(f + nseg);
                    const int nj = nx.rj / P.n_hg, nhg = nx.rj - nj * P.n_hg;
                    load_q16(qv, P.b0 + nx.bl, nj * P.g + nhg * G, nhg);
                    const char *nkp;
                    dense_rows(nx, nkp, nvp);
                    nlim = nx.nseg - 1 - r;
                    const char *ptr[RT];
#pragma unroll
                    for (int i = 0; i < RT; i++) ptr[i] = nkp + (int64_t)min(i * RPI, nlim) * sS_b;
                    load_rows(ptr, kr, 0);
                    pref = true;
                }
            }

            if constexpr (SCATTER) {
                // this lane's head: mask bitmap, scale, online softmax, then
                // every head's p fetched back from the lanes that hold them
                uint64_t mbl = 0;
                if constexpr (MASKED) {
                    mbl = mbits[0];
#pragma unroll
                    for (int hh = 1; hh < MB; hh++) mbl = hl == hh ? mbits[hh] : mbl;
                }
                float mt = kNegInf;
#pragma unroll
                for (int i = 0; i < RT; i++) {
                    const int pos = i * RPI + r;
                    bool keep = ts + pos < hi && okc[i];
                    if constexpr (MASKED) keep = keep && !((mbl >> pos) & 1);
                    float xs = x[i] * qmul;
                    if constexpr (PSE) xs += pse_log2(pbr[i][0]);
                    x[i] = keep ? xs : kNegInf;
                    mt = fmaxf(mt, x[i]);
                }
                const bool raise = mt > m1 + kLazy;
                if (__builtin_amdgcn_ballot_w64(raise)) {
                    const float mn = raise ? mt : m1;
                    const float alpha = __builtin_amdgcn_exp2f(m1 - mn);
                    m1 = mn;
                    l1 *= alpha;
                    float ah[G];
                    gather_heads<G>(alpha, ah);
#pragma unroll
                    for (int hh = 0; hh < G; hh++)
#pragma unroll
                        for (int e = 0; e < 8; e++) acc[hh][e] *= ah[hh];
                }
                float ls = 0.f;
#pragma unroll
                for (int i = 0; i < RT; i++) {
                    x[i] = __builtin_amdgcn_exp2f(x[i] - m1);
                    ls += x[i];
                    gather_heads<G>(x[i], s[i]);
                }
                l1 += ls;
            } else {
                // scale; exclude positions past the segment, out-of-range blocks and masked ones
#pragma unroll
                for (int i = 0; i < RT; i++) {
                    const int pos = i * RPI + r;             // position within the tile
                    const bool in = ts + pos < hi && okc[i];
#pragma unroll
                    for (int hh = 0; hh < G; hh++) {
                        bool keep = in;
                        if constexpr (MASKED) keep = keep && !((mbits[hh] >> pos) & 1);
                        float xs = s[i][hh] * qmul;
                        if constexpr (PSE) xs += pse_log2((uint32_t)__shfl((int)pbr[0][hh], pos));
                        s[i][hh] = keep ? xs : kNegInf;
                    }
                }
                // online softmax (log2 domain) with a lazily raised maximum
                float mt[G];
                bool raise = false;
#pragma unroll
                for (int hh = 0; hh < G; hh++) {
                    mt[hh] = s[0][hh];
#pragma unroll
                    for (int i = 1; i < RT; i++) mt[hh] = fmaxf(mt[hh], s[i][hh]);
                    raise |= mt[hh] > m[hh] + kLazy;
                }
                if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
                    for (int hh = 0; hh < G; hh++) {
                        const float mn = mt[hh] > m[hh] + kLazy ? mt[hh] : m[hh];
                        const float alpha = __builtin_amdgcn_exp2f(m[hh] - mn);
                        m[hh] = mn;
                        l[hh] *= alpha;
#pragma unroll
                        for (int e = 0; e < 8; e++) acc[hh][e] *= alpha;
                    }
                }
#pragma unroll
                for (int hh = 0; hh < G; hh++) {
                    float ls = 0.f;
#pragma unroll
                    for (int i = 0; i < RT; i++) {
                        s[i][hh] = __builtin_amdgcn_exp2f(s[i][hh] - m[hh]);
                        ls += s[i][hh];
                    }
                    l[hh] += ls;
                }
            }
            // the next tile's bias is read while this tile's P.V runs
            if (more) issue_pse(ts + TT);
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
                    const uint32_t pp = pack_p(s[i][hh], s[i + 1][hh], DotK{});
#pragma unroll
                    for (int e = 0; e < 8; e++) acc[hh][e] = dot2(pp, vp[e], acc[hh][e], DotK{});
                }
            }
            if (!more) {
                if constexpr (kChain) {
                    if (pref) {
                        const char *ptr[RT];
#pragma unroll
                        for (int i = 0; i < RT; i++) ptr[i] = nvp + (int64_t)min(i * RPI, nlim) * sS_b;
                        load_rows(ptr, vr, 0);
                    }
                }
                break;
            }
            issue_v(ts + TT, skip_next);
#pragma unroll
            for (int hh = 0; hh < MB; hh++) mcur[hh] = mnext[hh];
            ts += TT;
        }

        if constexpr (SCATTER) {
            gather_heads<G>(m1, m);
            gather_heads<G>(l1, l);
        }

        // ------------------------------------------------------ merge row groups
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

        if constexpr (!I8) {
            if (P.row_mode) {   // the wave's quarter of the row goes to LDS for the merge below
                if (r == 0) {
                    extern __shared__ __attribute__((aligned(16))) float s_part[];   // [wave][G][D]
#pragma unroll
                    for (int hh = 0; hh < G; hh++) {
                        float4 *dst = reinterpret_cast<float4 *>(s_part + (wave * G + hh) * D + 8 * c);
                        dst[0] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
                        dst[1] = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
                        if (c == 0) s_ml[wave][hh] = make_float2(m[hh], l[hh]);
                    }
                }
                f += nseg;
                continue;
            }
        }
        if (r == 0) {
#pragma unroll
            for (int hh = 0; hh < G; hh++) {
                if (hg * G + hh >= P.g) break;
                const int64_t row = slot * G + hh;
                float4 *dst = reinterpret_cast<float4 *>(P.part_acc + row * D + 8 * c);
                dst[0] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
                dst[1] = make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
                if (c == 0) *reinterpret_cast<float2 *>(P.part_ml + row * 2) = make_float2(m[hh], l[hh]);
            }
        }
        f += nseg;
    }   // segments

    if constexpr (!I8) {
        if (P.row_mode) {
            // Merge the four quarters of the row in a fixed order (a wave with
            // an empty quarter contributes nothing), normalise, round to
            // nearest even and write the output.
            extern __shared__ __attribute__((aligned(16))) float s_part[];   // [wave][G][D]
            if (f0 == f1) {
                for (int i = lane; i < G * D; i += 64) s_part[wave * G * D + i] = 0.f;
                if (lane < G) s_ml[wave][lane] = make_float2(kMaxInit, 0.f);
            }
            __syncthreads();
            const int rpb = P.Nkv * P.n_hg;
            const int row = blockIdx.x;
            const int bl = row / rpb, rj = row - bl * rpb;
            const int j = rj / P.n_hg, hg = rj - j * P.n_hg;
            const int nh = min(G, P.g - hg * G);
            using T = std::conditional_t<KV == KV_BF16, __bf16, _Float16>;
            typedef T t8 __attribute__((ext_vector_type(8)));
            T *o = reinterpret_cast<T *>(P.out) + ((P.b0 + bl) * P.N + j * P.g + hg * G) * (int64_t)P.Dr;
            const int nc = P.Dr / 8;                   // output chunks of 8 columns per head
            for (int it = threadIdx.x; it < nh * nc; it += 64 * kWavesPerBlock) {
                const int hh = it / nc, c8 = it - hh * nc;
                float mx = kMaxInit;
#pragma unroll
                for (int w = 0; w < kWavesPerBlock; w++) mx = fmaxf(mx, s_ml[w][hh].x);
                float L = 0.f, a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < kWavesPerBlock; w++) {
                    const float2 ml = s_ml[w][hh];
                    const float wt = __builtin_amdgcn_exp2f(ml.x - mx);
                    L += ml.y * wt;
                    const float4 *src = reinterpret_cast<const float4 *>(s_part + (w * G + hh) * D + 8 * c8);
                    const float4 x0 = src[0], x1 = src[1];
                    a[0] += x0.x * wt; a[1] += x0.y * wt; a[2] += x0.z * wt; a[3] += x0.w * wt;
                    a[4] += x1.x * wt; a[5] += x1.y * wt; a[6] += x1.z * wt; a[7] += x1.w * wt;
                }
                t8 v;
#pragma unroll
                for (int e = 0; e < 8; e++) v[e] = (T)(L > 0.f ? a[e] / L : 0.f);
                *reinterpret_cast<t8 *>(o + hh * P.Dr + 8 * c8) = v;
            }
        }
    }
}

// int8 cache, D = 128, head groups of 8, dense, no mask or bias: the
// query-key products run on the matrix cores.  The query, scaled by K's
// antiquant scale and a power of two to |q'| < 2^14 and rounded to an
// integer, is split into q' = 128 a + b with a in [-128, 127], b in [0, 127];
// two v_mfma_i32_16x16x64_i8 products per 64 dimensions (a and b parts
// against the raw int8 keys) give the exact integer score 128 A + B of 16
// rows x 16 heads (8 real) per tile, with no byte widening of K at all.
// Lane (n, g) of the result holds row n of heads 4g .. 4g+3: the online
// softmax runs there, with the tile maximum per head taken over the integer
// scores (a 16-lane DPP reduction).  P.V runs on the matrix cores too: P and
// the tile's V rows, widened to fp16, are staged in the wave's LDS and read
// back transposed as the operands of one v_mfma_f32_16x16x16_f16 per 16
// output columns.  K and V tiles are loaded two tiles ahead, from scalar row
// bases with fixed per-lane offsets.
template <int KV>   // KV_I8 only (a template so each translation unit may include it)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
void split_kernel_i8m(const SplitParams P) {
    constexpr int D = 128, G = 8, RT = 4, RPI = 4, LPR = 16, TT = 16, KS = D / 64;
    // fp16 V tile rows at a 288-byte pitch: the transposed reads of a 16-lane
    // group (4 rows x 32 bytes) then fall in distinct banks
    constexpr int kVtPitch = 2 * D + 32;
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) i32x4 gi32x4;
    typedef float floatx4 __attribute__((ext_vector_type(4)));
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    typedef short shortx4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) char s_vt[kWavesPerBlock][16 * kVtPitch];
    __shared__ __attribute__((aligned(16))) char s_pp[kWavesPerBlock][16 * 32];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave_id = blockIdx.x * kWavesPerBlock + wave;
    if (wave_id >= P.n_pieces) return;
    const int r = lane / LPR, c = lane % LPR;      // V rows: row group r, 8-byte chunk c
    const int n = lane & 15, grp = lane >> 4;       // matrix layout: tile row n, k slice / head group
    const char *kb = reinterpret_cast<const char *>(P.k);
    const char *vb = reinterpret_cast<const char *>(P.v);

    int64_t f0 = 0, f1 = 0;
    piece_range(P, wave_id, lane, f0, f1);
    for (int64_t f = f0; f < f1;) {
        int cnt = 0;
        for (int e0 = 0; e0 < P.nb; e0 += 64) {
            const int e = e0 + lane;
            cnt += __popcll(__ballot(e < P.nb && P.pre[e] <= f));
        }
        const int bl = __builtin_amdgcn_readfirstlane(cnt - 1);
        const int len = P.len[bl];
        const int64_t within = f - P.pre[bl];
        const int rj = (int)(within / len);
        const int t0 = (int)(within - (int64_t)rj * len);
        const int nseg = (int)min((int64_t)(len - t0), f1 - f);
        const int j = rj / P.n_hg, hg = rj - j * P.n_hg;
        const int lo = P.lo[bl] + t0;
        const int hi = lo + nseg;
        const int64_t b = P.b0 + bl;
        const int64_t slot = P.sbase[bl] + (int64_t)rj * P.maxseg[bl] + (wave_id - row_cost(P, bl, rj) / P.piece);
        const int hbase = j * P.g + hg * G;

        // ------------------------------------------------ query (matrix A operand)
        // lane (n, grp): head n (real when n < 8 and inside the group), dims 64 ks + 16 grp + e
        const bool hok = n < G && hg * G + n < P.g;
        float qf[KS][16];
        float amax = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const int d0 = 64 * ks + 16 * grp;
            const char *qp = reinterpret_cast<const char *>(P.q) + ((b * P.N + hbase + (hok ? n : 0)) * D + d0) * 2;
            const u32x4 x0 = *reinterpret_cast<const u32x4 *>(qp), x1 = *reinterpret_cast<const u32x4 *>(qp + 16);
            u32x4 s0 = {0, 0, 0, 0}, s1 = {0, 0, 0, 0};
            if (P.aq_mode == 2) {
                const char *sp = reinterpret_cast<const char *>(P.k_scale) + ((int64_t)j * D + d0) * 2;
                s0 = *reinterpret_cast<const u32x4 *>(sp);
                s1 = *reinterpret_cast<const u32x4 *>(sp + 16);
            }
            const uint32_t s_all = reinterpret_cast<const uint16_t *>(P.k_scale)[0];
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const uint32_t qw = e < 8 ? x0[e >> 1] : x1[(e - 8) >> 1];
                const uint32_t sw = e < 8 ? s0[e >> 1] : s1[(e - 8) >> 1];
                const uint32_t qbits = (qw >> (16 * (e & 1))) & 0xFFFF;
                const uint32_t sbits = P.aq_mode == 2 ? (sw >> (16 * (e & 1))) & 0xFFFF : s_all;
                const float qe = P.q_bf16 ? bf16_to_f32(qbits) : f16_to_f32(qbits);
                const float se = P.q_bf16 ? bf16_to_f32(sbits) : f16_to_f32(sbits);
                qf[ks][e] = hok ? qe * se : 0.f;
                amax = fmaxf(amax, fabsf(qf[ks][e]));
            }
        }
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        int ex = 0;
        if (amax > 0.f) (void)frexpf(amax, &ex);        // amax < 2^ex
        // the sign of the score factor goes into q, so the factor is positive
        const float up = P.score_mul < 0.f ? -ldexpf(1.f, 14 - ex) : ldexpf(1.f, 14 - ex);
        const float qmul = fabsf(P.score_mul) * ldexpf(1.f, ex - 14);
        i32x4 qa[KS], qb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int w = 0; w < 4; w++) {
                uint32_t wa = 0, wb = 0;
#pragma unroll
                for (int e4 = 0; e4 < 4; e4++) {
                    int qi = (int)__builtin_rintf(qf[ks][4 * w + e4] * up);
                    qi = min(max(qi, -16383), 16383);
                    const int a = qi >> 7;                   // floor(qi / 128), in [-128, 127]
                    const int bb = qi - (a << 7);            // in [0, 127]
                    wa |= (uint32_t)(a & 0xFF) << (8 * e4);
                    wb |= (uint32_t)bb << (8 * e4);
                }
                qa[ks][w] = (int32_t)wa;
                qb[ks][w] = (int32_t)wb;
            }

        // ------------------------------------------------ addressing (dense, or per-batch tensors)
        const int64_t sS_b = P.sS;                     // int8: element stride = byte stride
        const char *kb_ = kb, *vb_ = vb;
        int64_t boff = b * P.sB, sN = P.sN;
        if (P.k_list) {
            kb_ = reinterpret_cast<const char *const *>(P.k_list)[b];
            vb_ = reinterpret_cast<const char *const *>(P.v_list)[b];
            boff = 0;
            if (P.list_bnsd) sN = (int64_t)P.list_seq[bl] * P.sS;
        }
        // wave-uniform row bases (scalar registers) plus fixed 32-bit lane
        // offsets: every load is a saddr + voffset global load
        const char *kbase = uniform_ptr(kb_ + boff + (int64_t)j * sN);
        const char *vbase = uniform_ptr(vb_ + boff + (int64_t)j * sN);
        const uint32_t sSu = (uint32_t)sS_b;
        const uint32_t koff = (uint32_t)n * sSu + 16u * grp;
        uint32_t voff[RT];
#pragma unroll
        for (int i = 0; i < RT; i++) voff[i] = (uint32_t)(i * RPI + r) * sSu + 8u * c;
        // K and V tiles run two deep: buffers A and B alternate, so a tile's
        // registers are reloaded only once its products are issued
        i32x4 kA[KS], kB[KS];
        uint32_t vA[RT][2], vB[RT][2];
#pragma unroll
        for (int i = 0; i < RT; i++) vA[i][0] = vA[i][1] = vB[i][0] = vB[i][1] = 0u;
        // a tile that runs past hi re-reads its last row in the lanes beyond it
        auto issue_k = [&](i32x4 (&kt)[KS], int ts) {
            const char *tb = kbase + (int64_t)ts * sS_b;
            uint32_t o = koff;
            if (ts + TT > hi) o = min((uint32_t)n, (uint32_t)(hi - 1 - ts)) * sSu + 16u * grp;
#pragma unroll
            for (int ks = 0; ks < KS; ks++) kt[ks] = __builtin_nontemporal_load((const gi32x4 *)(tb + o + 64 * ks));
        };
        auto issue_v = [&](uint32_t (&vr)[RT][2], int ts) {
            const char *tb = vbase + (int64_t)ts * sS_b;
            const bool part = ts + TT > hi;
#pragma unroll
            for (int i = 0; i < RT; i++) {
                uint32_t o = voff[i];
                if (part) o = min((uint32_t)(i * RPI + r), (uint32_t)(hi - 1 - ts)) * sSu + 8u * c;
                const u32x2 x = __builtin_nontemporal_load((const gu32x2 *)(tb + o));
                vr[i][0] = x[0];
                vr[i][1] = x[1];
            }
        };

        float m4[4], l4[4];
        floatx4 oacc[D / 16];        // O[4 grp + i][16 blk + n]
#pragma unroll
        for (int i = 0; i < 4; i++) {
            m4[i] = kMaxInit;
            l4[i] = 0.f;
        }
#pragma unroll
        for (int blk = 0; blk < D / 16; blk++) oacc[blk] = floatx4{0.f, 0.f, 0.f, 0.f};

        int ts = lo;
        char *pw = s_pp[wave];
        char *vw = s_vt[wave];
        // one tile: products with K in kt, V in vr; both are refilled with the
        // tile two ahead.  Returns whether another tile follows.
        auto tile = [&](i32x4 (&kt)[KS], uint32_t (&vr)[RT][2]) -> bool {
            i32x4 ca = {0, 0, 0, 0}, cb = {0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                ca = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[ks], kt[ks], ca, 0, 0, 0);
                cb = __builtin_amdgcn_mfma_i32_16x16x64_i8(qb[ks], kt[ks], cb, 0, 0, 0);
            }
            const bool more = ts + TT < hi, more2 = ts + 2 * TT < hi;
            if (more2) issue_k(kt, ts + 2 * TT);

            // scores of heads 4 grp + i at tile row n; the tile maximum per head
            const bool keep = ts + n < hi;
            float x[4], mt[4];
            // the maximum is taken over the integer scores (the scale factor
            // is positive, so it commutes with the rounding of the products);
            // row 0 of a tile is always inside the window
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int si = ca[i] * 128 + cb[i];
                x[i] = keep ? (float)si * qmul : kNegInf;
                int v = keep ? si : (-2147483647 - 1);
                v = max(v, dppi<0xB1>(v));
                v = max(v, dppi<0x4E>(v));
                v = max(v, dppi<0x141>(v));
                v = max(v, dppi<0x140>(v));
                mt[i] = (float)v * qmul;
            }
            bool raise = false;
#pragma unroll
            for (int i = 0; i < 4; i++) raise |= mt[i] > m4[i] + kLazy;
            if (__builtin_amdgcn_ballot_w64(raise)) {
                float alpha[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float mn = mt[i] > m4[i] + kLazy ? mt[i] : m4[i];
                    alpha[i] = __builtin_amdgcn_exp2f(m4[i] - mn);
                    m4[i] = mn;
                    l4[i] *= alpha[i];
                }
#pragma unroll
                for (int blk = 0; blk < D / 16; blk++)
#pragma unroll
                    for (int i = 0; i < 4; i++) oacc[blk][i] *= alpha[i];
            }
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                p[i] = __builtin_amdgcn_exp2f(x[i] - m4[i]);
                l4[i] += p[i];
            }
            // P stored row-major by tile row (16 heads per row): one 8-byte write per lane
            {
                f16x4 ph = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
                *reinterpret_cast<f16x4 *>(pw + n * 32 + 8 * grp) = ph;
            }
#pragma unroll
            for (int i = 0; i < RT; i++) {
                const uint32_t w0 = vr[i][0] ^ 0x80808080u, w1 = vr[i][1] ^ 0x80808080u;
                u32x4 h;
                h[0] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, w0, 0x04010400u));
                h[1] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, w0, 0x04030402u));
                h[2] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, w1, 0x04010400u));
                h[3] = i8pair_to_f16x2(__builtin_amdgcn_perm(kF16Hi, w1, 0x04030402u));
                *reinterpret_cast<u32x4 *>(vw + (i * RPI + r) * kVtPitch + 16 * c) = h;
            }
            if (more2) issue_v(vr, ts + 2 * TT);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // A: lane (h = n, g = grp) takes P[rows 4g .. 4g+3][head h], a transposed read
            const f16x4 pa = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) shortx4 *)(pw + (4 * grp + (n >> 2)) * 32 + 8 * (n & 3))));
            const char *vt0 = vw + (4 * grp + (n >> 2)) * kVtPitch + 8 * (n & 3);
#pragma unroll
            for (int blk = 0; blk < D / 16; blk++) {
                const f16x4 bv = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) shortx4 *)(vt0 + 32 * blk)));
                oacc[blk] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, bv, oacc[blk], 0, 0, 0);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            ts += TT;
            return more;
        };
        issue_k(kA, ts);
        issue_v(vA, ts);
        if (ts + TT < hi) {
            issue_k(kB, ts + TT);
            issue_v(vB, ts + TT);
        }
        while (tile(kA, vA) && tile(kB, vB)) {
        }

        // l summed over the tile rows (the 16 lanes of a head group); m is uniform there
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float v = l4[i] + dpp<0xB1>(l4[i]);
            v += dpp<0x4E>(v);
            v += dpp<0x141>(v);
            l4[i] = v + dpp<0x140>(v);
        }
        // lane (n, grp < 2) holds O[4 grp + i][16 blk + n]
        if (grp < 2) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int hh = 4 * grp + i;
                if (hg * G + hh >= P.g) break;
                const int64_t row = slot * G + hh;
#pragma unroll
                for (int blk = 0; blk < D / 16; blk++) P.part_acc[row * D + 16 * blk + n] = oacc[blk][i];
                if (n == 0) *reinterpret_cast<float2 *>(P.part_ml + row * 2) = make_float2(m4[i], l4[i]);
            }
        }
        f += nseg;
    }   // segments
}

using SplitFn = void (*)(const SplitParams);

template <int KV, int D, int G, bool PAGED>
SplitFn pick_extra(int extra) {
    if constexpr (KV == KV_I8 && D == 128 && G == 8 && !PAGED) {
        if (extra == EX_NONE) return split_kernel_i8m<KV_I8>;
    }
    return extra == EX_PSE ? split_kernel<KV, D, G, PAGED, EX_PSE>
         : extra == EX_MASK ? split_kernel<KV, D, G, PAGED, EX_MASK>
                            : split_kernel<KV, D, G, PAGED, EX_NONE>;
}

template <int KV, int D, int G>
const void *ptr_pm(bool paged, int extra) {
    return reinterpret_cast<const void *>(paged ? pick_extra<KV, D, G, true>(extra)
                                                : pick_extra<KV, D, G, false>(extra));
}

template <int KV, int D, int G, bool PAGED, int EXTRA>
hipError_t launch_one(const SplitParams &p, hipStream_t s) {
    const int blocks = (p.n_pieces + kWavesPerBlock - 1) / kWavesPerBlock;
    if constexpr (KV == KV_I8 && D == 128 && G == 8 && !PAGED && EXTRA == EX_NONE) {
        if (p.Dr == 128) {      // the matrix-core int8 kernel covers full 128-wide rows only
            hipLaunchKernelGGL(split_kernel_i8m<KV_I8>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, p);
            return hipGetLastError();
        }
    }
    {
        // row mode: every wave's partial state of the row, merged in LDS
        const size_t lds = p.row_mode ? (size_t)kWavesPerBlock * G * D * sizeof(float) : 0;
        hipLaunchKernelGGL((split_kernel<KV, D, G, PAGED, EXTRA>), dim3(blocks), dim3(64 * kWavesPerBlock), lds, s, p);
    }
    return hipGetLastError();
}

template <int KV, int D, int G, bool PAGED>
hipError_t launch_ex(const SplitParams &p, int extra, hipStream_t s) {
    switch (extra) {
    case EX_NONE: return launch_one<KV, D, G, PAGED, EX_NONE>(p, s);
    case EX_MASK: return launch_one<KV, D, G, PAGED, EX_MASK>(p, s);
    case EX_PSE: return launch_one<KV, D, G, PAGED, EX_PSE>(p, s);
    }
    return hipErrorInvalidValue;
}

template <int KV, int D, int G>
hipError_t launch_pm(const SplitParams &p, bool paged, int extra, hipStream_t s) {
    return paged ? launch_ex<KV, D, G, true>(p, extra, s) : launch_ex<KV, D, G, false>(p, extra, s);
}

template <int KV, int D>
hipError_t launch_g(const SplitParams &p, int G, bool paged, int extra, hipStream_t s) {
    switch (G) {
    case 1: return launch_pm<KV, D, 1>(p, paged, extra, s);
    case 2: return launch_pm<KV, D, 2>(p, paged, extra, s);
    case 4: return launch_pm<KV, D, 4>(p, paged, extra, s);
    case 8: return launch_pm<KV, D, 8>(p, paged, extra, s);
    }
    return hipErrorInvalidValue;
}

template <int KV, int D>
const void *ptr_g(int G, bool paged, int extra) {
    switch (G) {
    case 1: return ptr_pm<KV, D, 1>(paged, extra);
    case 2: return ptr_pm<KV, D, 2>(paged, extra);
    case 4: return ptr_pm<KV, D, 4>(paged, extra);
    case 8: return ptr_pm<KV, D, 8>(paged, extra);
    }
    return nullptr;
}

}  // namespace split_detail

template <int KV>
hipError_t launch_split_kv(const SplitParams &p, int D, int G, bool paged, int extra, hipStream_t s) {
    using namespace split_detail;
    switch (D) {
    case 64: return launch_g<KV, 64>(p, G, paged, extra, s);
    case 128: return launch_g<KV, 128>(p, G, paged, extra, s);
    case 256: return launch_g<KV, 256>(p, G, paged, extra, s);
    case 512: return launch_g<KV, 512>(p, G, paged, extra, s);
    }
    return hipErrorInvalidValue;
}

template <int KV>
const void *split_kernel_ptr(int D, int G, bool paged, int extra) {
    using namespace split_detail;
    switch (D) {
    case 64: return ptr_g<KV, 64>(G, paged, extra);
    case 128: return ptr_g<KV, 128>(G, paged, extra);
    case 256: return ptr_g<KV, 256>(G, paged, extra);
    case 512: return ptr_g<KV, 512>(G, paged, extra);
    }
    return nullptr;
}

}  // namespace ifa
