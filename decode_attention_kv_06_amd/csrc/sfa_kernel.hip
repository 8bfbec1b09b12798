// SparseFlashAttention decode, MLA-absorb mode, on gfx950.
//
// For one batch b, every query head h and the cache rows named by the batch's
// sparse indices (SparseFlashAttention README, "Formula"):
//     out[b,h] = softmax(scale * (q . K~^T + q_rope . K~rope^T)) . V~
// with K~, K~rope, V~ the rows block_table[b][t / bs], t % bs of key,
// key_rope and value for each valid index t (0 <= t < actual_seq_lengths_kv[b]).
//
// Mapping to the hardware:
//  * one workgroup (4 waves) per (batch, block of 64 heads, chunk of
//    indices); each wave owns 16 heads.  The head blocks of one chunk get
//    workgroup ids that differ by a multiple of 8, which places them on the
//    same XCD, so the second read of a gathered row is an L2 hit.
//  * at the start the chunk's valid indices are compacted (in order) into an
//    LDS table of physical row numbers.
//  * tiles of 32 gathered rows (1152 B of key + rope, 1024 B of value each)
//    are copied straight from HBM into double-buffered LDS with
//    global_load_lds_dwordx4, the next tile in flight while the current one
//    computes; the copies use no VGPRs.
//  * scores S^T[t][h] = K~[t][:] . q[h][:] come from v_mfma_f32_16x16x32
//    (A = K~ rows from LDS, B = the wave's 16 query heads held in registers,
//    18 k-steps over 576).  Their output layout (lane l: head l%16, rows
//    4(l/16)+i of each 16-row block) is, with k-slot 8g+i <-> row 4g+i and
//    8g+4+i <-> row 16+4g+i, exactly the A layout of the P.V product, so P
//    needs no data movement.  The V~ operand is read transposed from LDS with
//    ds_read_b64_tr_b16.  Accumulation is fp32; P is rounded to the input
//    dtype for the MFMA.
//  * softmax is online in the log2 domain with a lazily raised maximum; the
//    chunk's partial state is written to the workspace (or, with a single
//    chunk per batch, the normalised output directly).
#include "sfa.h"

namespace ifa {
namespace sfa_detail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 512, kDR = 64, kDK = kD + kDR;   // value/key width, rope width, score width
constexpr int kT = 32;                  // gathered rows per tile
constexpr int kKP = 1168;               // LDS pitch of a K~ row: 1024 B key + 128 B rope + 16 B pad
constexpr int kVP = 1056;               // LDS pitch of a V~ row: 1024 B + 32 B pad
constexpr int kKReg = kT * kKP;         // 37376 B
constexpr int kVReg = kT * kVP;         // 33792 B
constexpr int kBuf = kKReg + kVReg;     // one tile buffer
constexpr int kKIns = (kKReg + 1023) / 1024;   // 1 KiB DMA instructions for K~ (last one partial)
constexpr int kVIns = kVReg / 1024;            // for V~
constexpr int kIns = kKIns + kVIns;
constexpr int kChunkMax = 1024;         // sparse entries per workgroup
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxInit = -1.0e30f;
constexpr float kLazy = 8.0f;           // raise the running max only past this many log2 units

static_assert(kKReg % 16 == 0 && kVReg % 1024 == 0, "DMA granularity");

__device__ __forceinline__ uint32_t div_bs(uint32_t s, uint32_t magic, int shift) {
    uint32_t t1 = __umulhi(magic, s);
    return (t1 + ((s - t1) >> 1)) >> (shift - 1);
}

template <bool BF>
struct Mfma;
template <>
struct Mfma<true> {
    typedef bf16x8 vec8;
    __device__ static floatx4 run(vec8 a, vec8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static vec8 tr2(const char *p0, const char *p1) {
        const bf16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4 *)p0);
        const bf16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4 *)p1);
        return vec8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    }
    __device__ static vec8 pack(const float (&p)[8]) {
        vec8 r;
#pragma unroll
        for (int i = 0; i < 8; i++) r[i] = (__bf16)p[i];
        return r;
    }
    __device__ static void store(void *out, int64_t i, float v) { reinterpret_cast<__bf16 *>(out)[i] = (__bf16)v; }
};
template <>
struct Mfma<false> {
    typedef f16x8 vec8;
    __device__ static floatx4 run(vec8 a, vec8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static vec8 tr2(const char *p0, const char *p1) {
        const f16x4 x = __builtin_bit_cast(
            f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4 *)p0));
        const f16x4 y = __builtin_bit_cast(
            f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4 *)p1));
        return vec8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    }
    __device__ static vec8 pack(const float (&p)[8]) {
        vec8 r;
#pragma unroll
        for (int i = 0; i < 8; i++) r[i] = (_Float16)p[i];
        return r;
    }
    __device__ static void store(void *out, int64_t i, float v) { reinterpret_cast<_Float16 *>(out)[i] = (_Float16)v; }
};

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <bool BF>
__global__ __launch_bounds__(256, 1) void sfa_kernel(const SfaParams P) {
    using M = Mfma<BF>;
    using vec8 = typename M::vec8;
    // two tile buffers as distinct objects, so the compiler can tell a read of
    // one from the copies in flight into the other
    __shared__ __attribute__((aligned(16))) char s_buf0[kBuf];
    __shared__ __attribute__((aligned(16))) char s_buf1[kBuf];
    __shared__ int32_t s_rows[kChunkMax];
    __shared__ int32_t s_cnt[kWavesPerBlock];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;

    // workgroup -> (batch, chunk, head block); head blocks of one chunk share an XCD
    const int id = blockIdx.x;
    const int x8 = id & 7, k8 = id >> 3;
    const int hb = k8 % P.n_hb;
    const int grp = (k8 / P.n_hb) * 8 + x8;
    if (grp >= P.B * P.n_sc) return;               // whole workgroup leaves together
    const int b = grp / P.n_sc, sc = grp - b * P.n_sc;

    // ---------------------------------------------------- compact the chunk's valid rows
    const int64_t e_begin = (int64_t)sc * P.chunk;
    const int n_entries = (int)min((int64_t)P.chunk, P.sparse_size - e_begin);
    const int Lkv = P.lkv[b];
    const bool q_present = P.lq == nullptr || P.lq[b] > 0;
    const int32_t *ind = P.idx + (int64_t)b * P.sparse_size + e_begin;
    const int32_t *btab = P.bt + (int64_t)b * P.max_blocks;
    int nv = 0;
    for (int base = 0; base < n_entries; base += 256) {
        const int e = base + tid;
        bool valid = false;
        int32_t row = 0;
        if (e < n_entries && q_present) {
            const int t = ind[e];
            if (t >= 0 && t < Lkv) {
                const uint32_t qb = div_bs((uint32_t)t, P.bs_magic, P.bs_shift);
                // the kv length is device data: an index past the block table is left out
                const int blk = qb < (uint32_t)P.max_blocks ? btab[qb] : -1;
                if (blk >= 0 && blk < P.num_blocks) {
                    valid = true;
                    row = blk * P.bs + (t - (int)qb * P.bs);
                }
            }
        }
        const uint64_t bal = __ballot(valid);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (lane == 0) s_cnt[wave] = __popcll(bal);
        __syncthreads();
        int off = nv;
        for (int w = 0; w < wave; w++) off += s_cnt[w];
        if (valid) s_rows[off + before] = row;
        for (int w = 0; w < kWavesPerBlock; w++) nv += s_cnt[w];
        __syncthreads();
    }
    nv = __builtin_amdgcn_readfirstlane(nv);

    // ---------------------------------------------------- this wave's 16 heads
    const int h = hb * 64 + wave * 16 + l16;          // head of lanes l16 (score layout)
    const bool h_ok = h < P.QN;
    vec8 qreg[kDK / 32];
#pragma unroll
    for (int ks = 0; ks < kDK / 32; ks++) {
        u32x4 x = {0, 0, 0, 0};
        if (h_ok) {
            const char *src = ks < kD / 32
                ? reinterpret_cast<const char *>(P.q) + (((int64_t)b * P.QN + h) * kD + 32 * ks + 8 * g) * 2
                : reinterpret_cast<const char *>(P.q_rope) + (((int64_t)b * P.QN + h) * kDR + 32 * (ks - kD / 32) + 8 * g) * 2;
            x = *reinterpret_cast<const u32x4 *>(src);
        }
        qreg[ks] = __builtin_bit_cast(vec8, x);
    }

    // ---------------------------------------------------- gather tiles into LDS
    const char *keyb = reinterpret_cast<const char *>(P.key);
    const char *ropeb = reinterpret_cast<const char *>(P.key_rope);
    const char *valb = reinterpret_cast<const char *>(P.value);
    const int n_tiles = (nv + kT - 1) / kT;
    // Every wave issues the DMA instructions ins = wave, wave + 4, ...; each
    // instruction fills 1 KiB of the buffer, lane l bytes [16 l, 16 l + 16).
    constexpr int kInsW0 = (kIns + kWavesPerBlock - 1) / kWavesPerBlock;   // waves 0..(kIns % 4 - 1)
    auto issue_tile = [&](int tile, char *bufp) {
        char *kreg = bufp;
        char *vreg = kreg + kKReg;
        const int rbase = tile * kT;
        for (int ins = wave; ins < kIns; ins += kWavesPerBlock) {
            const char *src;
            char *dst;
            bool on = true;
            if (ins < kKIns) {
                const int o = ins * 1024 + lane * 16;
                on = o < kKReg;
                const int rr = min(o / kKP, kT - 1), col = o - rr * kKP;
                const int r = rbase + rr;
                const int64_t row = s_rows[r < nv ? r : 0];
                src = col < 1024 ? keyb + row * 1024 + col
                    : col < 1152 ? ropeb + row * 128 + (col - 1024) : keyb + row * 1024;
                dst = kreg + ins * 1024;
            } else {
                const int o = (ins - kKIns) * 1024 + lane * 16;
                const int rr = o / kVP, col = o - rr * kVP;
                const int r = rbase + rr;
                const int64_t row = s_rows[r < nv ? r : 0];
                src = col < 1024 ? valb + row * 1024 + col : valb + row * 1024;
                dst = vreg + (ins - kKIns) * 1024;
            }
            if (on)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src), dst, 16, 0, 0);
        }
    };

    floatx4 acc[kD / 16];
#pragma unroll
    for (int nb = 0; nb < kD / 16; nb++) acc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = kMaxInit, l_run = 0.f;    // per head l16 (lanes of one head agree on m_run)
    const float smul = P.score_mul;

    // one tile: wait for its copies, issue the next tile's copies into the
    // other buffer, compute
    auto step = [&](int tile, const char *cur, char *nxt) {
        if (tile + 1 < n_tiles) {
            issue_tile(tile + 1, nxt);
            // this wave's copies of the current tile are complete once at most
            // the next tile's copies are outstanding
            if (wave < kIns % kWavesPerBlock || kIns % kWavesPerBlock == 0) wait_vmcnt<kInsW0>();
            else wait_vmcnt<kInsW0 - 1>();
        } else {
            wait_vmcnt<0>();
        }
        // Every wave's copies of this tile have landed.  A bare s_barrier (no
        // fence) keeps the next tile's copies in flight across it.
        __builtin_amdgcn_s_barrier();
        const char *kreg = cur;
        const char *vreg = kreg + kKReg;
        // S^T for the two 16-row blocks of the tile
        floatx4 sc2[2];
#pragma unroll
        for (int tb = 0; tb < 2; tb++) {
            floatx4 cacc = {0.f, 0.f, 0.f, 0.f};
            const char *arow = kreg + (tb * 16 + l16) * kKP + 16 * g;
#pragma unroll
            for (int ks = 0; ks < kDK / 32; ks++) {
                const vec8 a = *reinterpret_cast<const vec8 *>(arow + 64 * ks);
                cacc = M::run(a, qreg[ks], cacc);
            }
            sc2[tb] = cacc;
        }
        // scale, exclude rows past the valid count
        float p[8];
        float mt = kNegInf;
#pragma unroll
        for (int tb = 0; tb < 2; tb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = tile * kT + tb * 16 + 4 * g + i;
                const float s = r < nv ? sc2[tb][i] * smul : kNegInf;
                p[tb * 4 + i] = s;
                mt = fmaxf(mt, s);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const bool raise = mt > m_run + kLazy;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float mn = raise ? mt : m_run;
            const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
            m_run = mn;
            l_run *= alpha;
            // the accumulator rows of this lane are heads 4g + i; their alpha
            // lives in lanes 4g + i (score layout: head = lane % 16)
            float ai[4];
#pragma unroll
            for (int i = 0; i < 4; i++) ai[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
            for (int nb = 0; nb < kD / 16; nb++)
#pragma unroll
                for (int i = 0; i < 4; i++) acc[nb][i] *= ai[i];
        }
#pragma unroll
        for (int i = 0; i < 8; i++) {
            p[i] = __builtin_amdgcn_exp2f(p[i] - m_run);
            l_run += p[i];
        }
        const vec8 pa = M::pack(p);

        // O[h][d] += P[h][t] V~[t][d]: B operand read transposed from LDS
        // (lane j of a 16-lane group points at row 4g + j/4, columns 4(j%4)..+3
        // of the 16-column block; the second read covers rows 16 + 4g + j/4)
        const char *v0 = vreg + (4 * g + (l16 >> 2)) * kVP + 8 * (l16 & 3);
        const char *v1 = v0 + 16 * kVP;
#pragma unroll
        for (int nb = 0; nb < kD / 16; nb++) {
            const vec8 bv = M::tr2(v0 + 32 * nb, v1 + 32 * nb);
            acc[nb] = M::run(pa, bv, acc[nb]);
        }
        // all LDS reads of this buffer are done (their results fed the MFMAs
        // above) before any wave starts the copy two tiles ahead into it
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt untouched
        __builtin_amdgcn_s_barrier();
    };
    if (n_tiles > 0) issue_tile(0, s_buf0);
    for (int tile = 0; tile < n_tiles; tile += 2) {
        step(tile, s_buf0, s_buf1);
        if (tile + 1 < n_tiles) step(tile + 1, s_buf1, s_buf0);
    }

    // ---------------------------------------------------- epilogue
    // l of head l16 summed over the four lane groups (m_run already agrees)
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    float li[4], mi[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        li[i] = __shfl(l_run, 4 * g + i);
        mi[i] = __shfl(m_run, 4 * g + i);
    }
    const int hrow0 = hb * 64 + wave * 16 + 4 * g;     // heads of this lane's accumulator rows
    if (P.direct) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int hh = hrow0 + i;
            if (hh >= P.QN) continue;
            const float inv = li[i] > 0.f ? 1.f / li[i] : 0.f;
#pragma unroll
            for (int nb = 0; nb < kD / 16; nb++)
                M::store(P.out, ((int64_t)b * P.QN + hh) * kD + 16 * nb + l16, acc[nb][i] * inv);
        }
    } else {
        const int64_t prow = ((int64_t)b * P.n_sc + sc) * P.QN;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int hh = hrow0 + i;
            if (hh >= P.QN) continue;
            float *dst = P.part_acc + (prow + hh) * kD + l16;
#pragma unroll
            for (int nb = 0; nb < kD / 16; nb++) dst[16 * nb] = acc[nb][i];
            if (l16 == 0) *reinterpret_cast<float2 *>(P.part_ml + (prow + hh) * 2) = make_float2(mi[i], li[i]);
        }
    }
}

// Merges the chunk states of one (b, h) row in chunk order and rounds.
template <bool BF>
__global__ __launch_bounds__(256) void sfa_combine_kernel(const SfaParams P) {
    using M = Mfma<BF>;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= P.B * P.QN) return;
    const int b = row / P.QN, hh = row - b * P.QN;
    const float2 *ml = reinterpret_cast<const float2 *>(P.part_ml);
    auto prow = [&](int s) -> int64_t { return ((int64_t)b * P.n_sc + s) * P.QN + hh; };
    float Mx = kNegInf;
    for (int s = 0; s < P.n_sc; s++) Mx = fmaxf(Mx, ml[prow(s)].x);
    float L = 0.f, o[kD / 64];
#pragma unroll
    for (int e = 0; e < kD / 64; e++) o[e] = 0.f;
    for (int s = 0; s < P.n_sc; s++) {
        const float2 v = ml[prow(s)];
        const float w = __builtin_amdgcn_exp2f(v.x - Mx);
        L += w * v.y;
        const float *a = P.part_acc + prow(s) * kD;
#pragma unroll
        for (int e = 0; e < kD / 64; e++) o[e] += w * a[lane + 64 * e];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int e = 0; e < kD / 64; e++) M::store(P.out, ((int64_t)b * P.QN + hh) * kD + lane + 64 * e, o[e] * inv);
}

}  // namespace sfa_detail

hipError_t sfa_launch(const SfaParams &p, bool bf16, int grid, hipStream_t s, hipEvent_t ev_begin,
                      hipEvent_t ev_end) {
    using namespace sfa_detail;
    if (ev_begin && hipEventRecord(ev_begin, s) != hipSuccess) return hipErrorUnknown;
    if (bf16)
        hipLaunchKernelGGL(sfa_kernel<true>, dim3(grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(sfa_kernel<false>, dim3(grid), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_end && hipEventRecord(ev_end, s) != hipSuccess) return hipErrorUnknown;
    if (!p.direct) {
        const int rows = p.B * p.QN;
        const int blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
        if (bf16)
            hipLaunchKernelGGL(sfa_combine_kernel<true>, dim3(blocks), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL(sfa_combine_kernel<false>, dim3(blocks), dim3(256), 0, s, p);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace ifa
