// SparseFlashAttention decode, MLA-absorb mode, on gfx950.
//
// For one batch b, every query head h and the cache rows named by the batch's
// sparse indices (SparseFlashAttention README, "Formula"):
//     out[b,h] = softmax(scale * (q . K~^T + q_rope . K~rope^T)) . V~
// with K~, K~rope, V~ the rows block_table[b][t / bs], t % bs of key,
// key_rope and value for each valid index t (0 <= t < actual_seq_lengths_kv[b]).
//
// Mapping to the hardware (sfa_kernel; sfa_wide_kernel below takes every
// head of a chunk in one workgroup when that halves an oversized grid):
//  * one workgroup (4 waves) per (batch, block of 64 heads, chunk of
//    indices); each wave owns 16 heads.  Each XCD takes a contiguous range
//    of (batch, chunk) groups with all their head blocks, so the second read
//    of a gathered row, and the query and block-table rows that the chunks
//    of a batch share, are L2 hits.
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
// LDS row pitch of K~ and V~ rows: 1024 B + 32 B.  With 64 four-byte banks this
// is conflict-free both for the 16-byte A-operand reads (row = lane % 16) and
// for the transposed 8-byte V~ reads (row = 4 (lane / 16) + (lane % 16) / 4).
constexpr int kRP = 1056;
constexpr int kRopeOff = kT * kRP;      // rope rows of a key slot: 32 x 128 B, columns swizzled
constexpr int kSlot = kRopeOff + kT * 128;   // one ring slot (the key half of a tile is the larger)
constexpr int kChunkMax = kSfaChunkMax;   // sparse entries per workgroup (a multiple of 256)
// Output staging at the end: each wave's 64 heads x 128 columns (256 B rows at
// a 272-byte pitch, so the 2-byte writes of four heads a lane group apart fall
// in distinct banks); two waves share one ring slot.
constexpr int kStgPitch = 272;
constexpr int kKIns = 9;                // DMA instructions per wave for a key half-tile (8 rows + rope)
constexpr int kVIns = 8;                // ... for a value half-tile
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxInit = -1.0e30f;
constexpr float kLazy = 8.0f;           // raise the running max only past this many log2 units
constexpr float kLn2 = 0.69314718055994531f;   // log2-domain maxima back to the natural-log domain

static_assert(kT == 8 * kWavesPerBlock, "each wave copies 8 rows of a tile");
static_assert(2 * 64 * kStgPitch <= kRopeOff + kT * 128, "two waves' output blocks fit one ring slot");
static_assert(4 * kSlot + kWavesPerBlock * 64 * 16 + 4 * kChunkMax + 4 * 64 * 2 + 4 * 4 * 3 <= 160 * 1024, "LDS budget");
static_assert(kChunkMax % 256 == 0, "two entries per thread");

__device__ __forceinline__ uint32_t div_bs(uint32_t s, uint32_t magic, int shift) {
    uint32_t t1 = __umulhi(magic, s);
    return (t1 + ((s - t1) >> 1)) >> (shift - 1);
}

// 16-byte chunk c of rope row r sits at chunk c ^ rope_swz(r) of that row, so
// that the A-operand reads of 16 rows spread over all banks.
__device__ __forceinline__ int rope_swz(int r) { return 2 * ((r >> 1) & 3); }

// HBM -> LDS copy of 16 bytes per lane: lane l writes LDS bytes
// [dst + 16 l, dst + 16 l + 16); dst is wave-uniform.  Issued as assembly, so
// the compiler neither tracks nor waits for these copies: every wait on them
// is an explicit vmcnt below.  (The compiler's own tracking of LDS-DMA stores
// loses the slot a read belongs to across the ring loop and then drains all
// copies in flight.)  M0 takes the LDS address; one wait state separates its
// write from the copy that reads it.
__device__ __forceinline__ void dma16(const void *src, char *dst) {
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)dst;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
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
    __device__ static float load(const void *in, int64_t i) { return (float)reinterpret_cast<const __bf16 *>(in)[i]; }
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
    __device__ static float load(const void *in, int64_t i) { return (float)reinterpret_cast<const _Float16 *>(in)[i]; }
};

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// max(x, x of lane ^ 16) and max(x, x of lane ^ 32) with the gfx950 row-swap
// permutes: one swap returns, in every lane, the values of both rows of the
// pair, so their max (or sum) is the pairwise reduction.  No LDS round trip.
// The two halves are copied to scalars before the bit casts: a bit cast of a
// vector element read in place has been compiled as a read of element 0.
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x), false, false);
    const uint32_t a = r[0], b = r[1];
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x), false, false);
    const uint32_t a = r[0], b = r[1];
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// Workgroup barrier without a memory fence (the copies in flight must stay in
// flight across it).  The empty assembly statements keep the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// lgkmcnt(0) with the other counters left alone.  The compiler's own waits
// before an LDS read's first use are lgkmcnt(0) whenever LDS-DMA copies are in
// flight; waiting explicitly before issuing the next operand group keeps that
// group's reads in flight during the current MFMAs.
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// The chunk's valid cache rows, compacted in order into the LDS table
// `s_rows`; returns their count (wave-uniform).  Every thread of the
// workgroup calls it (it synchronises the workgroup twice).
__device__ __forceinline__ int compact_chunk(const SfaParams &P, int qr, int sc, int32_t *s_rows,
                                             int32_t (*s_cnt)[kWavesPerBlock]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // ---------------------------------------------------- the row's batch and attended range
    // Query row -> batch b, place s among the batch's Lq query rows; the
    // cache rows of batch b start at kv0 and hold Lkv positions; positions
    // t < limit are attended (limit = Lkv, or the causal bound Lkv - Lq + s + 1
    // under sparse_mode 3; 0 for a padding query row).  Lengths are device
    // data: every bound is clamped so no read leaves its tensor.
    int b, s, Lq;
    if (P.layout_q == 0) {
        b = qr / P.QS;
        s = qr - b * P.QS;
        Lq = P.lq ? P.lq[b] : P.QS;
    } else {
        int cnt = 0;                                   // prefix sums <= qr: the batch that owns row qr
        for (int e0 = 0; e0 < P.B; e0 += 64) {
            const int e = e0 + lane;
            cnt += __popcll(__ballot(e < P.B && P.lq[e] <= qr));
        }
        b = __builtin_amdgcn_readfirstlane(cnt);
        const int start = b > 0 ? P.lq[b - 1] : 0;
        s = qr - start;
        Lq = b < P.B ? P.lq[b] - start : 0;
        if (b >= P.B) b = P.B - 1;
    }
    int64_t kv0 = 0, Lkv;
    if (P.layout_kv == 2) {
        kv0 = b > 0 ? P.lkv[b - 1] : 0;
        kv0 = min(max(kv0, (int64_t)0), P.kv_rows);
        Lkv = min((int64_t)P.lkv[b] - kv0, P.kv_rows - kv0);
    } else if (P.layout_kv == 1) {
        kv0 = (int64_t)b * P.kv_seq;
        Lkv = P.lkv ? min((int64_t)P.lkv[b], P.kv_seq) : P.kv_seq;
    } else {
        Lkv = P.lkv[b];
    }
    int64_t limit = Lkv;
    if (P.sparse_mode == 3) limit = min(limit, Lkv - Lq + s + 1);
    if (s >= Lq) limit = 0;
    limit = max(limit, (int64_t)0);

    // ---------------------------------------------------- compact the chunk's valid rows
    // Row slot j = 256 k + tid (k = 0, 1) is position u = j % sparse_block_size
    // of the block named by entry j / sparse_block_size; all index loads, then
    // all block-table loads, are issued together.  Valid rows keep their order.
    const int64_t e_begin = (int64_t)sc * P.chunk;
    const int n_entries = (int)min((int64_t)P.chunk, P.sparse_size - e_begin);
    const int n_slots = n_entries << P.sbs_shift;
    const int32_t *ind = P.idx + (int64_t)qr * P.sparse_size + e_begin;
    const int32_t *btab = P.bt + (int64_t)b * P.max_blocks;
    constexpr int kPer = kChunkMax / 256;
    int tv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int j = 256 * k + tid;
        tv[k] = j < n_slots ? ind[j >> P.sbs_shift] : -1;
    }
    int64_t pos[kPer];
    bool valid[kPer];
    int blk[kPer];
    uint32_t qbv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int j = 256 * k + tid;
        pos[k] = ((int64_t)tv[k] << P.sbs_shift) + (j & ((1 << P.sbs_shift) - 1));
        valid[k] = tv[k] >= 0 && pos[k] < limit;
        if (P.layout_kv == 0) {
            qbv[k] = div_bs((uint32_t)(valid[k] ? pos[k] : 0), P.bs_magic, P.bs_shift);
            // the kv length is device data: a position past the block table is left out
            const bool look = valid[k] && qbv[k] < (uint32_t)P.max_blocks;
            blk[k] = look ? btab[qbv[k]] : -1;
        }
    }
    int before[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        if (P.layout_kv == 0) valid[k] = blk[k] >= 0 && blk[k] < P.num_blocks;
        const uint64_t bal = __ballot(valid[k]);
        before[k] = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (lane == 0) s_cnt[k][wave] = __popcll(bal);
    }
    __syncthreads();
    int nv = 0;
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        int off = nv;
        for (int w = 0; w < wave; w++) off += s_cnt[k][w];
        if (valid[k])
            s_rows[off + before[k]] = P.layout_kv == 0 ? blk[k] * P.bs + ((int)pos[k] - (int)qbv[k] * P.bs)
                                                      : (int)(kv0 + pos[k]);
        for (int w = 0; w < kWavesPerBlock; w++) nv += s_cnt[k][w];
    }
    __syncthreads();
    nv = __builtin_amdgcn_readfirstlane(nv);
    return nv;
}

// Gather copies of one tile half.  Wave w copies tile rows 8w .. 8w+7: one
// 1 KiB instruction per key row and per value row (the row base is
// wave-uniform) and one instruction for the eight rope rows (lane l: row
// 8w + l/8, 16-byte chunk l%8).  `rows` holds, in lane l, the physical row of
// tile row 8w + l/8; tiles past the last repeat its last row.
__device__ __forceinline__ int tile_rows(const int32_t *s_rows, int tile, int nv, int lane, int wave) {
    return s_rows[min(tile * kT + 8 * wave + (lane >> 3), nv - 1)];
}
__device__ __forceinline__ void issue_key_half(const SfaParams &P, char *slot, int rows, int lane, int wave) {
    const char *keyb = reinterpret_cast<const char *>(P.key);
    const char *ropeb = reinterpret_cast<const char *>(P.key_rope);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int64_t row = __builtin_amdgcn_readlane(rows, 8 * j);
        dma16(keyb + row * 1024 + lane * 16, slot + (8 * wave + j) * kRP);
    }
    const int r = 8 * wave + (lane >> 3);
    dma16(ropeb + (int64_t)rows * 128 + 16 * ((lane & 7) ^ rope_swz(r)), slot + kRopeOff + wave * 1024);
}
__device__ __forceinline__ void issue_value_half(const SfaParams &P, char *slot, int rows, int lane, int wave) {
    const char *valb = reinterpret_cast<const char *>(P.value);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int64_t row = __builtin_amdgcn_readlane(rows, 8 * j);
        dma16(valb + row * 1024 + lane * 16, slot + (8 * wave + j) * kRP);
    }
}

// Half-tile h (key rows of tile h/2 for even h, value rows for odd h) lives in
// ring slot h % 4.  Before computing half-tile h a wave waits until only its
// copies of halves h+1 and h+2 may still be in flight.  Halves past the last
// tile are still copied (the last valid row again, never read), so that count
// is the same at every step.

template <bool BF, bool ALIAS>
__global__ __launch_bounds__(256, 1) void sfa_kernel(const SfaParams P) {
    using M = Mfma<BF>;
    using vec8 = typename M::vec8;
    // the four ring slots as distinct objects, so the compiler can tell a read
    // of one from the copies in flight into another
    __shared__ __attribute__((aligned(16))) char s_slot0[kSlot];
    __shared__ __attribute__((aligned(16))) char s_slot1[kSlot];
    __shared__ __attribute__((aligned(16))) char s_slot2[kSlot];
    __shared__ __attribute__((aligned(16))) char s_slot3[kSlot];
    __shared__ __attribute__((aligned(16))) char s_p[kWavesPerBlock * 64 * 16];   // P of each head group
    __shared__ int32_t s_rows[kChunkMax];
    __shared__ float s_alpha[64];           // rescale factor of each head for the current tile
    __shared__ float s_linv[64];            // 1 / l of each head (single-chunk output)
    __shared__ __attribute__((aligned(16))) int32_t s_flag[kWavesPerBlock];   // group raised its running max this tile
    __shared__ int32_t s_cnt[2][kWavesPerBlock];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;

    // workgroup -> (query row, chunk, head block).  Workgroup ids congruent
    // mod 8 run on one XCD; XCD x takes the contiguous range of (query row,
    // chunk) groups [x g8, (x + 1) g8) with all their head blocks, so the
    // chunks of a query row (one query and block-table row) and the head
    // blocks of a chunk (the same gathered rows) meet in one L2.
    const int id = blockIdx.x;
    const int x8 = id & 7, k8 = id >> 3;
    const int hb = k8 % P.n_hb;
    const int g8 = (P.R * P.n_sc + 7) >> 3;
    const int grp = x8 * g8 + k8 / P.n_hb;
    if (grp >= P.R * P.n_sc) return;               // whole workgroup leaves together
    const int qr = grp / P.n_sc, sc = grp - qr * P.n_sc;

    // Head groups of 16: wave w computes the scores of group w; every wave
    // accumulates P.V for all four groups over its own 128 output columns.  A
    // group past the head count keeps P = 0 and is never stored.
    const int n_act = min(kWavesPerBlock, (P.QN - hb * 64 + 15) / 16);   // >= 1
    const bool qk_wave = wave < n_act;
    if (!qk_wave) *reinterpret_cast<u32x4 *>(s_p + (wave * 64 + lane) * 16) = u32x4{0, 0, 0, 0};
    if (lane == 0) s_flag[wave] = 0;

    // ---------------------------------------------------- query rows (issued first)
    const int h = hb * 64 + wave * 16 + l16;          // head of lanes l16 (score layout)
    const bool h_ok = h < P.QN;
    vec8 qreg[kDK / 32];
#pragma unroll
    for (int ks = 0; ks < kDK / 32; ks++) {
        u32x4 x = {0, 0, 0, 0};
        if (h_ok) {
            const char *src = ks < kD / 32
                ? reinterpret_cast<const char *>(P.q) + (((int64_t)qr * P.QN + h) * kD + 32 * ks + 8 * g) * 2
                : reinterpret_cast<const char *>(P.q_rope) + (((int64_t)qr * P.QN + h) * kDR + 32 * (ks - kD / 32) + 8 * g) * 2;
            x = *reinterpret_cast<const u32x4 *>(src);
        }
        qreg[ks] = __builtin_bit_cast(vec8, x);
    }

    const int nv = compact_chunk(P, qr, sc, s_rows, s_cnt);

    // ---------------------------------------------------- gather copies
    const int n_tiles = (nv + kT - 1) / kT;
    auto rows_of = [&](int tile) { return tile_rows(s_rows, tile, nv, lane, wave); };
    auto issue_k = [&](char *slot, int rows) { issue_key_half(P, slot, rows, lane, wave); };
    auto issue_v = [&](char *slot, int rows) { issue_value_half(P, slot, rows, lane, wave); };

    // acc[hg][j]: heads 16 hg + 4g + i (i = 0..3) of the block, output column
    // 128 wave + 16 j + l16
    floatx4 acc[kWavesPerBlock][8];
#pragma unroll
    for (int hg = 0; hg < kWavesPerBlock; hg++)
#pragma unroll
        for (int j = 0; j < 8; j++) acc[hg][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = kMaxInit, l_run = 0.f;    // head l16 of group `wave` (lanes of one head agree on m_run)
    float m_true = kNegInf;                 // the largest score itself (m_run is raised lazily, so may lag it)
    const float smul = P.score_mul;

    // scores of tile `tile` for head group `wave` from its key slot, the
    // online-softmax update, and P (A-operand layout) and the rescale factors
    // published in LDS
    auto qk = [&](int tile, const char *ks_, auto &&pre) {
        // 36 products: step i takes row block i % 2 and k-step i / 2, so the
        // two accumulation chains interleave.
        constexpr int kSteps = 2 * (kDK / 32);
        auto a_ptr = [&](int i) -> const char * {
            const int tb = i & 1, ks = i >> 1;
            const int r = tb * 16 + l16;
            if (ks < kD / 32) return ks_ + r * kRP + 64 * ks + 16 * g;
            return ks_ + kRopeOff + r * 128 + 16 * ((4 * (ks - kD / 32) + g) ^ rope_swz(r));
        };
        floatx4 sc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        // groups of kGrp steps: the reads of group j + 1 are issued before the
        // MFMAs of group j (the scheduling fences keep that order)
        constexpr int kGrp = 6, kGroups = kSteps / kGrp;
        static_assert(kSteps % kGrp == 0, "group size");
        vec8 abuf[2][kGrp];
#pragma unroll
        for (int i = 0; i < kGrp; i++) abuf[0][i] = *reinterpret_cast<const vec8 *>(a_ptr(i));
        pre();      // the step's copies issue while the first operands are read
#pragma unroll
        for (int j = 0; j < kGroups; j++) {
            // operands of group j have arrived; only then issue group j + 1, so
            // that its reads stay in flight during the MFMAs of group j
            lds_wait();
            __builtin_amdgcn_sched_barrier(0);
            if (j + 1 < kGroups) {
#pragma unroll
                for (int i = 0; i < kGrp; i++)
                    abuf[(j + 1) & 1][i] = *reinterpret_cast<const vec8 *>(a_ptr((j + 1) * kGrp + i));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kGrp; i++) {
                const int st = j * kGrp + i;
                sc2[st & 1] = M::run(abuf[j & 1][i], qreg[st >> 1], sc2[st & 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
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
        mt = max_xor16(mt);
        mt = max_xor32(mt);
        m_true = fmaxf(m_true, mt);
        const bool raise = mt > m_run + kLazy;
        float alpha = 1.f;
        int flag = 0;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float mn = raise ? mt : m_run;
            alpha = __builtin_amdgcn_exp2f(m_run - mn);
            // nothing has been accumulated before the first tile
            flag = tile > 0;
            m_run = mn;
            l_run *= alpha;
        }
#pragma unroll
        for (int i = 0; i < 8; i++) {
            p[i] = __builtin_amdgcn_exp2f(p[i] - m_run);
            l_run += p[i];
        }
        *reinterpret_cast<vec8 *>(s_p + (wave * 64 + lane) * 16) = M::pack(p);
        if (g == 0) s_alpha[wave * 16 + l16] = alpha;
        if (lane == 0) s_flag[wave] = flag;
    };
    // O[h][d] += P[h][t] V~[t][d] over this wave's 128 columns and every active
    // head group.  The V~ operand is read transposed from LDS (lane j of a
    // 16-lane group points at row 4g + j/4, columns 4(j%4)..+3 of the 16-column
    // block; the second read covers rows 16 + 4g + j/4) and serves all groups.
    auto pv = [&](const char *vs_, auto &&pre) {
        const u32x4 fl = *reinterpret_cast<const u32x4 *>(s_flag);
        vec8 pa[kWavesPerBlock];
#pragma unroll
        for (int hg = 0; hg < kWavesPerBlock; hg++) pa[hg] = *reinterpret_cast<const vec8 *>(s_p + (hg * 64 + lane) * 16);
        const char *v0 = vs_ + (4 * g + (l16 >> 2)) * kRP + 8 * (l16 & 3) + 256 * wave;
        const char *v1 = v0 + 16 * kRP;
        constexpr int kPfV = 4, kGroups = 8 / kPfV;
        vec8 bbuf[2][kPfV];
#pragma unroll
        for (int i = 0; i < kPfV; i++) bbuf[0][i] = M::tr2(v0 + 32 * i, v1 + 32 * i);
        pre();      // the step's copies issue while the first operands are read
        // a raised running max rescales what the group accumulated so far
        if (fl[0] | fl[1] | fl[2] | fl[3]) {
#pragma unroll
            for (int hg = 0; hg < kWavesPerBlock; hg++) {
                if (!fl[hg]) continue;
                float ai[4];
#pragma unroll
                for (int i = 0; i < 4; i++) ai[i] = s_alpha[hg * 16 + 4 * g + i];
#pragma unroll
                for (int j = 0; j < 8; j++)
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[hg][j][i] *= ai[i];
            }
        }
#pragma unroll
        for (int jg = 0; jg < kGroups; jg++) {
            lds_wait();
            __builtin_amdgcn_sched_barrier(0);
            if (jg + 1 < kGroups) {
#pragma unroll
                for (int i = 0; i < kPfV; i++) {
                    const int j = (jg + 1) * kPfV + i;
                    bbuf[(jg + 1) & 1][i] = M::tr2(v0 + 32 * j, v1 + 32 * j);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kPfV; i++)
#pragma unroll
                for (int hg = 0; hg < kWavesPerBlock; hg++)
                    acc[hg][jg * kPfV + i] = M::run(pa[hg], bbuf[jg & 1][i], acc[hg][jg * kPfV + i]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // End of a half step: this wave's LDS reads of the slot have returned and
    // its LDS writes are done before any wave may overwrite or read them.
    auto end_half = [&]() { lds_wait(); };

    // ---------------------------------------------------- pipeline
    // The compiler's own vector-memory loads (query, indices, block table) are
    // consumed by now; the copies below are the only ones in flight from here.
    if constexpr (ALIAS) {
        // The value tensor is the key tensor: a tile's value rows are its key
        // rows, already in the key slot, so a tile is one copy (key and rope)
        // into slot t % 4, three tiles ahead.  Step t waits for tile t,
        // synchronises (every wave's copies of tile t have landed and every
        // wave is done with tile t - 1, whose slot tile t + 3 reuses), issues
        // tile t + 3, scores tile t, synchronises again (P and the rescale
        // factors are visible) and applies P.V from the same slot.
        if (n_tiles > 0) {
            issue_k(s_slot0, rows_of(0));
            issue_k(s_slot1, rows_of(1));
            issue_k(s_slot2, rows_of(2));
        }
        auto step = [&](int t, char *cur, char *nxt) {
            wait_vmcnt<2 * kKIns>();
            ring_barrier();
            {
                auto pre = [&]() { issue_k(nxt, rows_of(t + 3)); };
                if (qk_wave) qk(t, cur, pre);
                else pre();
            }
            end_half();
            ring_barrier();
            pv(cur, [&]() {});
            end_half();
        };
        for (int t = 0; t < n_tiles; t += 4) {
            step(t, s_slot0, s_slot3);
            if (t + 1 >= n_tiles) break;
            step(t + 1, s_slot1, s_slot0);
            if (t + 2 >= n_tiles) break;
            step(t + 2, s_slot2, s_slot1);
            if (t + 3 >= n_tiles) break;
            step(t + 3, s_slot3, s_slot2);
        }
    } else {
        // Half-tiles h = 0, 1, 2 are issued up front; step h waits for half h,
        // synchronises the workgroup (every wave's copies of half h have
        // landed, every wave is done with half h - 1, whose slot half h + 3
        // reuses, and P of the tile is visible), issues half h + 3 and
        // computes half h.  `rows_n` holds the rows of the next tile whose
        // halves are still to be issued.
        int rows_n = 0;
        if (n_tiles > 0) {
            rows_n = rows_of(0);
            issue_k(s_slot0, rows_n);
            issue_v(s_slot1, rows_n);
            rows_n = rows_of(1);
            issue_k(s_slot2, rows_n);
        }
        // two tiles (four half steps, one per slot) per iteration
        for (int t = 0; t < n_tiles; t += 2) {
            // h = 2t: scores of tile t (slot 0); issue V(t+1) into slot 3
            wait_vmcnt<kKIns + kVIns>();
            ring_barrier();
            {
                auto pre = [&]() { issue_v(s_slot3, rows_n); rows_n = rows_of(t + 2); };
                if (qk_wave) qk(t, s_slot0, pre);
                else pre();
            }
            end_half();
            // h = 2t+1: P.V of tile t (slot 1); issue K(t+2) into slot 0
            wait_vmcnt<kKIns + kVIns>();
            ring_barrier();
            pv(s_slot1, [&]() { issue_k(s_slot0, rows_n); });
            end_half();
            if (t + 1 >= n_tiles) break;
            // h = 2t+2: scores of tile t+1 (slot 2); issue V(t+2) into slot 1
            wait_vmcnt<kKIns + kVIns>();
            ring_barrier();
            {
                auto pre = [&]() { issue_v(s_slot1, rows_n); rows_n = rows_of(t + 3); };
                if (qk_wave) qk(t + 1, s_slot2, pre);
                else pre();
            }
            end_half();
            // h = 2t+3: P.V of tile t+1 (slot 3); issue K(t+3) into slot 2
            wait_vmcnt<kKIns + kVIns>();
            ring_barrier();
            pv(s_slot3, [&]() { issue_k(s_slot2, rows_n); });
            end_half();
        }
    }

    // the copies past the last tile land before the workgroup's LDS is released
    wait_vmcnt<0>();

    // ---------------------------------------------------- epilogue
    // Every chunk writes its output normalised by its own sum: directly when
    // the batch has one chunk, else in the input dtype to the workspace with
    // (m, l) beside it for the combine.
    const int64_t prow = ((int64_t)qr * P.n_sc + sc) * P.QN;  // partial rows of this chunk
    if (qk_wave) {
        // l of head l16 summed over the four lane groups (m_run already agrees)
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        if (g == 0) {
            s_linv[wave * 16 + l16] = l_run > 0.f ? 1.f / l_run : 0.f;
            // the chunk's (max, sum) relative to its largest score, which the
            // merge and the softmax_max / softmax_sum outputs use
            const bool any = l_run > 0.f;
            const float m_out = any ? m_true : m_run;
            const float l_out = any ? l_run * __builtin_amdgcn_exp2f(m_run - m_true) : 0.f;
            if (!P.direct && h_ok) *reinterpret_cast<float2 *>(P.part_ml + (prow + h) * 2) = make_float2(m_out, l_out);
            if (P.direct && h_ok && P.lse_max) {
                const int64_t o = (int64_t)qr * P.QN + h;
                P.lse_max[o] = any ? m_out * kLn2 : kNegInf;
                P.lse_sum[o] = l_out;
            }
        }
    }
    __syncthreads();
    // The wave's 64 x 128 block of the output, scaled and rounded, is staged
    // in LDS (the ring slots are free once every wave has passed the barrier
    // above) and written with 16-byte stores: 256 contiguous bytes per head,
    // instead of 2-byte stores that scatter 32-byte pieces.
    char *stg = (wave < 2 ? s_slot0 : s_slot2) + (wave & 1) * (64 * kStgPitch);
#pragma unroll
    for (int hg = 0; hg < kWavesPerBlock; hg++) {
        if (hg >= n_act) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = hg * 16 + 4 * g + i;
            const float inv = s_linv[row];
#pragma unroll
            for (int j = 0; j < 8; j++) M::store(stg, row * (kStgPitch / 2) + 16 * j + l16, acc[hg][j][i] * inv);
        }
    }
    char *dst = reinterpret_cast<char *>(P.direct ? P.out : P.part_o);
    const int64_t row0 = P.direct ? (int64_t)qr * P.QN : prow;
#pragma unroll
    for (int k = 0; k < 16; k++) {
        const int row = 4 * k + (lane >> 4);            // head of the block
        const int hh = hb * 64 + row;
        if (row >= 16 * n_act || hh >= P.QN) continue;
        const u32x4 x = *reinterpret_cast<const u32x4 *>(stg + row * kStgPitch + 16 * l16);
        *reinterpret_cast<u32x4 *>(dst + ((row0 + hh) * kD + 128 * wave + 8 * l16) * 2) = x;
    }
}

// All heads of a query row in one workgroup.  The planner takes it when there
// are more than 64 heads and the workgroups of 64 heads would not all fit on
// the compute units at once (one workgroup per CU): it halves that grid, so
// the call runs in one round instead of two.
//  * wave w scores heads 32w .. 32w+31 (two groups of 16) and accumulates
//    their P.V over all 512 output columns;
//  * so every gathered row is copied into LDS once per chunk, each key operand
//    read from LDS serves both head groups, P stays in the wave's registers
//    (the score layout is the P.V operand layout), and each wave keeps its own
//    heads' softmax state: no P, rescale factors or flags cross waves;
//  * the register file holds the query of 32 heads (144 registers) and the
//    accumulators of 32 heads x 512 columns (256); that fits with the
//    accumulators in VGPR-form MFMAs (this file's build flag) and the running
//    max rescale kept out of the score step (see below);
//  * the copy ring, the pipeline and the chunk table are those of sfa_kernel.
template <bool BF, bool ALIAS>
__global__ __launch_bounds__(256, 1) void sfa_wide_kernel(const SfaParams P) {
    using M = Mfma<BF>;
    using vec8 = typename M::vec8;
    __shared__ __attribute__((aligned(16))) char s_slot0[kSlot];
    __shared__ __attribute__((aligned(16))) char s_slot1[kSlot];
    __shared__ __attribute__((aligned(16))) char s_slot2[kSlot];
    __shared__ __attribute__((aligned(16))) char s_slot3[kSlot];
    __shared__ int32_t s_rows[kChunkMax];
    __shared__ int32_t s_cnt[2][kWavesPerBlock];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;

    // workgroup -> (query row, chunk); XCD x (ids congruent mod 8) takes the
    // contiguous groups [x g8, (x + 1) g8), so the chunks of a query row share
    // its query and block-table rows in one L2
    const int id = blockIdx.x;
    const int x8 = id & 7, k8 = id >> 3;
    const int g8 = (P.R * P.n_sc + 7) >> 3;
    const int grp = x8 * g8 + k8;
    if (grp >= P.R * P.n_sc) return;               // whole workgroup leaves together
    const int qr = grp / P.n_sc, sc = grp - qr * P.n_sc;
    const bool act = 32 * wave < P.QN;             // the wave has heads (wave-uniform)

    // ---------------------------------------------------- query rows (issued first)
    // qreg[hg]: head 32 wave + 16 hg + l16, dims 32 ks + 8 g .. + 7 of q | q_rope
    vec8 qreg[2][kDK / 32];
#pragma unroll
    for (int hg = 0; hg < 2; hg++) {
        const int h = 32 * wave + 16 * hg + l16;
#pragma unroll
        for (int ks = 0; ks < kDK / 32; ks++) {
            u32x4 x = {0, 0, 0, 0};
            if (h < P.QN) {
                const char *src = ks < kD / 32
                    ? reinterpret_cast<const char *>(P.q) + (((int64_t)qr * P.QN + h) * kD + 32 * ks + 8 * g) * 2
                    : reinterpret_cast<const char *>(P.q_rope) + (((int64_t)qr * P.QN + h) * kDR + 32 * (ks - kD / 32) + 8 * g) * 2;
                x = *reinterpret_cast<const u32x4 *>(src);
            }
            qreg[hg][ks] = __builtin_bit_cast(vec8, x);
        }
    }

    const int nv = compact_chunk(P, qr, sc, s_rows, s_cnt);

    // ---------------------------------------------------- gather copies
    const int n_tiles = (nv + kT - 1) / kT;
    auto rows_of = [&](int tile) { return tile_rows(s_rows, tile, nv, lane, wave); };
    auto issue_k = [&](char *slot, int rows) { issue_key_half(P, slot, rows, lane, wave); };
    auto issue_v = [&](char *slot, int rows) { issue_value_half(P, slot, rows, lane, wave); };

    // acc[hg][j]: heads 32 wave + 16 hg + 4g + i (i = 0..3), output column 16 j + l16
    floatx4 acc[2][kD / 16];
#pragma unroll
    for (int hg = 0; hg < 2; hg++)
#pragma unroll
        for (int j = 0; j < kD / 16; j++) acc[hg][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    // softmax state of head 32 wave + 16 hg + l16 (the lanes of one head agree)
    float m_run[2] = {kMaxInit, kMaxInit}, l_run[2] = {0.f, 0.f};
    float m_true[2] = {kNegInf, kNegInf};   // the largest score itself (m_run is raised lazily)
    vec8 pa[2];                              // P of the current tile, the A operand of P.V
    // A raised running max rescales the group's accumulators at the start of
    // the P.V step, behind a wave-uniform flag: any use of the accumulators
    // by vector instructions inside the score step made the compiler move
    // all of them between register files on every tile.
    float alpha_t[2] = {1.f, 1.f};           // rescale factor of head l16 for this tile
    bool raised[2] = {false, false};         // wave-uniform: the group raised its running max
    const float smul = P.score_mul;

    // scores of tile `tile` for both head groups from its key slot, the
    // online-softmax update and P
    auto qk = [&](int tile, const char *ks_, auto &&pre) {
        // 36 operand reads (row block i % 2, k-step i / 2), each feeding the
        // MFMAs of both head groups: four interleaved accumulation chains
        constexpr int kSteps = 2 * (kDK / 32);
        auto a_ptr = [&](int i) -> const char * {
            const int tb = i & 1, ks = i >> 1;
            const int r = tb * 16 + l16;
            if (ks < kD / 32) return ks_ + r * kRP + 64 * ks + 16 * g;
            return ks_ + kRopeOff + r * 128 + 16 * ((4 * (ks - kD / 32) + g) ^ rope_swz(r));
        };
        floatx4 sc2[2][2];
#pragma unroll
        for (int hg = 0; hg < 2; hg++) sc2[hg][0] = sc2[hg][1] = floatx4{0.f, 0.f, 0.f, 0.f};
        constexpr int kGrp = 6, kGroups = kSteps / kGrp;
        static_assert(kSteps % kGrp == 0, "group size");
        vec8 abuf[2][kGrp];
#pragma unroll
        for (int i = 0; i < kGrp; i++) abuf[0][i] = *reinterpret_cast<const vec8 *>(a_ptr(i));
        pre();
#pragma unroll
        for (int j = 0; j < kGroups; j++) {
            lds_wait();
            __builtin_amdgcn_sched_barrier(0);
            if (j + 1 < kGroups) {
#pragma unroll
                for (int i = 0; i < kGrp; i++)
                    abuf[(j + 1) & 1][i] = *reinterpret_cast<const vec8 *>(a_ptr((j + 1) * kGrp + i));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kGrp; i++) {
                const int st = j * kGrp + i;
#pragma unroll
                for (int hg = 0; hg < 2; hg++)
                    sc2[hg][st & 1] = M::run(abuf[j & 1][i], qreg[hg][st >> 1], sc2[hg][st & 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int hg = 0; hg < 2; hg++) {
            float p[8];
            float mt = kNegInf;
#pragma unroll
            for (int tb = 0; tb < 2; tb++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int r = tile * kT + tb * 16 + 4 * g + i;
                    const float s = r < nv ? sc2[hg][tb][i] * smul : kNegInf;
                    p[tb * 4 + i] = s;
                    mt = fmaxf(mt, s);
                }
            mt = max_xor16(mt);
            mt = max_xor32(mt);
            m_true[hg] = fmaxf(m_true[hg], mt);
            const bool raise = mt > m_run[hg] + kLazy;
            alpha_t[hg] = 1.f;
            if (__builtin_amdgcn_ballot_w64(raise)) {
                const float mn = raise ? mt : m_run[hg];
                const float alpha = __builtin_amdgcn_exp2f(m_run[hg] - mn);
                m_run[hg] = mn;
                l_run[hg] *= alpha;
                alpha_t[hg] = alpha;
                raised[hg] = tile > 0;
            }
#pragma unroll
            for (int i = 0; i < 8; i++) {
                p[i] = __builtin_amdgcn_exp2f(p[i] - m_run[hg]);
                l_run[hg] += p[i];
            }
            pa[hg] = M::pack(p);
        }
    };
    // O[h][d] += P[h][t] V~[t][d] for the wave's two head groups over all 512
    // columns; each transposed V~ operand serves both groups
    auto pv = [&](const char *vs_, auto &&pre) {
        const char *v0 = vs_ + (4 * g + (l16 >> 2)) * kRP + 8 * (l16 & 3);
        const char *v1 = v0 + 16 * kRP;
        constexpr int kPfV = 4, kGroups = (kD / 16) / kPfV;
        vec8 bbuf[2][kPfV];
#pragma unroll
        for (int i = 0; i < kPfV; i++) bbuf[0][i] = M::tr2(v0 + 32 * i, v1 + 32 * i);
        pre();
#pragma unroll
        for (int hg = 0; hg < 2; hg++) {
            if (!__builtin_amdgcn_readfirstlane((int)raised[hg])) continue;
            raised[hg] = false;
            // accumulator rows are heads 4g + i: their factors sit in lanes 4g + i
            float ai[4];
#pragma unroll
            for (int i = 0; i < 4; i++) ai[i] = __shfl(alpha_t[hg], 4 * g + i);
#pragma unroll
            for (int j = 0; j < kD / 16; j++)
#pragma unroll
                for (int i = 0; i < 4; i++) acc[hg][j][i] *= ai[i];
        }
#pragma unroll
        for (int jg = 0; jg < kGroups; jg++) {
            lds_wait();
            __builtin_amdgcn_sched_barrier(0);
            if (jg + 1 < kGroups) {
#pragma unroll
                for (int i = 0; i < kPfV; i++) {
                    const int j = (jg + 1) * kPfV + i;
                    bbuf[(jg + 1) & 1][i] = M::tr2(v0 + 32 * j, v1 + 32 * j);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kPfV; i++)
#pragma unroll
                for (int hg = 0; hg < 2; hg++)
                    acc[hg][jg * kPfV + i] = M::run(pa[hg], bbuf[jg & 1][i], acc[hg][jg * kPfV + i]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto end_half = [&]() { lds_wait(); };

    // ---------------------------------------------------- pipeline (as in sfa_kernel)
    if constexpr (ALIAS) {
        // the value rows are the key rows: one copy per tile into slot t % 4,
        // three tiles ahead; no P crosses waves, so one barrier a tile
        if (n_tiles > 0) {
            issue_k(s_slot0, rows_of(0));
            issue_k(s_slot1, rows_of(1));
            issue_k(s_slot2, rows_of(2));
        }
        auto step = [&](int t, char *cur, char *nxt) {
            wait_vmcnt<2 * kKIns>();
            ring_barrier();
            auto pre = [&]() { issue_k(nxt, rows_of(t + 3)); };
            if (act) {
                qk(t, cur, pre);
                pv(cur, [&]() {});
            } else {
                pre();
            }
            end_half();
        };
        for (int t = 0; t < n_tiles; t += 4) {
            step(t, s_slot0, s_slot3);
            if (t + 1 >= n_tiles) break;
            step(t + 1, s_slot1, s_slot0);
            if (t + 2 >= n_tiles) break;
            step(t + 2, s_slot2, s_slot1);
            if (t + 3 >= n_tiles) break;
            step(t + 3, s_slot3, s_slot2);
        }
    } else {
        int rows_n = 0;
        if (n_tiles > 0) {
            rows_n = rows_of(0);
            issue_k(s_slot0, rows_n);
            issue_v(s_slot1, rows_n);
            rows_n = rows_of(1);
            issue_k(s_slot2, rows_n);
        }
        for (int t = 0; t < n_tiles; t += 2) {
            wait_vmcnt<kKIns + kVIns>();
            ring_barrier();
            {
                auto pre = [&]() { issue_v(s_slot3, rows_n); rows_n = rows_of(t + 2); };
                if (act) qk(t, s_slot0, pre);
                else pre();
            }
            end_half();
            wait_vmcnt<kKIns + kVIns>();
            ring_barrier();
            {
                auto pre = [&]() { issue_k(s_slot0, rows_n); };
                if (act) pv(s_slot1, pre);
                else pre();
            }
            end_half();
            if (t + 1 >= n_tiles) break;
            wait_vmcnt<kKIns + kVIns>();
            ring_barrier();
            {
                auto pre = [&]() { issue_v(s_slot1, rows_n); rows_n = rows_of(t + 3); };
                if (act) qk(t + 1, s_slot2, pre);
                else pre();
            }
            end_half();
            wait_vmcnt<kKIns + kVIns>();
            ring_barrier();
            {
                auto pre = [&]() { issue_k(s_slot2, rows_n); };
                if (act) pv(s_slot3, pre);
                else pre();
            }
            end_half();
        }
    }
    wait_vmcnt<0>();

    // ---------------------------------------------------- epilogue
    const int64_t prow = ((int64_t)qr * P.n_sc + sc) * P.QN;  // partial rows of this chunk
    float linv[2] = {0.f, 0.f};
#pragma unroll
    for (int hg = 0; hg < 2; hg++) {
        // l of head l16 summed over the four lane groups (m_run already agrees)
        float l = l_run[hg];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        linv[hg] = l > 0.f ? 1.f / l : 0.f;
        const int h = 32 * wave + 16 * hg + l16;
        if (g == 0 && h < P.QN) {
            const bool any = l > 0.f;
            const float m_out = any ? m_true[hg] : m_run[hg];
            const float l_out = any ? l * __builtin_amdgcn_exp2f(m_run[hg] - m_true[hg]) : 0.f;
            if (!P.direct) *reinterpret_cast<float2 *>(P.part_ml + (prow + h) * 2) = make_float2(m_out, l_out);
            if (P.direct && P.lse_max) {
                const int64_t o = (int64_t)qr * P.QN + h;
                P.lse_max[o] = any ? m_out * kLn2 : kNegInf;
                P.lse_sum[o] = l_out;
            }
        }
    }
    // Every wave is past the ring; wave w stages its 32 heads x 512 columns,
    // scaled and rounded, in ring slot w (1040-byte rows: the 2-byte writes of
    // the four lane groups, heads 4 apart, fall in distinct banks) and writes
    // them with 16-byte stores, one 1 KiB head row per instruction.
    __syncthreads();
    if (!act) return;
    constexpr int kWPitch = 1040;
    static_assert(32 * kWPitch <= kSlot, "a wave's output block fits one ring slot");
    char *stg = wave == 0 ? s_slot0 : wave == 1 ? s_slot1 : wave == 2 ? s_slot2 : s_slot3;
#pragma unroll
    for (int hg = 0; hg < 2; hg++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = 16 * hg + 4 * g + i;
            const float inv = __shfl(linv[hg], 4 * g + i);
#pragma unroll
            for (int j = 0; j < kD / 16; j++) M::store(stg, row * (kWPitch / 2) + 16 * j + l16, acc[hg][j][i] * inv);
        }
    }
    char *dst = reinterpret_cast<char *>(P.direct ? P.out : P.part_o);
    const int64_t row0 = P.direct ? (int64_t)qr * P.QN : prow;
#pragma unroll
    for (int r = 0; r < 32; r++) {
        const int hh = 32 * wave + r;
        if (hh >= P.QN) break;
        const u32x4 x = *reinterpret_cast<const u32x4 *>(stg + r * kWPitch + 16 * lane);
        *reinterpret_cast<u32x4 *>(dst + ((row0 + hh) * kD + 8 * lane) * 2) = x;
    }
}

// Merges the chunk outputs of one (query row, head) in chunk order:
// out = sum_s w_s o_s / sum_s w_s with w_s = l_s 2^(m_s - max m), and rounds.
template <bool BF>
__global__ __launch_bounds__(256) void sfa_combine_kernel(const SfaParams P) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= P.R * P.QN) return;
    const int qr = row / P.QN, hh = row - qr * P.QN;
    const float2 *ml = reinterpret_cast<const float2 *>(P.part_ml);
    auto prow = [&](int s) -> int64_t { return ((int64_t)qr * P.n_sc + s) * P.QN + hh; };
    // lane l merges elements 8 l .. 8 l + 7 of the head's row: one 16-byte
    // load per chunk
    const char *po = reinterpret_cast<const char *>(P.part_o) + 16 * lane;
    auto part = [&](int s) { return *reinterpret_cast<const u32x4v *>(po + prow(s) * (kD * 2)); };
    auto elem = [](const u32x4v &x, int e) -> float {
        const uint32_t w = x[e >> 1];
        const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
        return BF ? __builtin_bit_cast(float, h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    };
    // One memory round trip for the common case: lane s holds (m, l) of chunk
    // s (s < 64), and the rows of the first U chunks are requested with them.
    const int n = P.n_sc;
    constexpr int U = 8;
    float2 v0 = make_float2(kNegInf, 0.f);
    if (lane < n) v0 = ml[prow(lane)];
    u32x4v x[U];
#pragma unroll
    for (int u = 0; u < U; u++) x[u] = part(min(u, n - 1));
    float Mx = v0.x;
    for (int s0 = 64; s0 < n; s0 += 64)
        if (s0 + lane < n) Mx = fmaxf(Mx, ml[prow(s0 + lane)].x);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Mx = fmaxf(Mx, __shfl_xor(Mx, o));
    // weight of chunk `lane` (0 past the last chunk: l = 0 there)
    const float w0 = v0.y * __builtin_amdgcn_exp2f(v0.x - Mx);
    float L = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; e++) o[e] = 0.f;
    // chunks in order: the first U from registers, the rest one by one
#pragma unroll
    for (int u = 0; u < U; u++) {
        if (u >= n) break;
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w0), u));
        L += w;
#pragma unroll
        for (int e = 0; e < 8; e++) o[e] += w * elem(x[u], e);
    }
    for (int s = U; s < n; s++) {
        const u32x4v xs = part(s);
        const float2 v = ml[prow(s)];
        const float w = v.y * __builtin_amdgcn_exp2f(v.x - Mx);
        L += w;
#pragma unroll
        for (int e = 0; e < 8; e++) o[e] += w * elem(xs, e);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (P.lse_max && lane == 0) {   // softmax_max / softmax_sum of the row (natural-log domain)
        const int64_t oi = (int64_t)qr * P.QN + hh;
        P.lse_max[oi] = L > 0.f ? Mx * kLn2 : kNegInf;
        P.lse_sum[oi] = L;
    }
    u32x4v y;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        uint32_t lo, hi;
        if (BF) {
            lo = __builtin_bit_cast(uint16_t, (__bf16)(o[e] * inv));
            hi = __builtin_bit_cast(uint16_t, (__bf16)(o[e + 1] * inv));
        } else {
            lo = __builtin_bit_cast(uint16_t, (_Float16)(o[e] * inv));
            hi = __builtin_bit_cast(uint16_t, (_Float16)(o[e + 1] * inv));
        }
        y[e >> 1] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4v *>(reinterpret_cast<char *>(P.out) + (((int64_t)qr * P.QN + hh) * kD + 8 * lane) * 2) = y;
}

}  // namespace sfa_detail

hipError_t sfa_launch(const SfaParams &p, bool bf16, int grid, hipStream_t s, hipEvent_t ev_begin,
                      hipEvent_t ev_end) {
    using namespace sfa_detail;
    if (ev_begin && hipEventRecord(ev_begin, s) != hipSuccess) return hipErrorUnknown;
    // a value tensor that is the key tensor takes the pipelines that copy each
    // row once
    const bool alias = p.value == p.key;
    auto kernel = p.wide ? (bf16 ? (alias ? sfa_wide_kernel<true, true> : sfa_wide_kernel<true, false>)
                                 : (alias ? sfa_wide_kernel<false, true> : sfa_wide_kernel<false, false>))
                         : (bf16 ? (alias ? sfa_kernel<true, true> : sfa_kernel<true, false>)
                                 : (alias ? sfa_kernel<false, true> : sfa_kernel<false, false>));
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_end && hipEventRecord(ev_end, s) != hipSuccess) return hipErrorUnknown;
    if (!p.direct) {
        const int rows = p.R * p.QN;
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
