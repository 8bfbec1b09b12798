// Host side of libifadecode: argument validation, the split planner and the
// launches behind the C ABI declared in include/ifa_decode.h.
//
// Validation follows the parameter tables and constraint lists of the
// IncreFlashAttention README, the aclnnIncreFlashAttentionV2 page and the
// SparseFlashAttention README; it makes no HIP call, so an invalid call
// returns before touching the device.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <stddef.h>

#include <algorithm>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "ifa_decode.h"
#include "internal.h"
#include "sfa.h"

namespace {

using namespace ifa;

constexpr int kAbiVersion = 7;
constexpr int kRowModeTiles = 4;     // longest row (in split-kernel tiles) that row mode takes

bool is_float_dt(int dt) { return dt == IFA_DT_F16 || dt == IFA_DT_BF16; }

int parse_layout(const char *s, int *out) {
    if (!s || !strcmp(s, "BSH")) { *out = 0; return IFA_OK; }
    if (!strcmp(s, "BNSD")) { *out = 1; return IFA_OK; }
    if (!strcmp(s, "BSND")) { *out = 2; return IFA_OK; }
    return IFA_ERR_PARAM_INVALID;
}

// ----------------------------------------------------------------- planning

struct Window { int32_t lo, hi; };

// One launch covers up to kSliceBatches batches.
struct SlicePlan {
    int b0 = 0, nb = 0;
    int64_t total = 0, piece = 0;
    int32_t seg_cost = 0;
    int n_pieces = 0;
    std::vector<int64_t> pre;         // nb + 1 entries
    std::vector<int32_t> sbase, maxseg;
    int64_t slot_base = 0, slots = 0;
};

// The head dim a call runs on: the smallest compiled size that holds D.
int compiled_head_dim(int D) { return D <= 64 ? 64 : D <= 128 ? 128 : D <= 256 ? 256 : 512; }

struct IfaPlan {
    int kv = 0, D = 0, G = 0, n_hg = 0, g = 0, N = 0, Nkv = 0, B = 0;
    int Dc = 0;                          // compiled head dim: the smallest of 64/128/256/512 >= D
    bool paged = false;
    bool out_i8 = false;                 // int8 output (finished by the combine)
    bool row_mode = false;               // one workgroup per row, finished in place, no combine
    int extra = EX_NONE;                 // split kernel variant (mask / positional bias)
    std::vector<Window> win;             // per batch
    std::vector<int64_t> list_seq;       // per-batch caches: positions of each tensor
    std::vector<SlicePlan> slices;
    int64_t total_slots = 0;
    size_t workspace = 0;
};

std::mutex g_mu;
int g_resident[64][3][4][4][2][3];   // [dev][kv][log2 D/64][log2 G][paged][extra] resident waves, 0 = unknown

int current_device(int *dev) { return hipGetDevice(dev) == hipSuccess ? IFA_OK : IFA_ERR_RUNTIME; }

int resident_waves(int kv, int D, int G, bool paged, int extra) {
    int dev = 0;
    if (current_device(&dev) != IFA_OK || dev < 0 || dev >= 64) return 0;
    const int di = D == 64 ? 0 : D == 128 ? 1 : D == 256 ? 2 : 3;
    const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
    std::lock_guard<std::mutex> lk(g_mu);
    int &slot = g_resident[dev][kv][di][gi][paged ? 1 : 0][extra];
    if (!slot) slot = split_resident_waves(kv, D, G, paged, extra);
    return slot;
}

// Balancing: the rows (b, j, hg) of a slice are laid end to end, each row
// start charged a tile and a half of extra cost, and the cost is cut into
// n_pieces equal pieces, one per resident wave of the split kernel, so every
// wave gets the same work (positions plus row starts).  A row meets at most
// ceil(len / piece) + 1 pieces, which bounds its partial slots.
int finish_plan(IfaPlan &p, int64_t split_tokens) {
    p.G = 1;
    while (p.G < p.g && p.G < 8) p.G <<= 1;
    p.n_hg = (p.g + p.G - 1) / p.G;
    int waves = 0;
    if (split_tokens <= 0) {
        waves = resident_waves(p.kv, p.Dc, p.G, p.paged, p.extra);
        if (waves <= 0) return IFA_ERR_RUNTIME;
        // A plain dense stream with head groups of 2 or 4 (8-row tiles, 16 KB of
        // K/V in flight per wave) reads HBM faster with half the resident waves,
        // one per SIMD, each streaming twice as far: measured 4-9 % faster on
        // MI355X.  Paged, masked, biased, int8 and 8-head-group kernels do more
        // work per byte or keep fewer bytes in flight, and stay at full residency.
        if (!p.paged && p.extra == EX_NONE && p.kv != KV_I8 && (p.G == 2 || p.G == 4))
            waves = std::max(1, waves / 2);
    }
    const int64_t rows_per_batch = (int64_t)p.Nkv * p.n_hg;
    p.slices.clear();
    p.total_slots = 0;
    // Row mode: when every row is at most a few tiles long and the rows fit in
    // the resident waves, one workgroup per row finishes the call in one
    // launch: its four waves take a quarter of the window each (one tile at
    // most), merge their states in LDS and write the output.  A second launch
    // for the combine would cost more than the whole stream.  16-bit caches
    // and outputs only (the int8 epilogues live in the combine).
    p.row_mode = false;
    if (split_tokens <= 0 && p.kv != KV_I8 && !p.out_i8 && p.B <= kSliceBatches) {
        const int64_t tile = (int64_t)(p.G >= 8 ? 4 : 8) * (512 / p.Dc);   // positions per split-kernel tile
        int32_t max_len = 0;
        for (const Window &w : p.win) max_len = std::max(max_len, w.hi - w.lo);
        p.row_mode = max_len <= kRowModeTiles * tile && (int64_t)p.B * rows_per_batch * kWavesPerBlock <= waves &&
                     (int64_t)p.B * rows_per_batch <= kRowTab;
    }
    if (p.row_mode) {
        SlicePlan sp;
        sp.b0 = 0;
        sp.nb = p.B;
        sp.pre.resize(sp.nb + 1);
        sp.sbase.assign(sp.nb, 0);
        sp.maxseg.assign(sp.nb, 0);
        int64_t pos = 0, max_len = 1;
        for (int i = 0; i < sp.nb; i++) {
            sp.pre[i] = pos;
            pos += (int64_t)(p.win[i].hi - p.win[i].lo) * rows_per_batch;
            max_len = std::max<int64_t>(max_len, p.win[i].hi - p.win[i].lo);
        }
        sp.pre[sp.nb] = pos;
        sp.total = pos;
        sp.piece = max_len;
        sp.n_pieces = (int)(sp.nb * rows_per_batch * kWavesPerBlock);   // one workgroup per row
        p.slices.push_back(std::move(sp));
        p.workspace = 0;
        return IFA_OK;
    }
    for (int b0 = 0; b0 < p.B; b0 += kSliceBatches) {
        SlicePlan sp;
        sp.b0 = b0;
        sp.nb = std::min(kSliceBatches, p.B - b0);
        sp.pre.resize(sp.nb + 1);
        sp.sbase.resize(sp.nb);
        sp.maxseg.resize(sp.nb);
        int64_t pos = 0;
        for (int i = 0; i < sp.nb; i++) {
            sp.pre[i] = pos;
            pos += (int64_t)(p.win[b0 + i].hi - p.win[b0 + i].lo) * rows_per_batch;
        }
        sp.pre[sp.nb] = pos;
        sp.total = pos;
        // Each row start is charged about a tile and a half of positions: a
        // wave whose piece starts a new row (a new query, first tiles, a
        // partial state written) measured about that much longer.  With an
        // explicit work-item size a piece is exactly that many positions.
        const int64_t tile = (int64_t)(p.G >= 8 ? 4 : 8) * (512 / p.Dc);
        sp.seg_cost = split_tokens > 0 ? 0 : (int32_t)(3 * tile / 2);
        const int64_t total_cost = pos + (int64_t)sp.seg_cost * rows_per_batch * sp.nb;
        if (split_tokens > 0) sp.piece = split_tokens;
        else sp.piece = std::max<int64_t>(64, (total_cost + waves - 1) / std::max(1, waves));
        sp.n_pieces = (int)((total_cost + sp.piece - 1) / sp.piece);
        int64_t slots = 0;
        for (int i = 0; i < sp.nb; i++) {
            const int64_t len = p.win[b0 + i].hi - p.win[b0 + i].lo;
            sp.maxseg[i] = len > 0 ? (int32_t)((len + sp.piece - 1) / sp.piece + 1) : 0;
            sp.sbase[i] = (int32_t)slots;
            slots += rows_per_batch * sp.maxseg[i];
        }
        if (slots > INT32_MAX || total_cost / sp.piece > INT32_MAX) return IFA_ERR_PARAM_INVALID;
        sp.slot_base = p.total_slots;
        sp.slots = slots;
        p.total_slots += slots;
        p.slices.push_back(std::move(sp));
    }
    const size_t acc = (size_t)p.total_slots * p.G * p.Dc * sizeof(float);
    const size_t ml = (size_t)p.total_slots * p.G * 2 * sizeof(float);
    p.workspace = (acc + 255) / 256 * 256 + (ml + 255) / 256 * 256;
    if (getenv("IFA_DEBUG_PLAN")) {
        for (const SlicePlan &sp : p.slices)
            fprintf(stderr, "ifa plan: kv=%d D=%d g=%d G=%d n_hg=%d slice b0=%d nb=%d positions=%lld piece=%lld "
                    "waves=%d slots=%lld\n", p.kv, p.D, p.g, p.G, p.n_hg, sp.b0, sp.nb, (long long)sp.total,
                    (long long)sp.piece, sp.n_pieces, (long long)sp.slots);
    }
    return IFA_OK;
}

// ----------------------------------------------------------------- IFA validation

struct IfaCommon {
    int layout = 0;
    int64_t Nkv = 0;
};

// Output quantisation fields (int8 output); zero when the caller's struct predates them.
struct QuantArgs {
    const void *scale = nullptr, *offset = nullptr;
    int64_t count = 0;
    int dtype = 0;
};

int check_quant(int dq, int dout, int64_t N, int64_t D, const QuantArgs &qa) {
    if (dout != IFA_DT_I8) return qa.scale || qa.offset ? IFA_ERR_PARAM_INVALID : IFA_OK;
    if (!qa.scale) return IFA_ERR_PARAM_NULLPTR;                     // README: quantScale2 required
    if (qa.dtype != IFA_DT_F32 && !(qa.dtype == IFA_DT_BF16 && dq == IFA_DT_BF16)) return IFA_ERR_PARAM_INVALID;
    if (qa.count != 1 && qa.count != N * D) return IFA_ERR_PARAM_INVALID;
    return IFA_OK;
}

int check_common(const void *q, const void *out, int dq, int dkv, int dout, const char *layout, int64_t B, int64_t N,
                 int64_t Nkv_in, int64_t D, double scale, const void *mask, int dmask, int64_t mB, int64_t mN,
                 const void *pse, int64_t pse_b, const void *aqs, const void *aqo, int aq_mode,
                 int64_t split_tokens, IfaCommon *c) {
    if (!q || !out) return IFA_ERR_PARAM_NULLPTR;
    if (!is_float_dt(dq) || (dout != dq && dout != IFA_DT_I8)) return IFA_ERR_PARAM_INVALID;
    if (dkv != dq && dkv != IFA_DT_I8) return IFA_ERR_PARAM_INVALID;
    if (parse_layout(layout, &c->layout) != IFA_OK) return IFA_ERR_PARAM_INVALID;
    if (B < 1 || B > 65536 || N < 1 || N > 256) return IFA_ERR_PARAM_INVALID;
    if (Nkv_in < 0 || Nkv_in > N) return IFA_ERR_PARAM_INVALID;
    c->Nkv = Nkv_in == 0 ? N : Nkv_in;
    if (N % c->Nkv) return IFA_ERR_PARAM_INVALID;
    // any head dim up to 512 that keeps rows in whole 16-byte lanes; the
    // kernels run it on the next compiled size (64, 128, 256, 512)
    if (D < 8 || D > 512 || D % 8) return IFA_ERR_PARAM_INVALID;
    if (!std::isfinite(scale)) return IFA_ERR_PARAM_INVALID;
    if (mask) {
        if (dmask != IFA_DT_BOOL && dmask != IFA_DT_I8 && dmask != IFA_DT_U8) return IFA_ERR_PARAM_INVALID;
        if ((mB != 1 && mB != B) || (mN != 1 && mN != N)) return IFA_ERR_PARAM_INVALID;
    }
    if (pse && pse_b != 1 && pse_b != B) return IFA_ERR_PARAM_INVALID;
    if (dkv == IFA_DT_I8) {
        if (aq_mode != IFA_ANTIQUANT_PER_TENSOR && aq_mode != IFA_ANTIQUANT_PER_CHANNEL) return IFA_ERR_PARAM_INVALID;
        if (!aqs || !aqo) return IFA_ERR_PARAM_NULLPTR;
    } else if (aq_mode != IFA_ANTIQUANT_NONE || aqs || aqo) {
        return IFA_ERR_PARAM_INVALID;
    }
    if (split_tokens < 0 || split_tokens % 16 || split_tokens > (1 << 24)) return IFA_ERR_PARAM_INVALID;
    return IFA_OK;
}

int kv_kind(int dkv) { return dkv == IFA_DT_F16 ? KV_F16 : dkv == IFA_DT_BF16 ? KV_BF16 : KV_I8; }

QuantArgs dense_quant(const ifa_decode_args *a) {
    QuantArgs q;
    if (a->struct_size >= sizeof(ifa_decode_args)) {
        q.scale = a->quant_scale2;
        q.offset = a->quant_offset2;
        q.count = a->quant_count;
        q.dtype = a->dtype_quant;
    }
    return q;
}

QuantArgs paged_quant(const ifa_paged_args *a) {
    QuantArgs q;
    if (a->struct_size >= sizeof(ifa_paged_args)) {
        q.scale = a->quant_scale2;
        q.offset = a->quant_offset2;
        q.count = a->quant_count;
        q.dtype = a->dtype_quant;
    }
    return q;
}

int plan_dense(const ifa_decode_args *a, IfaPlan &p, IfaCommon &c) {
    if (!a) return IFA_ERR_PARAM_NULLPTR;
    if (a->struct_size < offsetof(ifa_decode_args, pse_batch)) return IFA_ERR_PARAM_INVALID;
    const bool has_pse_dims = a->struct_size >= offsetof(ifa_decode_args, key_list);
    if (a->pse_shift && !has_pse_dims) return IFA_ERR_PARAM_INVALID;
    int rc = check_common(a->query, a->attention_out, a->dtype_q, a->dtype_kv, a->dtype_out, a->input_layout,
                          a->batch, a->num_heads, a->num_key_value_heads, a->head_dim, a->scale_value, a->atten_mask,
                          a->dtype_mask, a->mask_batch, a->mask_heads, a->pse_shift,
                          has_pse_dims ? a->pse_batch : 0, a->antiquant_scale, a->antiquant_offset,
                          a->antiquant_mode, a->split_tokens, &c);
    if (rc) return rc;
    // per-batch caches (tensor lists), from ABI version 4 on
    const bool has_lists = a->struct_size >= offsetof(ifa_decode_args, quant_scale2);
    const bool lists = has_lists && (a->key_list || a->value_list || a->kv_list_seq_len);
    if (lists) {
        if (!a->key_list || !a->value_list || !a->kv_list_seq_len) return IFA_ERR_PARAM_NULLPTR;
        if (a->key || a->value || a->kv_padding_size || a->batch > 256) return IFA_ERR_PARAM_INVALID;
        p.list_seq.assign(a->kv_list_seq_len, a->kv_list_seq_len + a->batch);
        for (int64_t sb : p.list_seq)
            if (sb < 1 || sb > (int64_t)1 << 30) return IFA_ERR_PARAM_INVALID;
    } else {
        if (!a->key || !a->value) return IFA_ERR_PARAM_NULLPTR;
        p.list_seq.clear();
    }
    rc = check_quant(a->dtype_q, a->dtype_out, a->num_heads, a->head_dim, dense_quant(a));
    if (rc) return rc;
    const int64_t S = lists ? 0 : a->kv_seq_len;
    if (!lists && (S < 1 || S > (int64_t)1 << 30)) return IFA_ERR_PARAM_INVALID;
    if (a->kv_padding_size && a->kv_padding_size_count != 1 && a->kv_padding_size_count != a->batch)
        return IFA_ERR_PARAM_INVALID;
    p.B = (int)a->batch;
    p.N = (int)a->num_heads;
    p.Nkv = (int)c.Nkv;
    p.g = p.N / p.Nkv;
    p.D = (int)a->head_dim;
    p.Dc = compiled_head_dim(p.D);
    p.kv = kv_kind(a->dtype_kv);
    p.paged = false;
    p.win.resize(p.B);
    int64_t max_hi = 0;
    for (int b = 0; b < p.B; b++) {
        const int64_t Sb = lists ? p.list_seq[b] : S;
        int64_t L = Sb, lo = 0, hi = Sb;
        if (a->actual_seq_lengths) {
            L = a->actual_seq_lengths[b];
            if (L < 0 || L > Sb) return IFA_ERR_PARAM_INVALID;
            lo = 0;
            hi = L;
            if (a->kv_padding_size) {
                int64_t pad = a->kv_padding_size[a->kv_padding_size_count == 1 ? 0 : b];
                if (pad < 0) pad = 0;                       // README: pad < 0 is set to 0
                lo = S - pad - L;
                hi = S - pad;
                if (lo < 0 || hi < 0) lo = hi = 0;         // README: start or end < 0 -> zeros
            }
        }
        p.win[b] = {(int32_t)lo, (int32_t)hi};
        max_hi = std::max(max_hi, hi);
    }
    if (a->atten_mask && a->mask_seq < max_hi) return IFA_ERR_PARAM_INVALID;
    if (a->pse_shift && a->pse_seq < max_hi) return IFA_ERR_PARAM_INVALID;
    p.extra = a->pse_shift ? EX_PSE : a->atten_mask ? EX_MASK : EX_NONE;
    p.out_i8 = a->dtype_out == IFA_DT_I8;
    return IFA_OK;
}

int plan_paged(const ifa_paged_args *a, IfaPlan &p, IfaCommon &c) {
    if (!a) return IFA_ERR_PARAM_NULLPTR;
    if (a->struct_size < offsetof(ifa_paged_args, pse_batch)) return IFA_ERR_PARAM_INVALID;
    const bool has_pse_dims = a->struct_size >= offsetof(ifa_paged_args, quant_scale2);
    if (a->pse_shift && !has_pse_dims) return IFA_ERR_PARAM_INVALID;
    int rc = check_common(a->query, a->attention_out, a->dtype_q, a->dtype_kv, a->dtype_out, a->input_layout,
                          a->batch, a->num_heads, a->num_key_value_heads, a->head_dim, a->scale_value, a->atten_mask,
                          a->dtype_mask, a->mask_batch, a->mask_heads, a->pse_shift,
                          has_pse_dims ? a->pse_batch : 0, a->antiquant_scale, a->antiquant_offset,
                          a->antiquant_mode, a->split_tokens, &c);
    if (rc) return rc;
    if (!a->key_cache || !a->value_cache || !a->block_table || !a->actual_seq_lengths) return IFA_ERR_PARAM_NULLPTR;
    rc = check_quant(a->dtype_q, a->dtype_out, a->num_heads, a->head_dim, paged_quant(a));
    if (rc) return rc;
    const int64_t bs = a->block_size;
    const int align = a->dtype_kv == IFA_DT_I8 ? 32 : 16;
    if (bs < 16 || bs > 512 || bs % align) return IFA_ERR_PARAM_INVALID;
    if (a->max_blocks_per_seq < 1 || a->num_blocks < 1 || a->num_blocks > INT32_MAX) return IFA_ERR_PARAM_INVALID;
    if (a->kv_cache_layout != 0 && a->kv_cache_layout != 1) return IFA_ERR_PARAM_INVALID;
    // README: BSH / BSND queries only pair with the (blocknum, blocksize, H) cache.
    if (a->kv_cache_layout == 0 && c.layout != 1) return IFA_ERR_PARAM_INVALID;
    const int64_t reach = a->max_blocks_per_seq * bs;
    if (reach > (int64_t)1 << 30) return IFA_ERR_PARAM_INVALID;
    p.B = (int)a->batch;
    p.N = (int)a->num_heads;
    p.Nkv = (int)c.Nkv;
    p.g = p.N / p.Nkv;
    p.D = (int)a->head_dim;
    p.Dc = compiled_head_dim(p.D);
    p.kv = kv_kind(a->dtype_kv);
    p.paged = true;
    p.win.resize(p.B);
    int64_t max_hi = 0, blocks_needed = 0;
    for (int b = 0; b < p.B; b++) {
        const int64_t L = a->actual_seq_lengths[b];
        if (L < 0 || L > reach) return IFA_ERR_PARAM_INVALID;
        p.win[b] = {0, (int32_t)L};
        max_hi = std::max(max_hi, L);
        blocks_needed += (L + bs - 1) / bs;
    }
    // README: blocknum may not be smaller than the blocks the lengths need.
    if (blocks_needed > a->num_blocks) return IFA_ERR_PARAM_INVALID;
    if (a->atten_mask && a->mask_seq < max_hi) return IFA_ERR_PARAM_INVALID;
    if (a->pse_shift && a->pse_seq < max_hi) return IFA_ERR_PARAM_INVALID;
    p.extra = a->pse_shift ? EX_PSE : a->atten_mask ? EX_MASK : EX_NONE;
    p.out_i8 = a->dtype_out == IFA_DT_I8;
    return IFA_OK;
}

// ----------------------------------------------------------------- launching

uint32_t bs_magic(uint32_t d, int *shift) {
    int l = 0;
    while (((uint64_t)1 << l) < d) l++;
    *shift = l;
    return (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
}

struct Launch {
    const void *q, *k, *v;
    void *out;
    const uint8_t *mask;
    int64_t mask_sB, mask_sH;
    int mask_mode;
    const void *pse;
    int64_t pse_sB, pse_sH;
    const int32_t *block_table;
    int64_t sB, sN, sS, blk_stride, head_stride, row_stride;
    int max_blocks, block_size, num_blocks;
    const void *aqs, *aqo;
    int aq_mode;
    const void *const *k_list;
    const void *const *v_list;
    int list_bnsd;
    QuantArgs quant;
    bool out_i8;
    bool q_bf16;
    double scale;
    hipEvent_t ev_begin, ev_end;
};

int run(const IfaPlan &p, const Launch &L, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (p.workspace && !ws) return IFA_ERR_PARAM_NULLPTR;
    if (ws_bytes < p.workspace) return IFA_ERR_PARAM_INVALID;
    float *part_acc = reinterpret_cast<float *>(ws);
    const size_t acc_bytes = ((size_t)p.total_slots * p.G * p.Dc * sizeof(float) + 255) / 256 * 256;
    float *part_ml = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + acc_bytes);

    SplitParams sp;
    memset(&sp, 0, sizeof sp);
    sp.q = L.q;
    sp.k = L.k;
    sp.v = L.v;
    sp.mask = L.mask;
    sp.pse = L.pse;
    sp.pse_sB = L.pse_sB;
    sp.pse_sH = L.pse_sH;
    sp.block_table = L.block_table;
    sp.k_scale = L.aqs;
    sp.k_list = L.k_list;
    sp.v_list = L.v_list;
    sp.list_bnsd = L.list_bnsd;
    sp.sB = L.sB;
    sp.sN = L.sN;
    sp.sS = L.sS;
    sp.blk_stride = L.blk_stride;
    sp.head_stride = L.head_stride;
    sp.row_stride = L.row_stride;
    sp.mask_sB = L.mask_sB;
    sp.mask_sH = L.mask_sH;
    sp.N = p.N;
    sp.Nkv = p.Nkv;
    sp.g = p.g;
    sp.n_hg = p.n_hg;
    sp.max_blocks = L.max_blocks;
    sp.block_size = L.block_size;
    sp.num_blocks = L.num_blocks;
    if (p.paged) sp.bs_magic = bs_magic((uint32_t)L.block_size, &sp.bs_shift);
    sp.mask_mode = L.mask_mode;
    sp.aq_mode = L.aq_mode;
    sp.q_bf16 = L.q_bf16;
    sp.score_mul = (float)(L.scale * 1.4426950408889634);
    sp.out = L.out;
    sp.row_mode = p.row_mode ? 1 : 0;
    const int64_t rows_pb = (int64_t)p.Nkv * p.n_hg;
    if (p.row_mode) {
        for (int64_t r = 0; r < (int64_t)p.B * rows_pb; r++) {
            const Window &w = p.win[r / rows_pb];
            sp.row_win[r] = ((int64_t)(w.hi - w.lo) << 32) | (uint32_t)w.lo;
        }
    }
    sp.Dr = p.D;

    CombineParams cp;
    memset(&cp, 0, sizeof cp);
    cp.out = L.out;
    cp.v_scale = L.aqs;
    cp.v_offset = L.aqo;
    cp.N = p.N;
    cp.Nkv = p.Nkv;
    cp.g = p.g;
    cp.G = p.G;
    cp.n_hg = p.n_hg;
    cp.D = p.Dc;
    cp.Dr = p.D;
    cp.out_bf16 = L.q_bf16;
    cp.aq_mode = L.aq_mode;
    cp.out_i8 = L.out_i8;
    cp.q_scale2 = L.quant.scale;
    cp.q_offset2 = L.quant.offset;
    cp.q2_bf16 = L.quant.dtype == IFA_DT_BF16;
    cp.q2_per_channel = L.quant.count > 1;

    const bool timed = L.ev_begin && L.ev_end;
    if (timed && hipEventRecord(L.ev_begin, stream) != hipSuccess) return IFA_ERR_RUNTIME;
    for (size_t si = 0; si < p.slices.size(); si++) {
        const SlicePlan &s = p.slices[si];
        sp.nb = cp.nb = s.nb;
        sp.b0 = cp.b0 = s.b0;
        sp.total = s.total;
        sp.piece = cp.piece = s.piece;
        sp.seg_cost = cp.seg_cost = s.seg_cost;
        sp.n_pieces = s.n_pieces;
        for (int i = 0; i < s.nb; i++) {
            sp.pre[i] = cp.pre[i] = s.pre[i];
            sp.lo[i] = p.win[s.b0 + i].lo;
            sp.len[i] = cp.len[i] = p.win[s.b0 + i].hi - p.win[s.b0 + i].lo;
            sp.sbase[i] = cp.sbase[i] = s.sbase[i];
            sp.maxseg[i] = cp.maxseg[i] = s.maxseg[i];
            sp.list_seq[i] = p.list_seq.empty() ? 0 : (int32_t)p.list_seq[s.b0 + i];
        }
        sp.pre[s.nb] = cp.pre[s.nb] = s.pre[s.nb];
        sp.part_acc = part_acc + s.slot_base * p.G * p.Dc;
        sp.part_ml = part_ml + s.slot_base * p.G * 2;
        cp.part_acc = sp.part_acc;
        cp.part_ml = sp.part_ml;
        if ((s.total > 0 || p.row_mode) && launch_split(sp, p.kv, p.Dc, p.G, p.paged, p.extra, stream) != hipSuccess)
            return IFA_ERR_RUNTIME;
        if (timed && si + 1 == p.slices.size() && hipEventRecord(L.ev_end, stream) != hipSuccess)
            return IFA_ERR_RUNTIME;
        if (!p.row_mode && launch_combine(cp, stream) != hipSuccess) return IFA_ERR_RUNTIME;
    }
    return IFA_OK;
}

Launch dense_launch(const ifa_decode_args *a, const IfaPlan &p, const IfaCommon &c) {
    Launch L;
    memset(&L, 0, sizeof L);
    L.q = a->query;
    L.k = a->key;
    L.v = a->value;
    L.out = a->attention_out;
    const int64_t S = a->kv_seq_len, D = p.D, Nkv = p.Nkv;
    if (!p.list_seq.empty()) {   // per-batch tensors: batch 0 of each; BNSD head stride from its S
        L.k_list = a->key_list;
        L.v_list = a->value_list;
        L.list_bnsd = c.layout == 1;
    }
    if (c.layout == 1) {         // BNSD: [B, Nkv, S, D]
        L.sB = Nkv * S * D;
        L.sN = S * D;
        L.sS = D;
    } else {                     // BSH / BSND: [B, S, Nkv, D]
        L.sB = S * Nkv * D;
        L.sN = D;
        L.sS = Nkv * D;
    }
    if (a->atten_mask) {
        L.mask = reinterpret_cast<const uint8_t *>(a->atten_mask);
        L.mask_sB = a->mask_batch == 1 ? 0 : a->mask_heads * a->mask_seq;
        L.mask_sH = a->mask_heads == 1 ? 0 : a->mask_seq;
        L.mask_mode = a->mask_heads == 1 ? 1 : 2;
    }
    if (a->pse_shift) {
        L.pse = a->pse_shift;
        L.pse_sB = a->pse_batch == 1 ? 0 : a->num_heads * a->pse_seq;
        L.pse_sH = a->pse_seq;
    }
    L.aqs = a->antiquant_scale;
    L.aqo = a->antiquant_offset;
    L.aq_mode = a->dtype_kv == IFA_DT_I8 ? a->antiquant_mode : 0;
    L.q_bf16 = a->dtype_q == IFA_DT_BF16;
    L.scale = a->scale_value;
    L.out_i8 = a->dtype_out == IFA_DT_I8;
    L.quant = dense_quant(a);
    L.ev_begin = reinterpret_cast<hipEvent_t>(a->profile_event_begin);
    L.ev_end = reinterpret_cast<hipEvent_t>(a->profile_event_end);
    return L;
}

Launch paged_launch(const ifa_paged_args *a, const IfaPlan &p) {
    Launch L;
    memset(&L, 0, sizeof L);
    L.q = a->query;
    L.k = a->key_cache;
    L.v = a->value_cache;
    L.out = a->attention_out;
    const int64_t bs = a->block_size, D = p.D, Nkv = p.Nkv;
    L.block_table = a->block_table;
    L.max_blocks = (int)a->max_blocks_per_seq;
    L.block_size = (int)bs;
    L.num_blocks = (int)a->num_blocks;
    L.blk_stride = Nkv * bs * D;
    if (a->kv_cache_layout == 0) {   // (blocknum, KV_N, blocksize, D)
        L.head_stride = bs * D;
        L.row_stride = D;
    } else {                         // (blocknum, blocksize, KV_N*D)
        L.head_stride = D;
        L.row_stride = Nkv * D;
    }
    if (a->atten_mask) {
        L.mask = reinterpret_cast<const uint8_t *>(a->atten_mask);
        L.mask_sB = a->mask_batch == 1 ? 0 : a->mask_heads * a->mask_seq;
        L.mask_sH = a->mask_heads == 1 ? 0 : a->mask_seq;
        L.mask_mode = a->mask_heads == 1 ? 1 : 2;
    }
    if (a->pse_shift) {
        L.pse = a->pse_shift;
        L.pse_sB = a->pse_batch == 1 ? 0 : a->num_heads * a->pse_seq;
        L.pse_sH = a->pse_seq;
    }
    L.aqs = a->antiquant_scale;
    L.aqo = a->antiquant_offset;
    L.aq_mode = a->dtype_kv == IFA_DT_I8 ? a->antiquant_mode : 0;
    L.q_bf16 = a->dtype_q == IFA_DT_BF16;
    L.scale = a->scale_value;
    L.out_i8 = a->dtype_out == IFA_DT_I8;
    L.quant = paged_quant(a);
    L.ev_begin = reinterpret_cast<hipEvent_t>(a->profile_event_begin);
    L.ev_end = reinterpret_cast<hipEvent_t>(a->profile_event_end);
    return L;
}

// ----------------------------------------------------------------- built-in scratch

// Device memory of ifa_decode_noalloc: the split kernel's partial states
// (sums, maxima, normalisers) for callers that cannot allocate a workspace.
// Every GPU the library runs on holds its own copy for the life of the
// process.  In host code `scratch` names a host-side stand-in, never the
// device address: kernels and copies get the address hipGetSymbolAddress
// returns for the current device, taken once per device.
constexpr size_t kScratchBytes = (size_t)IFA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void *g_scratch[64];   // per-device address of `scratch`, null until first use

int scratch_address(void **out) {
    int dev = 0;
    if (current_device(&dev) != IFA_OK || dev < 0 || dev >= 64) return IFA_ERR_RUNTIME;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return IFA_ERR_RUNTIME;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return IFA_OK;
}

}  // namespace

extern "C" {

int ifa_abi_version(void) { return kAbiVersion; }

const char *ifa_status_string(int status) {
    switch (status) {
    case IFA_OK: return "IFA_OK";
    case IFA_ERR_PARAM_NULLPTR: return "IFA_ERR_PARAM_NULLPTR: a mandatory pointer is NULL";
    case IFA_ERR_PARAM_INVALID: return "IFA_ERR_PARAM_INVALID: unsupported dtype, layout, shape or constraint";
    case IFA_ERR_RUNTIME: return "IFA_ERR_RUNTIME: a HIP call or kernel launch failed";
    }
    return "unknown status";
}

int ifa_decode_workspace_size(const ifa_decode_args *a, size_t *bytes) {
    if (!bytes) return IFA_ERR_PARAM_NULLPTR;
    IfaPlan p;
    IfaCommon c;
    int rc = plan_dense(a, p, c);
    if (rc) return rc;
    rc = finish_plan(p, a->split_tokens);
    if (rc) return rc;
    *bytes = p.workspace;
    return IFA_OK;
}

int ifa_decode(const ifa_decode_args *a, void *ws, size_t ws_bytes, ifa_stream_t stream) {
    IfaPlan p;
    IfaCommon c;
    int rc = plan_dense(a, p, c);
    if (rc) return rc;
    rc = finish_plan(p, a->split_tokens);
    if (rc) return rc;
    return run(p, dense_launch(a, p, c), ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

int ifa_decode_noalloc(const ifa_decode_args *a, ifa_stream_t stream) {
    IfaPlan p;
    IfaCommon c;
    int rc = plan_dense(a, p, c);
    if (rc) return rc;
    rc = finish_plan(p, a->split_tokens);
    if (rc) return rc;
    if (p.workspace > kScratchBytes) {
        fprintf(stderr, "ifa_decode_noalloc: the call needs %zu bytes of scratch, more than the built-in %zu\n",
                p.workspace, kScratchBytes);
        return IFA_ERR_PARAM_INVALID;
    }
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    return run(p, dense_launch(a, p, c), ws, kScratchBytes, reinterpret_cast<hipStream_t>(stream));
}

int ifa_decode_paged_workspace_size(const ifa_paged_args *a, size_t *bytes) {
    if (!bytes) return IFA_ERR_PARAM_NULLPTR;
    IfaPlan p;
    IfaCommon c;
    int rc = plan_paged(a, p, c);
    if (rc) return rc;
    rc = finish_plan(p, a->split_tokens);
    if (rc) return rc;
    *bytes = p.workspace;
    return IFA_OK;
}

int ifa_decode_paged(const ifa_paged_args *a, void *ws, size_t ws_bytes, ifa_stream_t stream) {
    IfaPlan p;
    IfaCommon c;
    int rc = plan_paged(a, p, c);
    if (rc) return rc;
    rc = finish_plan(p, a->split_tokens);
    if (rc) return rc;
    return run(p, paged_launch(a, p), ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

int sfa_decode_mla_workspace_size(const sfa_mla_args *a, size_t *bytes) {
    return ifa::sfa_workspace_size(a, bytes);
}

int sfa_decode_mla_plan(const sfa_mla_args *a, sfa_mla_plan *plan) { return ifa::sfa_plan_info(a, plan); }

int sfa_decode_mla(const sfa_mla_args *a, void *ws, size_t ws_bytes, ifa_stream_t stream) {
    return ifa::sfa_run(a, ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
