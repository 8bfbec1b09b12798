// Host side of the sparse MLA-absorb decode path (SparseFlashAttention README:
// parameter table and constraints).
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <stddef.h>

#include <algorithm>

#include "sfa.h"

namespace ifa {

namespace {

// The call's shape once validated: query rows, layouts and the breadth fields
// (zero when the caller's struct predates them).
struct SfaShape {
    int layout_q = 0, layout_kv = 0, sbs_shift = 0;
    int64_t R = 0, q_tokens = 0, kv_tokens = 0, kv_seq = 0, kv_rows = 0;
    float *lse_max = nullptr, *lse_sum = nullptr;   // return_softmax_lse outputs
};

int validate(const sfa_mla_args *a, SfaShape &sh) {
    if (!a) return IFA_ERR_PARAM_NULLPTR;
    if (a->struct_size < offsetof(sfa_mla_args, q_tokens)) return IFA_ERR_PARAM_INVALID;
    const bool breadth = a->struct_size >= offsetof(sfa_mla_args, softmax_max_out);
    const bool lse_fields = a->struct_size >= sizeof(sfa_mla_args);
    sh.q_tokens = breadth ? a->q_tokens : 0;
    sh.kv_tokens = breadth ? a->kv_tokens : 0;
    sh.kv_seq = breadth ? a->kv_seq : 0;
    if (!a->layout_query || !strcmp(a->layout_query, "BSND")) sh.layout_q = 0;
    else if (!strcmp(a->layout_query, "TND")) sh.layout_q = 1;
    else return IFA_ERR_PARAM_INVALID;
    if (!a->layout_kv || !strcmp(a->layout_kv, "PA_BSND")) sh.layout_kv = 0;
    else if (!strcmp(a->layout_kv, "BSND")) sh.layout_kv = 1;
    else if (!strcmp(a->layout_kv, "TND")) sh.layout_kv = 2;
    else return IFA_ERR_PARAM_INVALID;
    if (!a->query || !a->query_rope || !a->key || !a->key_rope || !a->value || !a->sparse_indices ||
        !a->attention_out)
        return IFA_ERR_PARAM_NULLPTR;
    if (sh.layout_kv == 0 && !a->block_table) return IFA_ERR_PARAM_NULLPTR;
    // README: the kv lengths are required for TND and PA_BSND caches, the
    // query lengths (prefix sums) for TND queries
    if (sh.layout_kv != 1 && !a->actual_seq_lengths_kv) return IFA_ERR_PARAM_NULLPTR;
    if (sh.layout_q == 1 && !a->actual_seq_lengths_query) return IFA_ERR_PARAM_NULLPTR;
    if (a->dtype != IFA_DT_F16 && a->dtype != IFA_DT_BF16) return IFA_ERR_PARAM_INVALID;
    if (a->batch < 1 || a->batch > 65536) return IFA_ERR_PARAM_INVALID;
    if (sh.layout_q == 0) {
        if (a->q_seq < 1 || a->q_seq > 65536) return IFA_ERR_PARAM_INVALID;
        sh.R = a->batch * a->q_seq;
    } else {
        if (sh.q_tokens < 1) return IFA_ERR_PARAM_INVALID;
        sh.R = sh.q_tokens;
    }
    if (sh.R > (1 << 24)) return IFA_ERR_PARAM_INVALID;
    if (a->kv_heads != 1) return IFA_ERR_PARAM_INVALID;                       // KV_N only 1
    if (a->head_dim != 512 || a->rope_dim != 64) return IFA_ERR_PARAM_INVALID; // Q_D = KV_D = 512, Dr = 64
    if (a->q_heads < 1 || a->q_heads > 128) return IFA_ERR_PARAM_INVALID;
    if (a->sparse_size < 1 || a->sparse_size > (1 << 24)) return IFA_ERR_PARAM_INVALID;
    if (sh.layout_kv == 0) {
        if (a->block_size < 16 || a->block_size > 1024 || a->block_size % 16) return IFA_ERR_PARAM_INVALID;
        if (a->num_blocks < 1 || a->num_blocks * a->block_size > INT32_MAX) return IFA_ERR_PARAM_INVALID;
        if (a->max_blocks < 1 || a->max_blocks * a->block_size > INT32_MAX) return IFA_ERR_PARAM_INVALID;
        sh.kv_rows = a->num_blocks * a->block_size;
    } else if (sh.layout_kv == 1) {
        if (sh.kv_seq < 1 || a->batch * sh.kv_seq > INT32_MAX) return IFA_ERR_PARAM_INVALID;
        sh.kv_rows = a->batch * sh.kv_seq;
    } else {
        if (sh.kv_tokens < 1 || sh.kv_tokens > INT32_MAX) return IFA_ERR_PARAM_INVALID;
        sh.kv_rows = sh.kv_tokens;
    }
    // README: sparse_block_size a power of two in [1, 128], dividing block_size for a paged cache
    const int64_t sbs = a->sparse_block_size;
    if (sbs < 1 || sbs > 128 || (sbs & (sbs - 1))) return IFA_ERR_PARAM_INVALID;
    if (sh.layout_kv == 0 && a->block_size % sbs) return IFA_ERR_PARAM_INVALID;
    while ((1 << sh.sbs_shift) < sbs) sh.sbs_shift++;
    if (a->sparse_mode != 0 && a->sparse_mode != 3) return IFA_ERR_PARAM_INVALID;
    if (a->attention_mode != 2) return IFA_ERR_PARAM_INVALID;
    if (!std::isfinite(a->scale_value)) return IFA_ERR_PARAM_INVALID;
    if (a->split_hint < 0 || a->split_hint > 64) return IFA_ERR_PARAM_INVALID;
    if (lse_fields) {
        if (a->return_softmax_lse == 1) {
            // README: softmax_max / softmax_sum are returned only when layout_kv is not PA_BSND
            if (sh.layout_kv == 0) return IFA_ERR_PARAM_INVALID;
            if (!a->softmax_max_out || !a->softmax_sum_out) return IFA_ERR_PARAM_NULLPTR;
            sh.lse_max = a->softmax_max_out;
            sh.lse_sum = a->softmax_sum_out;
        } else if (a->return_softmax_lse != 0 || a->softmax_max_out || a->softmax_sum_out) {
            return IFA_ERR_PARAM_INVALID;
        }
    }
    return IFA_OK;
}

// Chunk outputs are kept in the input dtype (2 bytes), 256-byte aligned.
size_t part_o_bytes(size_t rows) { return (rows * 512 * 2 + 255) / 256 * 256; }

struct SfaPlan {
    int n_hb = 0, n_sc = 0, chunk = 0, grid = 0;
    bool wide = false;
    size_t workspace = 0;
};

int device_cus(int *cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return IFA_ERR_RUNTIME;
    return IFA_OK;
}

// Chunks of each query row's index list for `per` workgroups per chunk index
// (query rows x head blocks): the forced count, else about one workgroup per
// compute unit.  A chunk gathers at most kSfaChunkMax rows (entries x
// sparse_block_size) and a multiple of the 32-row tile when the list is long
// enough.  Fills n_sc, chunk and grid (workgroups, rounded to whole XCD
// rounds of 8 per head block).
int split_chunks(const sfa_mla_args *a, const SfaShape &sh, int64_t per, int cus, SfaPlan &p) {
    int64_t n_sc = a->split_hint > 0 ? a->split_hint : std::max<int64_t>(1, (cus + per / 2) / per);
    const int64_t gran = std::max(1, 32 >> sh.sbs_shift), cap = kSfaChunkMax >> sh.sbs_shift;
    int64_t chunk = (a->sparse_size + n_sc - 1) / n_sc;
    chunk = (chunk + gran - 1) / gran * gran;
    if (chunk > cap) chunk = cap;
    n_sc = (a->sparse_size + chunk - 1) / chunk;
    if (n_sc > (1 << 20)) return IFA_ERR_PARAM_INVALID;
    const int64_t grid = (sh.R * n_sc + 7) / 8 * 8 * p.n_hb;
    if (grid > INT32_MAX) return IFA_ERR_PARAM_INVALID;
    p.n_sc = (int)n_sc;
    p.chunk = (int)chunk;
    p.grid = (int)grid;
    return IFA_OK;
}

// Work split: workgroups of 64 heads x one chunk of one query row's index
// list (sfa_kernel), one workgroup per compute unit at most (each takes
// nearly all of a CU's LDS).  With more than 64 heads, when that grid would
// not fit on the CUs at once, one workgroup takes every head of a chunk
// (sfa_wide_kernel): half the workgroups, so the call runs in one round.
// The CU count is read only when it decides something (no forced chunk
// count, or more than 64 heads).
int plan(const sfa_mla_args *a, const SfaShape &sh, SfaPlan &p) {
    int cus = 0;
    if (a->split_hint == 0 || a->q_heads > 64) {
        const int rc = device_cus(&cus);
        if (rc) return rc;
    }
    p.wide = false;
    p.n_hb = (int)((a->q_heads + 63) / 64);
    int rc = split_chunks(a, sh, sh.R * p.n_hb, cus, p);
    if (rc) return rc;
    if (a->q_heads > 64 && p.grid > cus) {
        p.wide = true;
        p.n_hb = 1;
        rc = split_chunks(a, sh, sh.R, cus, p);
        if (rc) return rc;
    }
    p.workspace = 0;
    if (p.n_sc > 1) {
        const size_t rows = (size_t)sh.R * p.n_sc * a->q_heads;
        p.workspace = part_o_bytes(rows) + (rows * 2 * sizeof(float) + 255) / 256 * 256;
    }
    return IFA_OK;
}

uint32_t magic_for(uint32_t d, int *shift) {
    int l = 0;
    while (((uint64_t)1 << l) < d) l++;
    *shift = l;
    return (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
}

}  // namespace

int sfa_workspace_size(const sfa_mla_args *a, size_t *bytes) {
    if (!bytes) return IFA_ERR_PARAM_NULLPTR;
    SfaShape sh;
    int rc = validate(a, sh);
    if (rc) return rc;
    SfaPlan p;
    rc = plan(a, sh, p);
    if (rc) return rc;
    *bytes = p.workspace;
    return IFA_OK;
}

int sfa_plan_info(const sfa_mla_args *a, sfa_mla_plan *out) {
    if (!out) return IFA_ERR_PARAM_NULLPTR;
    SfaShape sh;
    int rc = validate(a, sh);
    if (rc) return rc;
    SfaPlan p;
    rc = plan(a, sh, p);
    if (rc) return rc;
    out->chunks = p.n_sc;
    out->chunk_entries = p.chunk;
    out->workgroups = p.grid;
    out->all_heads = p.wide ? 1 : 0;
    return IFA_OK;
}

int sfa_run(const sfa_mla_args *a, void *ws, size_t ws_bytes, hipStream_t stream) {
    SfaShape sh;
    int rc = validate(a, sh);
    if (rc) return rc;
    SfaPlan pl;
    rc = plan(a, sh, pl);
    if (rc) return rc;
    if (pl.workspace && !ws) return IFA_ERR_PARAM_NULLPTR;
    if (ws_bytes < pl.workspace) return IFA_ERR_PARAM_INVALID;
    SfaParams p;
    memset(&p, 0, sizeof p);
    p.q = a->query;
    p.q_rope = a->query_rope;
    p.key = a->key;
    p.key_rope = a->key_rope;
    p.value = a->value;
    p.idx = a->sparse_indices;
    p.bt = a->block_table;
    p.lkv = a->actual_seq_lengths_kv;
    p.lq = a->actual_seq_lengths_query;
    p.out = a->attention_out;
    p.lse_max = sh.lse_max;
    p.lse_sum = sh.lse_sum;
    const size_t rows = (size_t)sh.R * pl.n_sc * a->q_heads;
    p.part_o = ws;
    p.part_ml = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + part_o_bytes(rows));
    p.sparse_size = a->sparse_size;
    p.kv_seq = sh.kv_seq;
    p.kv_rows = sh.kv_rows;
    p.B = (int)a->batch;
    p.R = (int)sh.R;
    p.QS = sh.layout_q == 0 ? (int)a->q_seq : 1;
    p.QN = (int)a->q_heads;
    p.layout_q = sh.layout_q;
    p.layout_kv = sh.layout_kv;
    p.sparse_mode = (int)a->sparse_mode;
    p.sbs_shift = sh.sbs_shift;
    if (sh.layout_kv == 0) {
        p.bs = (int)a->block_size;
        p.max_blocks = (int)a->max_blocks;
        p.num_blocks = (int)a->num_blocks;
        p.bs_magic = magic_for((uint32_t)a->block_size, &p.bs_shift);
    }
    p.n_hb = pl.n_hb;
    p.wide = pl.wide;
    p.n_sc = pl.n_sc;
    p.chunk = pl.chunk;
    p.direct = pl.n_sc == 1;
    p.score_mul = (float)((double)a->scale_value * 1.4426950408889634);
    if (sfa_launch(p, a->dtype == IFA_DT_BF16, pl.grid, stream, reinterpret_cast<hipEvent_t>(a->profile_event_begin),
                   reinterpret_cast<hipEvent_t>(a->profile_event_end)) != hipSuccess)
        return IFA_ERR_RUNTIME;
    return IFA_OK;
}

}  // namespace ifa
