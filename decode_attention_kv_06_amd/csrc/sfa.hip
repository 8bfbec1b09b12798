// Host side of the sparse MLA-absorb decode path (SparseFlashAttention README:
// parameter table and constraints).
#include <math.h>
#include <string.h>

#include "sfa.h"

namespace ifa {

namespace {

int validate(const sfa_mla_args *a) {
    if (!a) return IFA_ERR_PARAM_NULLPTR;
    if (a->struct_size < sizeof(sfa_mla_args)) return IFA_ERR_PARAM_INVALID;
    if (!a->query || !a->query_rope || !a->key || !a->key_rope || !a->value || !a->sparse_indices ||
        !a->block_table || !a->actual_seq_lengths_kv || !a->attention_out)
        return IFA_ERR_PARAM_NULLPTR;
    if (a->dtype != IFA_DT_F16 && a->dtype != IFA_DT_BF16) return IFA_ERR_PARAM_INVALID;
    if (a->layout_query && strcmp(a->layout_query, "BSND")) return IFA_ERR_PARAM_INVALID;
    if (a->layout_kv && strcmp(a->layout_kv, "PA_BSND")) return IFA_ERR_PARAM_INVALID;
    if (a->batch < 1 || a->batch > 65536) return IFA_ERR_PARAM_INVALID;
    if (a->q_seq != 1) return IFA_ERR_PARAM_INVALID;
    if (a->kv_heads != 1) return IFA_ERR_PARAM_INVALID;                       // KV_N only 1
    if (a->head_dim != 512 || a->rope_dim != 64) return IFA_ERR_PARAM_INVALID; // Q_D = KV_D = 512, Dr = 64
    if (a->q_heads < 1 || a->q_heads > 128) return IFA_ERR_PARAM_INVALID;
    if (a->sparse_size < 1 || a->sparse_size > (1 << 24)) return IFA_ERR_PARAM_INVALID;
    if (a->block_size < 16 || a->block_size > 1024 || a->block_size % 16) return IFA_ERR_PARAM_INVALID;
    if (a->num_blocks < 1 || a->num_blocks > (int64_t)1 << 31) return IFA_ERR_PARAM_INVALID;
    if (a->max_blocks < 1 || a->max_blocks * a->block_size > ((int64_t)1 << 31) - 1) return IFA_ERR_PARAM_INVALID;
    if (a->sparse_block_size != 1) return IFA_ERR_PARAM_INVALID;
    if (a->sparse_mode != 0 && a->sparse_mode != 3) return IFA_ERR_PARAM_INVALID;
    if (a->attention_mode != 2) return IFA_ERR_PARAM_INVALID;
    if (!std::isfinite(a->scale_value)) return IFA_ERR_PARAM_INVALID;
    if (a->split_hint < 0 || a->split_hint > 64) return IFA_ERR_PARAM_INVALID;
    return IFA_OK;
}

}  // namespace

int sfa_workspace_size(const sfa_mla_args *a, size_t *bytes) {
    if (!bytes) return IFA_ERR_PARAM_NULLPTR;
    int rc = validate(a);
    if (rc) return rc;
    *bytes = 0;
    return IFA_OK;
}

int sfa_run(const sfa_mla_args *a, void *ws, size_t ws_bytes, hipStream_t stream) {
    (void)ws;
    (void)ws_bytes;
    (void)stream;
    int rc = validate(a);
    if (rc) return rc;
    return IFA_ERR_PARAM_INVALID;   // kernel not built yet
}

}  // namespace ifa
