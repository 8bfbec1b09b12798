// Internal interface of the sparse (MLA-absorb) decode path.
#pragma once

#include "ifa_decode.h"
#include "internal.h"

namespace ifa {

// Cache rows gathered by one workgroup at most (the kernel's LDS row table).
constexpr int kSfaChunkMax = 512;

// Arguments of the gather + MFMA kernel and its chunk combine.
//
// Query rows: BSND queries give B * QS rows (row b * QS + s), TND queries
// their Q_T packed rows; q, q_rope, the index lists and the output all
// follow that row order.  Cache rows: a paged cache names rows through the
// block table; a BSND cache holds batch b at rows b * kv_seq + t, a TND
// cache at rows lkv[b - 1] + t.
struct SfaParams {
    const void *q, *q_rope, *key, *key_rope, *value;
    const int32_t *idx;       // [R, sparse_size]
    const int32_t *bt;        // [B, max_blocks] (paged cache only)
    const int32_t *lkv;       // [B]: counts, or prefix sums (TND cache); nullptr: kv_seq each (BSND cache)
    const int32_t *lq;        // [B]: counts (BSND query) or prefix sums (TND query); nullptr: QS each
    void *out;                // [R, QN, 512]
    void *part_o;             // [R, n_sc, QN, 512], input dtype: each chunk's output normalised by its own sum
    float *part_ml;           // [R, n_sc, QN, 2]: the chunk's score max (log2 domain) and its sum
                              // of exp2(score - max)
    float *lse_max, *lse_sum; // [R, QN] softmax_max / softmax_sum (natural log domain), or nullptr
    int64_t sparse_size;
    int64_t kv_seq;           // BSND cache: positions per batch
    int64_t kv_rows;          // rows of the key tensor (bounds every cache row the kernel reads)
    int32_t B, R, QS, QN, bs, max_blocks, num_blocks;
    int32_t layout_q;         // 0 BSND, 1 TND
    int32_t layout_kv;        // 0 PA_BSND, 1 BSND, 2 TND
    int32_t sparse_mode;      // 0 all, 3 rightDownCausal
    int32_t sbs_shift;        // log2 sparse_block_size
    uint32_t bs_magic;
    int32_t bs_shift;
    int32_t n_hb;             // blocks of 64 heads (1 with `wide`)
    int32_t wide;             // more than 64 heads: sfa_wide_kernel, one workgroup per chunk for every head
    int32_t n_sc;             // index chunks per query row
    int32_t chunk;            // index entries per chunk (chunk << sbs_shift <= kSfaChunkMax rows)
    int32_t direct;           // one chunk per row: write the normalised output directly
    float score_mul;          // scale * log2(e)
};

hipError_t sfa_launch(const SfaParams &p, bool bf16, int grid, hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end);

int sfa_workspace_size(const sfa_mla_args *a, size_t *bytes);
int sfa_plan_info(const sfa_mla_args *a, sfa_mla_plan *out);
int sfa_run(const sfa_mla_args *a, void *ws, size_t ws_bytes, hipStream_t stream);

}  // namespace ifa
