// Internal interface of the sparse (MLA-absorb) decode path.
#pragma once

#include "ifa_decode.h"
#include "internal.h"

namespace ifa {

// Sparse entries handled by one workgroup at most (the kernel's LDS row table).
constexpr int kSfaChunkMax = 512;

// Arguments of the gather + MFMA kernel and its chunk combine.
struct SfaParams {
    const void *q, *q_rope, *key, *key_rope, *value;
    const int32_t *idx;       // [B, sparse_size]
    const int32_t *bt;        // [B, max_blocks]
    const int32_t *lkv;       // [B]
    const int32_t *lq;        // [B] or nullptr
    void *out;                // [B, QN, 512]
    void *part_o;             // [B, n_sc, QN, 512], input dtype: each chunk's output normalised by its own sum
    float *part_ml;           // [B, n_sc, QN, 2]: the chunk's running max (log2 domain) and sum
    int64_t sparse_size;
    int32_t B, QN, bs, max_blocks, num_blocks;
    uint32_t bs_magic;
    int32_t bs_shift;
    int32_t n_hb;             // blocks of 64 heads
    int32_t n_sc;             // index chunks per batch
    int32_t chunk;            // indices per chunk (<= 1024)
    int32_t direct;           // one chunk per batch: write the normalised output directly
    float score_mul;          // scale * log2(e)
};

hipError_t sfa_launch(const SfaParams &p, bool bf16, int grid, hipStream_t s, hipEvent_t ev_begin, hipEvent_t ev_end);

int sfa_workspace_size(const sfa_mla_args *a, size_t *bytes);
int sfa_run(const sfa_mla_args *a, void *ws, size_t ws_bytes, hipStream_t stream);

}  // namespace ifa
