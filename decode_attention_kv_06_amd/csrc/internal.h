// Internal kernel interface of libifadecode (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ifa {

// Batches handled by one launch; the per-batch window table travels in the
// kernel argument block, so it has a fixed capacity.
constexpr int kSliceBatches = 128;
constexpr int kWavesPerBlock = 4;

enum KvKind { KV_F16 = 0, KV_BF16 = 1, KV_I8 = 2 };

// Arguments of the split-KV decode kernel.  One wave processes one work item
// (b, kv head j, head group hg, chunk c): the KV positions
// [lo_b + c*chunk, min(hi_b, lo_b + (c+1)*chunk)) for query heads
// j*g + hg*G .. j*g + hg*G + G-1.
struct SplitParams {
    const void *q;          // [B, N, D] (any query layout, S = 1)
    const void *k;          // cache base
    const void *v;
    float *part_acc;        // [chunks][N][D]  unnormalised sum p*v
    float *part_ml;         // [chunks][N][2]  running max (log2 domain), sum p
    const uint8_t *mask;    // nullptr when absent
    const int32_t *block_table;
    const void *k_scale;    // int8 only: antiquant scale, q dtype
    int64_t sB, sN, sS;     // dense element strides of (b, j, s)
    int64_t blk_stride, head_stride, row_stride;   // paged element strides
    int64_t mask_sB, mask_sH;                      // mask strides (0 = broadcast)
    int32_t N, Nkv, g, n_hg;
    int32_t max_blocks, block_size, num_blocks;
    uint32_t bs_magic;      // s / block_size == (umulhi(s, magic) + s) >> bs_shift (or >> only)
    int32_t bs_shift, bs_pow2;
    int32_t mask_mode;      // 0 none, 1 shared by the heads, 2 per head
    int32_t aq_mode;        // int8: 1 per-tensor, 2 per-channel
    int32_t q_bf16;         // int8 kernels: query dtype is bf16
    float score_mul;        // scale * log2(e)
    int32_t chunk;          // positions per work item
    int32_t nb;             // batches in this slice
    int32_t b0;             // first batch of the slice
    int32_t n_items;
    int32_t lo[kSliceBatches];
    int32_t hi[kSliceBatches];
    int32_t cum[kSliceBatches + 1];   // chunk prefix sums
};

// Arguments of the split-combine kernel: one wave per (b, h) row.
struct CombineParams {
    const float *part_acc;
    const float *part_ml;
    void *out;              // [B, N, D], query dtype
    const void *v_scale;    // int8: antiquant (scale, offset) of V, q dtype
    const void *v_offset;
    int32_t N, Nkv, g, D;
    int32_t out_bf16;
    int32_t aq_mode;
    int32_t nb, b0;
    int32_t cum[kSliceBatches + 1];
};

hipError_t launch_split(const SplitParams &p, int kv, int D, int G, bool paged, hipStream_t s);
hipError_t launch_combine(const CombineParams &p, hipStream_t s);

// Resident waves of the split kernel for this shape (occupancy query).
int split_resident_waves(int kv, int D, int G, bool paged);

// Positions one wave handles per tile (the planner keeps chunks a multiple of it).
int split_tile_tokens(int kv, int D, int G);

}  // namespace ifa
