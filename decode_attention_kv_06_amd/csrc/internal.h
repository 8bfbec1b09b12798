// Internal kernel interface of libifadecode (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ifa {

// Batches handled by one launch; the per-batch window table travels in the
// kernel argument block, so it has a fixed capacity.
constexpr int kSliceBatches = 128;
// Rows of a row-mode call (listed in the kernel arguments, see SplitParams::row_win).
constexpr int kRowTab = 512;
constexpr int kWavesPerBlock = 4;

enum KvKind { KV_F16 = 0, KV_BF16 = 1, KV_I8 = 2 };

// Optional score terms of a split kernel variant: none, attenMask, or
// pseShift (with attenMask, when present, checked at run time).
enum SplitExtra { EX_NONE = 0, EX_MASK = 1, EX_PSE = 2 };

// Arguments of the split-KV decode kernel.
//
// Work is balanced in cost units: the rows (b, kv head j, head group hg),
// each of the batch's window length, are laid end to end, every row followed
// by seg_cost units that stand for the cost of starting a row, and wave w
// takes the positions whose costs fall in [w*piece, (w+1)*piece), cut into
// segments at row boundaries (a wave that meets a row start gets that many
// positions fewer).  Each segment writes one partial softmax state (G heads)
// to slot sbase[b] + (j*n_hg + hg)*maxseg[b] + (w - first piece of the row);
// the combine kernel recomputes the same slots from the same tables.
// Small problems (every row a few tiles long) run in row mode instead:
// workgroup w takes row w, each of its waves a quarter of the window; the
// waves merge their states in LDS and write the output, so one launch does
// the call.
struct SplitParams {
    const void *q;          // [B, N, D] (any query layout, S = 1)
    const void *k;          // cache base
    const void *v;
    float *part_acc;        // [slots][G][D]  unnormalised sum p*v
    float *part_ml;         // [slots][G][2]  running max (log2 domain), sum p
    const uint8_t *mask;    // nullptr when absent
    const void *pse;        // pseShift [pse_batch, N, 1, pse_seq], query dtype; nullptr when absent
    const int32_t *block_table;
    const void *k_scale;    // int8 only: antiquant scale, q dtype
    const void *const *k_list;   // per-batch caches: device array of B device pointers, or nullptr
    const void *const *v_list;
    void *out;              // row mode: the output [B, N, D] (query dtype), written in place
    int64_t sB, sN, sS;     // dense element strides of (b, j, s)
    int64_t blk_stride, head_stride, row_stride;   // paged element strides
    int64_t mask_sB, mask_sH;                      // mask strides (0 = broadcast)
    int64_t pse_sB, pse_sH;                        // pseShift strides (pse_sB 0 = broadcast)
    int64_t total;          // positions over all rows of the slice
    int64_t piece;          // cost units per wave
    int32_t seg_cost;       // cost units charged per row start (0: a piece is `piece` positions)
    int32_t n_pieces;
    int32_t N, Nkv, g, n_hg;
    int32_t max_blocks, block_size, num_blocks;
    uint32_t bs_magic;      // s / block_size via a round-up multiplier and shift
    int32_t bs_shift;
    int32_t mask_mode;      // 0 none, 1 shared by the heads, 2 per head
    int32_t aq_mode;        // int8: 1 per-tensor, 2 per-channel
    int32_t q_bf16;         // int8 kernels: query dtype is bf16
    int32_t list_bnsd;      // per-batch BNSD caches: the head stride is list_seq[b] * sS
    int32_t Dr;             // the call's head dim (<= the compiled D; lanes past it re-read the last
                            // 16-byte chunk of a row and carry a zero query)
    int32_t row_mode;       // one workgroup per (b, j, hg) row, merged, normalised and written out by it
                            // (16-bit caches and outputs); no partial states, no combine
    float score_mul;        // scale * log2(e)
    int32_t nb;             // batches in this slice
    int32_t b0;             // first batch of the slice
    int64_t row_win[kRowTab];         // row mode, row r (= workgroup r): (window length << 32) | window
                                      // start; its address needs no other argument, so the kernel reads
                                      // it in its first round of argument loads
    int64_t pre[kSliceBatches + 1];   // first flattened position of each batch's rows
    int32_t lo[kSliceBatches];        // window start of each batch
    int32_t len[kSliceBatches];       // window length of each batch
    int32_t sbase[kSliceBatches];     // first partial slot of each batch
    int32_t maxseg[kSliceBatches];    // slots reserved per row of each batch
    int32_t list_seq[kSliceBatches];  // per-batch caches: positions of each batch's tensor
};

// Arguments of the split-combine kernel: one wave per (b, h) row.
struct CombineParams {
    const float *part_acc;
    const float *part_ml;
    void *out;              // [B, N, D], query dtype
    const void *v_scale;    // int8: antiquant (scale, offset) of V, q dtype
    const void *v_offset;
    int64_t piece;
    int32_t seg_cost;
    int32_t N, Nkv, g, G, n_hg, D;   // D: the compiled head dim (partial-state row length)
    int32_t Dr;                      // the call's head dim (output row length)
    int32_t out_bf16;
    int32_t aq_mode;
    int32_t out_i8;         // int8 output: quantise with (q_scale2, q_offset2)
    int32_t q2_bf16;        // quant parameters are bf16 (else fp32)
    int32_t q2_per_channel; // one parameter per output channel h * D + d (else one for all)
    const void *q_scale2, *q_offset2;
    int32_t nb, b0;
    int64_t pre[kSliceBatches + 1];
    int32_t len[kSliceBatches];
    int32_t sbase[kSliceBatches];
    int32_t maxseg[kSliceBatches];
};

// Cost coordinate of the first position of row rj of slice batch bl (the
// rows before it each add seg_cost to their positions).
template <class PP>
__device__ __forceinline__ int64_t row_cost(const PP &P, int bl, int rj) {
    return P.pre[bl] + (int64_t)rj * P.len[bl] + (int64_t)P.seg_cost * ((int64_t)P.Nkv * P.n_hg * bl + rj);
}

hipError_t launch_split(const SplitParams &p, int kv, int D, int G, bool paged, int extra, hipStream_t s);
hipError_t launch_combine(const CombineParams &p, hipStream_t s);

// Resident waves of the split kernel for this shape (occupancy query).
int split_resident_waves(int kv, int D, int G, bool paged, int extra);

// Per-KV-dtype kernel sets (one translation unit each).
template <int KV>
hipError_t launch_split_kv(const SplitParams &p, int D, int G, bool paged, int extra, hipStream_t s);
template <int KV>
const void *split_kernel_ptr(int D, int G, bool paged, int extra);

}  // namespace ifa
