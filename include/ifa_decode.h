/*
 * ifa_decode.h — C ABI of the MI355X (gfx950) decode-attention library.
 *
 * Three operations, each with the two-phase calling convention of the
 * aclnnIncreFlashAttentionV2 page ("Function Prototype"): a workspace-size
 * query that validates the arguments, then a run call that enqueues the work
 * on a HIP stream.
 *
 *   ifa_decode        IncreFlashAttention over a dense padded KV cache
 *   ifa_decode_paged  IncreFlashAttention over a paged KV cache (block table)
 *   sfa_decode_mla    SparseFlashAttention, MLA-absorb mode (paged, BSND or TND cache)
 *
 * What is computed (IncreFlashAttention README "Formula"; V2 page "Formula"):
 *     attentionOut = softmax(scaleValue * query . key^T  [masked]) . value
 * with the query S axis fixed to 1, per batch over the KV positions the
 * README's constraints define (actual lengths, left padding, page attention),
 * and for SFA (SparseFlashAttention README "Formula") over the cache rows
 * named by sparse_indices, with the rope parts added to the scores.
 *
 * Conventions where the pages leave a choice open:
 *   - attenMask: a nonzero byte EXCLUDES the position (the V2 page's worked
 *     example passes an all-zero mask in an ordinary call);
 *   - GQA: query head h reads KV head h / (num_heads / num_key_value_heads);
 *   - an empty attention set (length 0, every position masked, no valid
 *     sparse index) gives an all-zero output row, like the left-padding rule;
 *   - antiquant: dequantised = (x + offset) * scale; index 0 of the leading
 *     axis of scale/offset is K, index 1 is V;
 *   - output rounding: fp32 result rounded to nearest-even into fp16/bf16.
 *
 * Ownership.  Every tensor is caller-owned device memory (pointers from
 * hipMalloc or a framework allocator).  The library allocates and frees
 * nothing, and keeps no pointer after a call returns.  Host arrays
 * (actual_seq_lengths, kv_padding_size) are read during the call only.  The
 * workspace is caller-allocated with at least the size the matching
 * *_workspace_size call returned for the same arguments; it must not be in
 * use by another call that may run concurrently.  attention_out and the
 * workspace must not alias any input; for SFA, value may alias key.
 *
 * Execution.  The run calls enqueue kernels on `stream` and return without
 * waiting (the V2 page's example synchronises the stream after the call).
 * No call synchronises the device or allocates, so a call can be captured
 * into a HIP graph.  Results are deterministic: the same inputs on the same
 * device give the same bytes (V2 page "Constraints > Deterministic computation").
 *
 * Errors (V2 page "Return Value"):
 *   IFA_ERR_PARAM_NULLPTR (161001)  a mandatory pointer is NULL
 *   IFA_ERR_PARAM_INVALID (161002)  a dtype, layout, shape, constraint or the
 *                                   workspace size is not supported
 *   IFA_ERR_RUNTIME       (361001)  a HIP call or kernel launch failed
 * Every check runs before anything is enqueued; on an error nothing is
 * launched and attention_out is untouched.
 */
#ifndef IFA_DECODE_H
#define IFA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t; NULL is the default stream. */
struct ihipStream_t;
typedef struct ihipStream_t *ifa_stream_t;

enum {
    IFA_OK = 0,
    IFA_ERR_PARAM_NULLPTR = 161001,
    IFA_ERR_PARAM_INVALID = 161002,
    IFA_ERR_RUNTIME = 361001
};

enum {
    IFA_DT_F16 = 1,  /* IEEE binary16 */
    IFA_DT_BF16 = 2, /* bfloat16 */
    IFA_DT_I8 = 3,   /* int8 (KV cache with antiquant; or mask) */
    IFA_DT_U8 = 4,   /* uint8 (mask) */
    IFA_DT_BOOL = 5, /* one byte per element, 0 or 1 (mask) */
    IFA_DT_F32 = 6   /* IEEE binary32 (output quantisation parameters) */
};

enum { IFA_ANTIQUANT_NONE = 0, IFA_ANTIQUANT_PER_TENSOR = 1, IFA_ANTIQUANT_PER_CHANNEL = 2 };

/*
 * Dense padded KV cache (IncreFlashAttention; V2 page parameter table).
 *
 * query / attention_out: (B,N,1,D) "BNSD", (B,1,N,D) "BSND" or (B,1,N*D)
 *   "BSH"; contiguous; dtype_q.
 * key / value: (B,N_kv,S,D) "BNSD", (B,S,N_kv,D) "BSND" or (B,S,N_kv*D)
 *   "BSH", the same layout as the query; contiguous; identical shapes.
 * actual_seq_lengths: host int64[batch], 0 <= L_b <= kv_seq_len, or NULL
 *   (every batch uses kv_seq_len).  Positions [0, L_b) are attended (right
 *   padding) unless kv_padding_size is given.
 * kv_padding_size: host int64[batch] or int64[1] (broadcast), or NULL.  With
 *   actual_seq_lengths present the window is [Smax - p - L_b, Smax - p),
 *   p = max(pad_b, 0); a window with start or end < 0 gives a zero row
 *   (README "Constraints > kv left padding").  Ignored without lengths.
 * atten_mask: device bytes (mask_batch, mask_heads, 1, mask_seq) with
 *   mask_batch in {1,B}, mask_heads in {1,N}, mask_seq >= every position
 *   attended; indexed by the physical cache position.  NULL for none.
 * antiquant_scale / antiquant_offset: device, dtype_q; per-tensor shape (2),
 *   per-channel (2,N_kv,1,D) (equivalently (2,N_kv,D) or (2,H)).  Required
 *   when dtype_kv is IFA_DT_I8, forbidden otherwise (README "Constraints >
 *   antiquantScale and antiquantOffset").
 * pse_shift: device, dtype_q, shape (pse_batch, N, 1, pse_seq) contiguous,
 *   pse_batch in {1,B} (1 = shared by every batch), pse_seq >= every position
 *   attended; NULL for none.  pse_shift[b][h][0][s] is added to the scaled
 *   score of query head h at cache position s, after scale_value and before
 *   the softmax, at the position coordinate the mask uses: the physical
 *   cache position here (IncreFlashAttention README "Formula" and
 *   "Constraints"; the placement after the scale is this library's reading).
 *   -inf excludes a position like a mask byte.  pse_batch and pse_seq are the
 *   two last fields of the struct; a struct_size that stops before them means
 *   no positional bias (pse_shift must then be NULL).
 * Envelope: 1 <= B <= 65536, 1 <= N <= 256, N % N_kv == 0,
 *   8 <= head_dim <= 512 with head_dim % 8 == 0 (the README bounds the head
 *   dim by 512; whole 16-byte row chunks are this library's requirement),
 *   dtype_out == dtype_q or IFA_DT_I8, dtype_kv == dtype_q or IFA_DT_I8.
 * Int8 output (dtype_out IFA_DT_I8; README "Constraints": quantScale2
 *   required, quantOffset2 optional, per-tensor or per-channel, fp32, or bf16
 *   with bf16 inputs): each output element o of head h, column d becomes
 *   clamp(round_half_even(o * s[c] + t[c]), -128, 127), c = 0 per-tensor or
 *   h * head_dim + d per-channel, o being the fp32 result before any
 *   rounding (the formula, the rounding and the saturation are this
 *   library's reading: the pages give none).  The quant fields are the last
 *   of each struct (ABI version 5) and must be NULL/0 for a float output.
 * key_list / value_list / kv_list_seq_len (all three, or none): the tensor
 *   lists of the V2 page ("Constraints", non-contiguous case): batch b reads
 *   its own key and value tensors, each of batch 1, kv_list_seq_len[b]
 *   positions and otherwise the shape of one batch of key/value in
 *   input_layout; key and value must then be NULL and kv_seq_len is not
 *   used.  The two pointer arrays live in device memory (caller-owned, read
 *   by the kernels); 1 <= batch <= 256 (V2 page); actual_seq_lengths, when
 *   given, must not exceed a batch's kv_list_seq_len; kv_padding_size must
 *   be NULL (left padding is defined on one padded buffer).  These three are
 *   the last fields of the struct (ABI version 4).
 * split_tokens: 0 lets the planner choose how many KV positions one work
 *   item covers; a positive multiple of 16 forces it (testing and tuning).
 * profile_event_begin / _end: NULL, or two hipEvent_t the call records on
 *   `stream` immediately before and after its split kernel, so a caller can
 *   time that kernel alone.  With more than 128 batches the split kernel runs
 *   once per 128-batch slice and the pair brackets all of them.
 */
typedef struct ifa_decode_args {
    uint32_t struct_size; /* sizeof(ifa_decode_args) */
    const void *query;
    const void *key;
    const void *value;
    void *attention_out;
    int32_t dtype_q, dtype_kv, dtype_out;
    const char *input_layout; /* "BSH" | "BNSD" | "BSND"; NULL means "BSH" */
    int64_t batch, num_heads, num_key_value_heads, head_dim, kv_seq_len;
    double scale_value;
    const int64_t *actual_seq_lengths;
    const int64_t *kv_padding_size;
    int64_t kv_padding_size_count; /* 1 or batch when kv_padding_size != NULL */
    const void *atten_mask;
    int32_t dtype_mask;
    int64_t mask_batch, mask_heads, mask_seq;
    const void *pse_shift;
    const void *antiquant_scale;
    const void *antiquant_offset;
    int32_t antiquant_mode;
    int64_t split_tokens;
    void *profile_event_begin; /* optional hipEvent_t recorded right before the split kernel */
    void *profile_event_end;   /* optional hipEvent_t recorded right after it (both or neither) */
    int64_t pse_batch, pse_seq; /* pse_shift shape (pse_batch, N, 1, pse_seq) */
    const void *const *key_list;    /* per-batch caches: device array of `batch` device pointers */
    const void *const *value_list;
    const int64_t *kv_list_seq_len; /* host int64[batch]: positions of each list tensor */
    const void *quant_scale2;       /* int8 output: quantScale2, device, quant_count values */
    const void *quant_offset2;      /* int8 output: quantOffset2 or NULL, same dtype and count */
    int64_t quant_count;            /* 1 (per-tensor) or num_heads * head_dim (per-channel) */
    int32_t dtype_quant;            /* IFA_DT_F32, or IFA_DT_BF16 with bf16 inputs */
} ifa_decode_args;

/*
 * Paged KV cache (README "Constraints > page attention").
 *
 * key_cache / value_cache: kv_cache_layout 0 = (num_blocks, N_kv, block_size,
 *   D) or 1 = (num_blocks, block_size, N_kv*D); identical shapes.  Layout 1
 *   is the only one allowed for "BSH"/"BSND" queries.
 * block_table: device int32 [batch, max_blocks_per_seq]; logical position s
 *   of batch b is row s % block_size of block block_table[b][s / block_size].
 *   Entries for positions < L_b must lie in [0, num_blocks); an entry outside
 *   that range is never dereferenced and its positions are left out.
 * actual_seq_lengths: host int64[batch], required, 0 <= L_b <=
 *   max_blocks_per_seq * block_size.
 * block_size: 16..512, a multiple of 16 (fp16/bf16) or of 32 (int8).
 * atten_mask and pse_shift index the logical position; mask_seq and
 *   pse_seq >= max L_b.
 * Left padding is not combined with paging (IFA_ERR_PARAM_INVALID).
 */
typedef struct ifa_paged_args {
    uint32_t struct_size; /* sizeof(ifa_paged_args) */
    const void *query;
    const void *key_cache;
    const void *value_cache;
    void *attention_out;
    int32_t dtype_q, dtype_kv, dtype_out;
    const char *input_layout;
    int64_t batch, num_heads, num_key_value_heads, head_dim;
    double scale_value;
    const int64_t *actual_seq_lengths;
    const void *atten_mask;
    int32_t dtype_mask;
    int64_t mask_batch, mask_heads, mask_seq;
    const void *pse_shift;
    const void *antiquant_scale;
    const void *antiquant_offset;
    int32_t antiquant_mode;
    const int32_t *block_table;
    int64_t max_blocks_per_seq, block_size, num_blocks;
    int32_t kv_cache_layout;
    int64_t split_tokens;
    void *profile_event_begin; /* as in ifa_decode_args */
    void *profile_event_end;
    int64_t pse_batch, pse_seq; /* as in ifa_decode_args */
    const void *quant_scale2;   /* int8 output, as in ifa_decode_args */
    const void *quant_offset2;
    int64_t quant_count;
    int32_t dtype_quant;
} ifa_paged_args;

/*
 * SparseFlashAttention, MLA-absorb mode (attention_mode 2) (SparseFlashAttention
 * README: Formula, parameter table, constraints).
 *
 * Query (layout_query):
 *   "BSND" (or NULL): query [B, q_seq, Q_N, 512], query_rope [B, q_seq, Q_N, 64],
 *     sparse_indices [B, q_seq, 1, sparse_size], attention_out [B, q_seq, Q_N, 512].
 *     actual_seq_lengths_query: device int32 [B] counts in [0, q_seq], or NULL
 *     (q_seq each); query rows past a batch's count give zero rows.
 *   "TND": query [q_tokens, Q_N, 512], query_rope [q_tokens, Q_N, 64],
 *     sparse_indices [q_tokens, 1, sparse_size], attention_out [q_tokens, Q_N, 512];
 *     actual_seq_lengths_query (required) holds the prefix sums of the batches'
 *     row counts, so batch b owns rows [lq[b-1], lq[b]) and lq[B-1] == q_tokens.
 * Cache (layout_kv), key and value of one shape, key_rope with 64 in place of 512:
 *   "PA_BSND" (or NULL): [num_blocks, block_size, 1, 512] with block_table
 *     device int32 [B, max_blocks]; position t of batch b is row t % block_size
 *     of block block_table[b][t / block_size]; block_size a multiple of 16, at
 *     most 1024.  actual_seq_lengths_kv: device int32 [B], required.
 *   "BSND": [B, kv_seq, 1, 512]; block_table unused;
 *     actual_seq_lengths_kv: device int32 [B] counts, or NULL (kv_seq each).
 *   "TND": [kv_tokens, 1, 512]; actual_seq_lengths_kv (required) holds prefix
 *     sums, batch b owning rows [lkv[b-1], lkv[b]).
 *   One dtype (fp16 or bf16) for every tensor; value may alias key.
 * Selection: entry i of a query row names block idx = sparse_indices[..][i]
 *   of sparse_block_size consecutive positions idx * sparse_block_size + u;
 *   a negative entry is invalid (valid entries first, invalid last, as the
 *   README asks; every valid entry is used wherever it stands, and each
 *   occurrence of a repeated index counts).  A position t is attended when
 *   t < limit, limit = Lkv (sparse_mode 0) or, under sparse_mode 3
 *   (rightDownCausal), min(Lkv, Lkv - Lq + s + 1) for query row s of Lq:
 *   the causal boundary through the bottom-right corner (this library's
 *   reading of the mode).  Positions past Lkv inside a block are left out;
 *   a paged position past the block table is invalid.
 * Envelope: kv_heads == 1, head_dim == 512, rope_dim == 64, 1 <= q_heads <=
 *   128, 1 <= q_seq <= 65536, sparse_size >= 1, sparse_block_size a power
 *   of two in [1, 128] (dividing block_size for a paged cache), sparse_mode
 *   0 or 3, attention_mode == 2; cache rows (num_blocks * block_size, B *
 *   kv_seq or kv_tokens) below 2^31.
 * q_tokens, kv_tokens and kv_seq are the three last fields of the struct; a
 *   struct_size that stops before them allows the BSND query and the
 *   PA_BSND cache only.
 * split_hint: 0 lets the planner choose the number of index chunks per
 *   query row (about one workgroup per compute unit, so a short call can get
 *   well over 64 chunks); 1 to 64 forces it (testing and tuning), anything
 *   else is IFA_ERR_PARAM_INVALID.  The
 *   planner reads the device's compute-unit count when split_hint is 0 or
 *   q_heads > 64 (IFA_ERR_RUNTIME without a device); sfa_decode_mla_plan
 *   reports what it chose.
 * return_softmax_lse (README parameter table: return_softmax_lse,
 *   softmax_max_out, softmax_sum_out): when 1, the call also writes, per
 *   query row and head, softmax_max_out = the maximum of the scaled scores
 *   the softmax takes, and softmax_sum_out = the sum of exp(score - max) over
 *   the attended positions; -inf and 0 for a row that attends nothing (the
 *   scores being the softmax's input after scale_value is this library's
 *   reading).  Shape [B, 1, Q_S, Q_N] for a BSND query, [1, Q_T, Q_N] for a
 *   TND one: element (query row) * Q_N + head.  Only with a BSND or TND
 *   cache, as the README allows (IFA_ERR_PARAM_INVALID with PA_BSND); both
 *   pointers are required then, and must be NULL when return_softmax_lse is
 *   0.  These are the last fields of the struct (ABI version 6); a shorter
 *   struct_size means no such outputs.
 */
typedef struct sfa_mla_args {
    uint32_t struct_size; /* sizeof(sfa_mla_args) */
    const void *query, *query_rope;
    const void *key, *key_rope, *value;
    const int32_t *sparse_indices;
    const int32_t *block_table;
    const int32_t *actual_seq_lengths_query;
    const int32_t *actual_seq_lengths_kv;
    void *attention_out;
    int32_t dtype;
    int64_t batch, q_seq, q_heads, kv_heads, head_dim, rope_dim;
    int64_t sparse_size, block_size, num_blocks, max_blocks;
    float scale_value;
    int64_t sparse_block_size, sparse_mode, attention_mode;
    const char *layout_query; /* "BSND" | "TND"; NULL means "BSND" */
    const char *layout_kv;    /* "PA_BSND" | "BSND" | "TND"; NULL means "PA_BSND" */
    int64_t split_hint;
    void *profile_event_begin; /* optional hipEvent_t pair recorded around the gather kernel */
    void *profile_event_end;
    int64_t q_tokens;  /* Q_T of a TND query */
    int64_t kv_tokens; /* KV_T of a TND cache */
    int64_t kv_seq;    /* KV_S of a BSND cache */
    float *softmax_max_out;     /* return_softmax_lse: device fp32, see above */
    float *softmax_sum_out;
    int32_t return_softmax_lse; /* 0 or 1 */
} sfa_mla_args;

/* Phase 1: validate and return the workspace bytes the run call needs. */
int ifa_decode_workspace_size(const ifa_decode_args *args, size_t *workspace_bytes);
int ifa_decode_paged_workspace_size(const ifa_paged_args *args, size_t *workspace_bytes);
int sfa_decode_mla_workspace_size(const sfa_mla_args *args, size_t *workspace_bytes);

/*
 * The launch sfa_decode_mla makes for these arguments (the same planner,
 * with the validation and return codes of sfa_decode_mla_workspace_size):
 * index chunks per query row, index entries per chunk, workgroups of the
 * gather kernel, and all_heads = 1 when one workgroup takes every query head
 * of a chunk, 0 for workgroups of 64 heads.  The planner takes all heads
 * when there are more than 64 and the 64-head workgroups (one per compute
 * unit at most) would not all fit on the device at once: that halves the
 * grid.  For tuning and tests; a call needs none of it.  `plan` is written
 * only on success.
 */
typedef struct sfa_mla_plan {
    int32_t chunks;
    int32_t chunk_entries;
    int32_t workgroups;
    int32_t all_heads;
} sfa_mla_plan;
int sfa_decode_mla_plan(const sfa_mla_args *args, sfa_mla_plan *plan);

/* Phase 2: validate again and enqueue on `stream`.  workspace may be NULL
 * only when the size query returned 0. */
int ifa_decode(const ifa_decode_args *args, void *workspace, size_t workspace_bytes, ifa_stream_t stream);
int ifa_decode_paged(const ifa_paged_args *args, void *workspace, size_t workspace_bytes, ifa_stream_t stream);
int sfa_decode_mla(const sfa_mla_args *args, void *workspace, size_t workspace_bytes, ifa_stream_t stream);

/*
 * ifa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It validates and computes exactly as ifa_decode
 * does, with the same kernels, and keeps the partial states in a built-in
 * device array of IFA_NOALLOC_SCRATCH_BYTES (32 MiB) that every GPU the
 * library runs on holds until the process ends.  A call whose workspace
 * (the size ifa_decode_workspace_size returns) exceeds that returns
 * IFA_ERR_PARAM_INVALID and launches nothing.  It allocates nothing and
 * calls no allocating routine; the first call on a device looks up that
 * device's copy of the array (a HIP runtime failure there is
 * IFA_ERR_RUNTIME).  All calls on one GPU share its array: calls that may
 * overlap on one GPU (other streams, other threads) race and must not be
 * issued; calls ordered on one stream are safe.
 */
#define IFA_NOALLOC_SCRATCH_BYTES (32u << 20)
int ifa_decode_noalloc(const ifa_decode_args *args, ifa_stream_t stream);

/* A static string naming a status code. */
const char *ifa_status_string(int status);

/* The library's ABI version (bumped when a struct changes). */
int ifa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* IFA_DECODE_H */
