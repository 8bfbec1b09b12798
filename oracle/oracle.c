/*
 * fp64 CPU oracle for decode attention (IncreFlashAttention and
 * SparseFlashAttention, MLA-absorb mode).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: it exists so tests, the smoke check and the CPU
 * baseline leg of the benchmark can check the HIP library against the plain
 * definition.  It shares no code, header or table with the library.
 *
 * What it computes (plain definition, no tiling, no online softmax):
 *
 *   IncreFlashAttention README, "Formula" section, and the
 *   aclnnIncreFlashAttentionV2 page, "Function > Formula":
 *       out = softmax(scale * q K^T) V         with the query S axis = 1
 *   restricted per batch to the KV positions the page defines:
 *     - actualSeqLengths: right padding, positions [0, L_b)      (V2 parameter table)
 *     - kv left padding: start = Smax - pad - L, end = Smax - pad;
 *       start or end < 0 gives an all-zero row; pad < 0 counts as 0
 *                                   (README "Constraints > kv left padding")
 *     - attenMask: a nonzero byte excludes the position            (reading, see below)
 *     - pseShift: an additive bias pse[b|0, h, 0, s] in the query dtype, added
 *       after the scale, at the same position coordinate as the mask
 *                                   (README "Function > Formula" and
 *                                    "Constraints"; placement is a reading)
 *     - GQA: query head h reads KV head h / (N / N_kv)              (reading)
 *     - page attention: logical position s lives in block
 *       blockTable[b][s / blockSize], row s % blockSize   (README "Constraints > page attention")
 *     - int8 antiquant: dequantised value = (x + offset) * scale, index 0 of the
 *       leading axis for K, 1 for V; per-tensor shape (2), per-channel
 *       (2, N_kv, 1, D)             (README "Constraints > antiquantScale / antiquantOffset"; reading)
 *
 *   SparseFlashAttention README, "Formula" and parameter table:
 *       out = softmax(q [K~]^T / sqrt(d_k)) V~
 *   where the rows of K~ and V~ are the cache rows named by sparse_indices,
 *   an index t being valid when 0 <= t < actual_seq_lengths_kv[b]; each row's
 *   score uses the 512-wide part plus the 64-wide rope part.  Query layouts
 *   BSND and TND, cache layouts PA_BSND, BSND and TND, several query rows per
 *   batch with sparse_mode 3 (rightDownCausal), and block-wise selection
 *   (sparse_block_size > 1: an index names sparse_block_size consecutive
 *   positions) as the parameter table describes them.
 *
 * Readings where the pages are silent: an empty attention set gives a zero
 * row; duplicate sparse indices each count; sparse_mode 3 with one query row
 * equals mode 0; the causal boundary of mode 3 puts query row s (of Lq) level
 * with KV position Lkv - Lq + s; query rows past actual_seq_lengths_query
 * give zero rows; a position past Lkv or the causal limit inside a selected
 * block is left out.
 *
 * Parity unpinned (conventions the pages do not fix): the GQA head map
 * h -> h / (N / N_kv) and the antiquant form (x + offset) * scale.  The tests
 * pin the rest of the arithmetic around them; the conventions themselves are
 * shared by both sides, not checked against the pages.
 *
 * Arithmetic: stored fp16/bf16/int8 values are widened exactly to double;
 * exp is libm exp in double; softmax subtracts the row maximum.
 *
 * Return value: 0 on success, a negative number for an input the oracle
 * cannot evaluate (a block id out of range, an unknown dtype or layout).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { O_F16 = 1, O_BF16 = 2, O_I8 = 3, O_F32 = 6 };

/* Threads the parallel row loops below may use from now on (n >= 1); returns
 * the count in effect.  Only the CPU-baseline timing changes it. */
int oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
enum { O_BSH = 0, O_BNSD = 1, O_BSND = 2 };

/* IEEE-754 binary16 -> double, written from the format's definition:
 * sign(1) exponent(5, bias 15) fraction(10); exponent 0 is subnormal. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

static double elem(const void *base, int dtype, int64_t i) {
    switch (dtype) {
    case O_F32: return (double)((const float *)base)[i];
    case O_F16: return oracle_f16_to_f64(((const uint16_t *)base)[i]);
    case O_BF16: return oracle_bf16_to_f64(((const uint16_t *)base)[i]);
    case O_I8: return (double)((const int8_t *)base)[i];
    default: return NAN;
    }
}

/* Softmax-weighted sum over n gathered rows.  x[i] are the scores, rows of V
 * are fetched through vrow(i, d).  Writes D doubles to out, and, when m_out
 * and z_out are given, the softmax's maximum score and its sum of
 * exp(score - maximum) (-inf and 0 when nothing is attended). */
typedef double (*vfetch_fn)(const void *ctx, int64_t i, int64_t d);

static void softmax_combine(const double *x, int64_t n, int64_t D, vfetch_fn vrow, const void *ctx,
                            double *w, double *out, double *m_out, double *z_out) {
    double m = -INFINITY;
    for (int64_t i = 0; i < n; i++)
        if (x[i] > m) m = x[i];
    if (m_out) *m_out = m;
    if (z_out) *z_out = 0.0;
    if (n == 0 || m == -INFINITY) {      /* nothing attended (every score -inf counts as none) */
        for (int64_t d = 0; d < D; d++) out[d] = 0.0;
        return;
    }
    double z = 0.0;
    for (int64_t i = 0; i < n; i++) {
        w[i] = exp(x[i] - m);
        z += w[i];
    }
    if (z_out) *z_out = z;
    for (int64_t d = 0; d < D; d++) {
        double acc = 0.0;
        for (int64_t i = 0; i < n; i++) acc += w[i] * vrow(ctx, i, d);
        out[d] = acc / z;
    }
}

/* ---------------------------------------------------------------- IFA ---- */

typedef struct {
    const void *v;
    int kv_dtype;
    const int64_t *rowoff; /* element offset of each gathered V row */
    const void *aq_scale, *aq_offset;
    int aq_dtype, aq_mode;
    int64_t j, Nkv, D;
} ifa_vctx;

static double aq_param(const void *p, int dtype, int mode, int which, int64_t j, int64_t Nkv, int64_t D,
                       int64_t d) {
    if (mode == 1) return elem(p, dtype, which);
    return elem(p, dtype, (which * Nkv + j) * D + d);
}

static double ifa_vfetch(const void *c, int64_t i, int64_t d) {
    const ifa_vctx *x = (const ifa_vctx *)c;
    double v = elem(x->v, x->kv_dtype, x->rowoff[i] + d);
    if (x->aq_mode) {
        double sc = aq_param(x->aq_scale, x->aq_dtype, x->aq_mode, 1, x->j, x->Nkv, x->D, d);
        double of = aq_param(x->aq_offset, x->aq_dtype, x->aq_mode, 1, x->j, x->Nkv, x->D, d);
        v = (v + of) * sc;
    }
    return v;
}

/*
 * Dense padded cache or paged cache.
 *   q, out: [B, N, D] for every query layout (query S axis is 1).
 *   dense k, v: layout BSH [B,S,Nkv*D], BNSD [B,Nkv,S,D], BSND [B,S,Nkv,D].
 *   paged (block_table != NULL): cache_layout 0 -> [nblk, Nkv, bs, D],
 *     1 -> [nblk, bs, Nkv*D]; block_table [B, max_blocks] int32.
 *   actual: per-batch lengths or NULL (-> S).  pad: per-batch kvPaddingSize or NULL.
 *   mask: bytes [mB, mN, 1, mS], mB in {1,B}, mN in {1,N}; nonzero excludes.
 *   rows: list of b*N+h rows to evaluate (NULL -> all); out has nrows*D doubles.
 *   k_list, v_list, list_seq (all or none): per-batch caches (the V2 page's
 *     tensor lists, "Constraints": one tensor per batch, batch 1, shapes equal
 *     but for S): batch b reads k_list[b] / v_list[b], a one-batch cache of
 *     list_seq[b] positions in `layout`; lengths default to list_seq[b];
 *     left padding is not combined with lists (reading).
 */
int oracle_ifa(const void *q, int q_dtype, const void *k, const void *v, int kv_dtype, int layout, int64_t B,
               int64_t N, int64_t Nkv, int64_t D, int64_t S, double scale, const int64_t *actual,
               const int64_t *pad, const uint8_t *mask, int64_t mB, int64_t mN, int64_t mS,
               const int32_t *block_table, int64_t max_blocks, int64_t block_size, int64_t num_blocks,
               int cache_layout, const void *aq_scale, const void *aq_offset, int aq_mode,
               const int64_t *rows, int64_t nrows, double *out, const void *pse, int64_t pB, int64_t pS,
               const void *const *k_list, const void *const *v_list, const int64_t *list_seq) {
    if (Nkv == 0) Nkv = N;
    if (k_list && (!v_list || !list_seq || pad || block_table)) return -3;
    if (N % Nkv) return -1;
    const int64_t g = N / Nkv;
    const int paged = block_table != NULL;
    const int64_t total = rows ? nrows : B * N;
    int err = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t r = 0; r < total; r++) {
        const int64_t bh = rows ? rows[r] : r;
        const int64_t b = bh / N, h = bh % N, j = h / g;
        double *o = out + r * D;
        const int64_t Sb = k_list ? list_seq[b] : S;     /* positions of this batch's cache */
        const void *kb = k_list ? k_list[b] : k, *vb = k_list ? v_list[b] : v;
        const int64_t L = actual ? actual[b] : Sb;
        if (L < 0 || L > Sb) { err |= 1; continue; }
        if (paged && L > max_blocks * block_size) { err |= 1; continue; }   /* past the block table */
        int64_t lo = 0, hi = L;
        if (!paged && pad && actual) {
            int64_t p = pad[b] < 0 ? 0 : pad[b];
            lo = S - p - L;
            hi = S - p;
            if (lo < 0 || hi < 0) {
                for (int64_t d = 0; d < D; d++) o[d] = 0.0;
                continue;
            }
        }
        int64_t n = hi > lo ? hi - lo : 0;
        double *x = (double *)malloc(sizeof(double) * (size_t)(n ? n : 1));
        double *w = (double *)malloc(sizeof(double) * (size_t)(n ? n : 1));
        int64_t *ko = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n ? n : 1));
        int64_t cnt = 0;
        for (int64_t s = lo; s < hi; s++) {
            if (mask) {
                if (s >= mS) { err |= 1; break; }       /* the mask is shorter than the window */
                int64_t mi = ((mB == 1 ? 0 : b) * mN + (mN == 1 ? 0 : h)) * mS + s;
                if (mask[mi]) continue;
            }
            int64_t off;
            if (paged) {
                int64_t blk = block_table[b * max_blocks + s / block_size];
                if (blk < 0 || blk >= num_blocks) { err |= 1; break; }
                if (cache_layout == 0)
                    off = ((blk * Nkv + j) * block_size + s % block_size) * D;
                else
                    off = (blk * block_size + s % block_size) * Nkv * D + j * D;
            } else if (k_list) {
                off = layout == O_BNSD ? (j * Sb + s) * D : s * Nkv * D + j * D;
            } else if (layout == O_BNSD) {
                off = ((b * Nkv + j) * S + s) * D;
            } else {
                off = (b * S + s) * Nkv * D + j * D;
            }
            double dot = 0.0;
            for (int64_t d = 0; d < D; d++) {
                double kv = elem(kb, kv_dtype, off + d);
                if (aq_mode) {
                    double sc = aq_param(aq_scale, q_dtype, aq_mode, 0, j, Nkv, D, d);
                    double of = aq_param(aq_offset, q_dtype, aq_mode, 0, j, Nkv, D, d);
                    kv = (kv + of) * sc;
                }
                dot += elem(q, q_dtype, (b * N + h) * D + d) * kv;
            }
            x[cnt] = scale * dot;
            if (pse) {
                if (s >= pS) { err |= 1; break; }
                x[cnt] += elem(pse, q_dtype, ((pB == 1 ? 0 : b) * N + h) * pS + s);
            }
            ko[cnt] = off;
            cnt++;
        }
        ifa_vctx c = {vb, kv_dtype, ko, aq_scale, aq_offset, q_dtype, aq_mode, j, Nkv, D};
        softmax_combine(x, cnt, D, ifa_vfetch, &c, w, o, NULL, NULL);
        free(x);
        free(w);
        free(ko);
    }
    return err ? -2 : 0;
}

/* ---------------------------------------------------------------- SFA ---- */

typedef struct {
    const void *value;
    int dtype;
    const int64_t *rowoff;
} sfa_vctx;

static double sfa_vfetch(const void *c, int64_t i, int64_t d) {
    const sfa_vctx *x = (const sfa_vctx *)c;
    return elem(x->value, x->dtype, x->rowoff[i] + d);
}

/*
 * MLA-absorb sparse attention (KV_N = 1), SparseFlashAttention README,
 * "Formula" and parameter table.
 *
 * Query rows.  layout_q 0 = BSND: q [B, QS, QN, D], row (b, s); lq[b] (or QS
 * when lq is NULL) of them are valid and the rest give zero rows.  layout_q
 * 1 = TND: q [QT, QN, D]; lq holds prefix sums, batch b owning rows
 * [lq[b-1], lq[b]).  q_rope, sparse_indices ([rows, sparse_size]) and the
 * output follow the same row order.
 *
 * Cache.  layout_kv 0 = PA_BSND: [num_blocks, block_size, 1, D], position t
 * of batch b in row block_table[b][t / block_size] * block_size + t %
 * block_size; lkv[b] positions.  1 = BSND: [B, KV_S, 1, D], row b * KV_S +
 * t; lkv[b] positions (KV_S when lkv is NULL).  2 = TND: [KV_T, 1, D]; lkv
 * holds prefix sums, batch b owning rows [lkv[b-1], lkv[b]).
 *
 * Selection.  Entry i of row (b, s) names block idx = sparse_indices[...][i]
 * of sparse_block_size positions, t = idx * sparse_block_size + u; a
 * negative idx is invalid.  A position is attended when t < limit: limit =
 * Lkv (sparse_mode 0), or min(Lkv, Lkv - Lq + s + 1) under sparse_mode 3
 * (the causal boundary through the bottom-right corner of the Lq x Lkv
 * score matrix).  Each occurrence of a repeated index counts.
 *
 *   scale is the float32 scale value widened to double.
 *   rows: list of (query row) * QN + head (NULL -> all); out has nrows*D doubles.
 *   lse_max, lse_sum (NULL, or nrows doubles each): softmax_max and
 *   softmax_sum of the README's return_softmax_lse outputs, per output row:
 *   the maximum of the scaled scores the softmax takes, and the sum of
 *   exp(score - maximum); -inf and 0 for a row that attends nothing (the
 *   scores being the softmax's own input, after the scale, is a reading).
 */
int oracle_sfa(const void *q, const void *q_rope, const void *key, const void *key_rope, const void *value,
               int dtype, const int32_t *sparse_indices, const int32_t *block_table, const int32_t *lkv,
               const int32_t *lq, int layout_q, int layout_kv, int64_t B, int64_t QS, int64_t q_rows,
               int64_t QN, int64_t D, int64_t DR, int64_t sparse_size, int64_t block_size, int64_t num_blocks,
               int64_t max_blocks, int64_t kv_seq, int sparse_mode, int64_t sparse_block_size, double scale,
               const int64_t *rows, int64_t nrows, double *out, double *lse_max, double *lse_sum) {
    if (layout_q != 0 && layout_q != 1) return -3;
    if (layout_kv < 0 || layout_kv > 2) return -3;
    if ((layout_q == 1 && !lq) || (layout_kv != 1 && !lkv) || sparse_block_size < 1) return -3;
    const int64_t total = rows ? nrows : q_rows * QN;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t r = 0; r < total; r++) {
        const int64_t rh = rows ? rows[r] : r;
        const int64_t qr = rh / QN, h = rh % QN;
        double *o = out + r * D;
        /* the query row's batch, its place in the batch, and the batch's query count */
        int64_t b, s, Lq;
        if (layout_q == 0) {
            b = qr / QS;
            s = qr % QS;
            Lq = lq ? lq[b] : QS;
        } else {
            b = 0;
            while (b < B && lq[b] <= qr) b++;
            if (b == B) { err |= 1; continue; }
            const int64_t start = b > 0 ? lq[b - 1] : 0;
            s = qr - start;
            Lq = lq[b] - start;
        }
        int64_t kv0 = 0, Lkv;
        if (layout_kv == 2) {
            kv0 = b > 0 ? lkv[b - 1] : 0;
            Lkv = lkv[b] - kv0;
        } else {
            Lkv = lkv ? lkv[b] : kv_seq;
            if (layout_kv == 1) {
                kv0 = b * kv_seq;
                if (Lkv > kv_seq) { err |= 1; continue; }   /* a length past the batch's cache */
            }
        }
        int64_t limit = Lkv;
        if (sparse_mode == 3 && Lkv - Lq + s + 1 < limit) limit = Lkv - Lq + s + 1;
        if (s >= Lq) limit = 0;                       /* a padding query row: zero output */
        const int64_t cap = sparse_size * sparse_block_size;
        double *x = (double *)malloc(sizeof(double) * (size_t)cap);
        double *w = (double *)malloc(sizeof(double) * (size_t)cap);
        int64_t *ko = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
        int64_t cnt = 0;
        for (int64_t i = 0; i < sparse_size && !err; i++) {
            const int64_t idx = sparse_indices[qr * sparse_size + i];
            if (idx < 0) continue;
            for (int64_t u = 0; u < sparse_block_size; u++) {
                const int64_t t = idx * sparse_block_size + u;
                if (t >= limit) continue;
                int64_t row;
                if (layout_kv == 0) {
                    if (t / block_size >= max_blocks) continue;      /* past the table: invalid */
                    int64_t blk = block_table[b * max_blocks + t / block_size];
                    if (blk < 0 || blk >= num_blocks) { err |= 1; break; }
                    row = blk * block_size + t % block_size;
                } else {
                    row = kv0 + t;
                }
                double dot = 0.0;
                for (int64_t d = 0; d < D; d++)
                    dot += elem(q, dtype, (qr * QN + h) * D + d) * elem(key, dtype, row * D + d);
                for (int64_t d = 0; d < DR; d++)
                    dot += elem(q_rope, dtype, (qr * QN + h) * DR + d) * elem(key_rope, dtype, row * DR + d);
                x[cnt] = scale * dot;
                ko[cnt] = row * D;
                cnt++;
            }
        }
        sfa_vctx c = {value, dtype, ko};
        softmax_combine(x, cnt, D, sfa_vfetch, &c, w, o, lse_max ? lse_max + r : NULL, lse_sum ? lse_sum + r : NULL);
        free(x);
        free(w);
        free(ko);
    }
    return err ? -2 : 0;
}

/* ------------------------------------------------------- output int8 ---- */

/*
 * Post-quantisation of the attention output into int8 (IncreFlashAttention
 * README "Constraints": quantScale2 required, quantOffset2 optional, per-tensor
 * or per-channel, fp32 or bf16).  The pages give no formula; the reading taken
 * is y = o * scale + offset on the exact output, rounded to the nearest
 * integer with ties to even, then saturated to [-128, 127].
 *   o: n doubles, channel of element i = i % C (C = 1 per-tensor, N*D
 *   per-channel over the output's heads); qs / qo: C values of q_dtype
 *   (qo may be NULL); out: n codes; pre (may be NULL): the value y before
 *   rounding, so a test can see how close it came to a rounding boundary.
 */
int oracle_quant_int8(const double *o, int64_t n, int64_t C, const void *qs, const void *qo, int q_dtype,
                      int8_t *out, double *pre) {
    if (C < 1) return -1;
    for (int64_t i = 0; i < n; i++) {
        const int64_t c = i % C;
        double y = o[i] * elem(qs, q_dtype, c);
        if (qo) y += elem(qo, q_dtype, c);
        if (pre) pre[i] = y;
        double r = nearbyint(y);                /* the default rounding mode: to nearest, ties to even */
        if (r > 127.0) r = 127.0;
        if (r < -128.0) r = -128.0;
        out[i] = (int8_t)r;
    }
    return 0;
}
