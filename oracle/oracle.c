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
 *   score uses the 512-wide part plus the 64-wide rope part.
 *
 * Readings where the pages are silent: an empty attention set gives a zero
 * row; duplicate sparse indices each count; sparse_mode 3 with one query row
 * equals mode 0.
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

enum { O_F16 = 1, O_BF16 = 2, O_I8 = 3 };
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
    case O_F16: return oracle_f16_to_f64(((const uint16_t *)base)[i]);
    case O_BF16: return oracle_bf16_to_f64(((const uint16_t *)base)[i]);
    case O_I8: return (double)((const int8_t *)base)[i];
    default: return NAN;
    }
}

/* Softmax-weighted sum over n gathered rows.  x[i] are the scores, rows of V
 * are fetched through vrow(i, d).  Writes D doubles to out. */
typedef double (*vfetch_fn)(const void *ctx, int64_t i, int64_t d);

static void softmax_combine(const double *x, int64_t n, int64_t D, vfetch_fn vrow, const void *ctx,
                            double *w, double *out) {
    double m = -INFINITY;
    for (int64_t i = 0; i < n; i++)
        if (x[i] > m) m = x[i];
    if (n == 0 || m == -INFINITY) {      /* nothing attended (every score -inf counts as none) */
        for (int64_t d = 0; d < D; d++) out[d] = 0.0;
        return;
    }
    double z = 0.0;
    for (int64_t i = 0; i < n; i++) {
        w[i] = exp(x[i] - m);
        z += w[i];
    }
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
 */
int oracle_ifa(const void *q, int q_dtype, const void *k, const void *v, int kv_dtype, int layout, int64_t B,
               int64_t N, int64_t Nkv, int64_t D, int64_t S, double scale, const int64_t *actual,
               const int64_t *pad, const uint8_t *mask, int64_t mB, int64_t mN, int64_t mS,
               const int32_t *block_table, int64_t max_blocks, int64_t block_size, int64_t num_blocks,
               int cache_layout, const void *aq_scale, const void *aq_offset, int aq_mode,
               const int64_t *rows, int64_t nrows, double *out, const void *pse, int64_t pB, int64_t pS) {
    if (Nkv == 0) Nkv = N;
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
        const int64_t L = actual ? actual[b] : S;
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
            } else if (layout == O_BNSD) {
                off = ((b * Nkv + j) * S + s) * D;
            } else {
                off = (b * S + s) * Nkv * D + j * D;
            }
            double dot = 0.0;
            for (int64_t d = 0; d < D; d++) {
                double kv = elem(k, kv_dtype, off + d);
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
        ifa_vctx c = {v, kv_dtype, ko, aq_scale, aq_offset, q_dtype, aq_mode, j, Nkv, D};
        softmax_combine(x, cnt, D, ifa_vfetch, &c, w, o);
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
 * MLA-absorb sparse decode, query layout BSND with Q_S = 1, KV_N = 1, cache
 * layout PA_BSND.
 *   q [B,1,QN,D], q_rope [B,1,QN,DR], key/value [nblk,bs,1,D], key_rope [nblk,bs,1,DR]
 *   sparse_indices [B,1,1,sparse_size] int32; block_table [B,max_blocks] int32;
 *   lkv [B] int32 (valid iff 0 <= t < lkv[b]).
 *   scale is the float32 scale value widened to double.
 *   rows: list of b*QN+h rows (NULL -> all); out has nrows*D doubles.
 */
int oracle_sfa(const void *q, const void *q_rope, const void *key, const void *key_rope, const void *value,
               int dtype, const int32_t *sparse_indices, const int32_t *block_table, const int32_t *lkv,
               int64_t B, int64_t QN, int64_t D, int64_t DR, int64_t sparse_size, int64_t block_size,
               int64_t num_blocks, int64_t max_blocks, double scale, const int64_t *rows, int64_t nrows,
               double *out) {
    const int64_t total = rows ? nrows : B * QN;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t r = 0; r < total; r++) {
        const int64_t bh = rows ? rows[r] : r;
        const int64_t b = bh / QN, h = bh % QN;
        double *o = out + r * D;
        double *x = (double *)malloc(sizeof(double) * (size_t)sparse_size);
        double *w = (double *)malloc(sizeof(double) * (size_t)sparse_size);
        int64_t *ko = (int64_t *)malloc(sizeof(int64_t) * (size_t)sparse_size);
        int64_t cnt = 0;
        for (int64_t i = 0; i < sparse_size; i++) {
            int64_t t = sparse_indices[b * sparse_size + i];
            if (t < 0 || t >= lkv[b]) continue;
            int64_t blk = block_table[b * max_blocks + t / block_size];
            if (blk < 0 || blk >= num_blocks) { err |= 1; break; }
            int64_t row = blk * block_size + t % block_size;
            double dot = 0.0;
            for (int64_t d = 0; d < D; d++)
                dot += elem(q, dtype, (b * QN + h) * D + d) * elem(key, dtype, row * D + d);
            for (int64_t d = 0; d < DR; d++)
                dot += elem(q_rope, dtype, (b * QN + h) * DR + d) * elem(key_rope, dtype, row * DR + d);
            x[cnt] = scale * dot;
            ko[cnt] = row * D;
            cnt++;
        }
        sfa_vctx c = {value, dtype, ko};
        softmax_combine(x, cnt, D, sfa_vfetch, &c, w, o);
        free(x);
        free(w);
        free(ko);
    }
    return err ? -2 : 0;
}
