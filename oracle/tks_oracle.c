/*
 * tks_oracle.c -- plain, slow CPU oracle for the sparse-attention indexer and
 * its per-query top-k, flat (DSA-style) and hierarchical (HISA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header
 * or table with the GPU library; it is written from the definitions below.
 *
 * What it computes (every sum in double, every loop in plain index order):
 *
 *  - Indexer score (HISA abstract: a lightweight indexer scores every
 *    historical key for each query; StreamIndex abstract: a learned scoring
 *    projection over the keys with H_I indexer heads):
 *        I[t,s] = sum_h w[t,h] * max(0, sum_d q[t,h,d] * k[s,d])
 *    For fp8 keys the key value is scale[s] * e4m3fn(code) and the per-head
 *    dot product is  scale[s] * sum_d q[t,h,d] * e4m3fn(code[s,d]).
 *    A score of -0 is taken as +0.
 *
 *  - Causal visibility (HISA abstract: the indexer scans the entire prefix
 *    for every query).  vis(t) = floor((q_pos0 + t) / ratio); key s is seen by
 *    query t iff s <= vis(t) and s < n_k (ratio > 1 is causality at the
 *    compressed-key granularity of the StreamIndex abstract).
 *
 *  - Flat top-k (HISA abstract: a per-query top-k index set): the visible keys
 *    ordered by score descending, then key index ascending; the first
 *    min(k, |visible|) are emitted in that order and the rest is -1.
 *
 *  - HISA stage 1 (HISA abstract, stage (1): pooled block representatives
 *    are scored and irrelevant regions discarded): kbar[b] is the bf16
 *    (nearest-even) rounding of the mean of the B keys of block b, summed in
 *    double in ascending key order, complete blocks only.  The local block
 *    L = floor(min(vis, n_k-1) / B) and, optionally, block 0 are forced; the
 *    complete blocks b < L (minus forced block 0) are scored with the same
 *    indexer on kbar and the best m_scored (score desc, block asc) are kept.
 *
 *  - HISA stage 2 (HISA abstract, stage (2): the original indexer applied
 *    only within the retained blocks): flat top-k over the visible keys whose
 *    block is kept.
 *
 *  - Key compression (StreamIndex abstract: the indexer reads keys
 *    compressed by a ratio m, m = 4 for V4-Flash): compressed key j is the
 *    bf16 (nearest-even) rounding of the mean of raw keys m*j .. m*j+m-1,
 *    summed in double in position order.  An fp8 key cache stores it as
 *    e4m3fn codes with one fp32 scale per key: scale = max_d |kc[d]| / 448
 *    (fp32 division), code[d] = nearest e4m3fn of kc[d] / scale (fp32
 *    division; ties to the even code, saturated at 448, sign kept); an
 *    all-zero key gets scale 0 and zero codes.  The pages give no formula
 *    for the compressor; this mean is the plainest reading of "compressed
 *    keys" that the HISA pooling (a block mean) also uses.
 *
 * Errors: a function returns 0 on success and a negative value on a bad
 * argument; outputs are then untouched.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t batch, n_q, n_k, heads, dim;
    int32_t q_pos0;
    int32_t causal_ratio;
    int32_t key_fp8; /* 0: keys are bf16 bit patterns; 1: e4m3fn codes + fp32 scale */
} orc_shape;

enum { ORC_FORCE_FIRST = 1, ORC_FORCE_LOCAL = 2 };

/* ---------------------------------------------------------------- decoding */

double orc_bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 * subnormals at exponent 0, S.1111.111 is NaN, no infinities. */
double orc_e4m3fn_to_double(uint8_t code) {
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Round a double to bf16, nearest with ties to even; returns the bit pattern.
 * bf16 has 8 significant bits: a normal number 1.m * 2^E (E >= -126) is
 * quantised to multiples of 2^(E-7), subnormals to multiples of 2^-133. */
uint16_t orc_double_to_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    int neg = signbit(x) ? 1 : 0;
    double a = fabs(x);
    uint16_t out;
    if (a == 0.0) {
        out = 0;
    } else {
        int ex;
        frexp(a, &ex);            /* a = f * 2^ex, f in [0.5, 1): E = ex - 1 */
        int E = ex - 1;
        if (E < -126) E = -126;   /* subnormal range keeps the 2^-133 quantum */
        double quantum = ldexp(1.0, E - 7);
        double n = rint(a / quantum); /* default rounding: nearest, ties even */
        double v = n * quantum;
        if (v >= ldexp(1.0, 128)) {
            out = 0x7F80; /* overflow to infinity */
        } else {
            float f = (float)v; /* exact: v has <= 8 significant bits */
            uint32_t u;
            memcpy(&u, &f, sizeof u);
            out = (uint16_t)(u >> 16);
        }
    }
    return (uint16_t)(out | (neg ? 0x8000 : 0));
}

/* OCP e4m3fn code of x: the nearest e4m3fn magnitude to |x| (saturated at
 * 448, the largest finite one), ties to the even code, sign bit copied.
 * Magnitudes below 2^-6 lie on the subnormal grid of step 2^-9; a normal
 * magnitude 1.m * 2^E (-6 <= E <= 8) on the grid of step 2^(E-3).  A value
 * rounding up to the next power of two lands on that binade's first code,
 * which the grid index gives by itself. */
uint8_t orc_float_to_e4m3fn(float x) {
    double a = fabs((double)x);
    if (a > 448.0) a = 448.0;
    int code;
    if (a < ldexp(1.0, -6)) {
        code = (int)rint(a / ldexp(1.0, -9)); /* 0 .. 8; 8 is 2^-6, code 0x08 */
    } else {
        int ex;
        frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1): E = ex - 1 */
        int E = ex - 1;
        int n = (int)rint(a / ldexp(1.0, E - 3)); /* 8 .. 16 significand steps */
        code = ((E + 7) << 3) + (n - 8);         /* n = 16 carries into E + 1 */
    }
    return (uint8_t)(code | (signbit(x) ? 0x80 : 0));
}

/* --------------------------------------------------------------- geometry */

static int64_t floor_div(int64_t a, int64_t b) {
    int64_t q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
    return q;
}

/* Number of keys visible to query t (a prefix 0..n-1 of the key sequence). */
int64_t orc_n_visible(const orc_shape* S, int64_t t) {
    int64_t vis = floor_div((int64_t)S->q_pos0 + t, S->causal_ratio);
    if (vis < 0) return 0;
    return vis + 1 < S->n_k ? vis + 1 : S->n_k;
}

static int check_shape(const orc_shape* S) {
    if (!S || S->batch < 0 || S->n_q < 0 || S->n_k < 0 || S->heads <= 0 || S->dim <= 0 ||
        S->causal_ratio <= 0 || (S->key_fp8 != 0 && S->key_fp8 != 1))
        return -1;
    return 0;
}

/* Dequantised key value k[b, s, d] as a double. */
static double key_value(const orc_shape* S, const void* k, const float* k_scale,
                        int64_t b, int64_t s, int64_t d) {
    int64_t off = (b * S->n_k + s) * S->dim + d;
    if (S->key_fp8)
        return (double)k_scale[b * S->n_k + s] * orc_e4m3fn_to_double(((const uint8_t*)k)[off]);
    return orc_bf16_to_double(((const uint16_t*)k)[off]);
}

/* ----------------------------------------------------------------- scoring */

/* Indexer score of one query (qrow: [heads, dim] bf16 bits, wrow: [heads])
 * against key s of batch element b. */
static double score_key(const orc_shape* S, const uint16_t* qrow, const float* wrow,
                        const void* k, const float* k_scale, int64_t b, int64_t s) {
    double total = 0.0;
    for (int64_t h = 0; h < S->heads; ++h) {
        const uint16_t* qh = qrow + h * S->dim;
        double x = 0.0;
        if (S->key_fp8) {
            const uint8_t* kc = (const uint8_t*)k + (b * S->n_k + s) * S->dim;
            for (int64_t d = 0; d < S->dim; ++d)
                x += orc_bf16_to_double(qh[d]) * orc_e4m3fn_to_double(kc[d]);
            x *= (double)k_scale[b * S->n_k + s];
        } else {
            const uint16_t* kr = (const uint16_t*)k + (b * S->n_k + s) * S->dim;
            for (int64_t d = 0; d < S->dim; ++d)
                x += orc_bf16_to_double(qh[d]) * orc_bf16_to_double(kr[d]);
        }
        double relu = x > 0.0 ? x : 0.0;
        total += (double)wrow[h] * relu;
    }
    return total + 0.0;
}

/* Same indexer on a pooled block representative (bf16 bits, [dim]). */
static double score_pooled(const orc_shape* S, const uint16_t* qrow, const float* wrow,
                           const uint16_t* kbar) {
    double total = 0.0;
    for (int64_t h = 0; h < S->heads; ++h) {
        const uint16_t* qh = qrow + h * S->dim;
        double x = 0.0;
        for (int64_t d = 0; d < S->dim; ++d)
            x += orc_bf16_to_double(qh[d]) * orc_bf16_to_double(kbar[d]);
        double relu = x > 0.0 ? x : 0.0;
        total += (double)wrow[h] * relu;
    }
    return total + 0.0;
}

/* Scores of a rectangle of (query, key) pairs; pairs a query cannot see
 * get -inf.  out: [batch, q_count, k_count]. */
int orc_index_scores(const orc_shape* S, const uint16_t* q, const float* w, const void* k,
                     const float* k_scale, int32_t q_begin, int32_t q_count, int32_t k_begin,
                     int32_t k_count, double* out) {
    if (check_shape(S) || q_begin < 0 || q_count < 0 || k_begin < 0 || k_count < 0 ||
        (int64_t)q_begin + q_count > S->n_q || (int64_t)k_begin + k_count > S->n_k)
        return -1;
    const int64_t n = (int64_t)S->batch * q_count;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
        int64_t b = i / q_count, t = q_begin + i % q_count;
        int64_t nv = orc_n_visible(S, t);
        for (int64_t j = 0; j < k_count; ++j) {
            int64_t s = k_begin + j;
            const int64_t row = b * S->n_q + t;
            out[i * k_count + j] =
                s < nv ? score_key(S, q + row * S->heads * S->dim, w + row * S->heads, k, k_scale,
                                   b, s)
                       : -INFINITY;
        }
    }
    return 0;
}

/* Scores of every key for the listed rows (q / w hold those rows only);
 * keys a query cannot see get -inf.  out: [n_rows, n_k]. */
int orc_row_scores(const orc_shape* S, const uint16_t* q, const float* w, const void* k,
                   const float* k_scale, const int64_t* rows, int64_t n_rows, double* out);

/* --------------------------------------------------------------- ordering */

typedef struct {
    double score;
    int64_t index;
} orc_entry;

/* Score descending, then index ascending: a total order on distinct indices. */
static int entry_before(const void* pa, const void* pb) {
    const orc_entry* a = (const orc_entry*)pa;
    const orc_entry* b = (const orc_entry*)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->index < b->index) ? -1 : (a->index > b->index);
}

/* Sort the n candidates and write the first min(k, n) to idx/val, pad -1 / NaN. */
static void emit_topk(orc_entry* cand, int64_t n, int32_t topk, int32_t* idx, double* val) {
    qsort(cand, (size_t)n, sizeof(orc_entry), entry_before);
    for (int32_t j = 0; j < topk; ++j) {
        if (j < n) {
            idx[j] = (int32_t)cand[j].index;
            if (val) val[j] = cand[j].score;
        } else {
            idx[j] = -1;
            if (val) val[j] = NAN;
        }
    }
}

/* Row ids are flat (b * n_q + t). */
static int check_rows(const orc_shape* S, const int64_t* rows, int64_t n_rows) {
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= (int64_t)S->batch * S->n_q) return -1;
    return 0;
}

int orc_row_scores(const orc_shape* S, const uint16_t* q, const float* w, const void* k,
                   const float* k_scale, const int64_t* rows, int64_t n_rows, double* out) {
    if (check_shape(S) || check_rows(S, rows, n_rows)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t b = rows[i] / S->n_q, t = rows[i] % S->n_q;
        int64_t nv = orc_n_visible(S, t);
        for (int64_t s = 0; s < S->n_k; ++s)
            out[i * S->n_k + s] = s < nv ? score_key(S, q + i * S->heads * S->dim,
                                                     w + i * S->heads, k, k_scale, b, s)
                                         : -INFINITY;
    }
    return 0;
}

/* Flat (DSA-style) top-k for the listed rows.  q / w hold the listed rows
 * only (q: [n_rows, heads, dim] bf16 bits, w: [n_rows, heads]).
 * idx: [n_rows, topk] int32; val: [n_rows, topk] double or NULL. */
int orc_topk_flat(const orc_shape* S, const uint16_t* q, const float* w, const void* k,
                  const float* k_scale, int32_t topk, const int64_t* rows, int64_t n_rows,
                  int32_t* idx, double* val) {
    if (check_shape(S) || topk <= 0 || check_rows(S, rows, n_rows)) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t b = rows[i] / S->n_q, t = rows[i] % S->n_q;
        int64_t nv = orc_n_visible(S, t);
        orc_entry* cand = (orc_entry*)malloc(sizeof(orc_entry) * (size_t)(nv > 0 ? nv : 1));
        if (!cand) {
            bad = 1;
            continue;
        }
        for (int64_t s = 0; s < nv; ++s) {
            cand[s].score = score_key(S, q + i * S->heads * S->dim, w + i * S->heads, k, k_scale,
                                      b, s);
            cand[s].index = s;
        }
        emit_topk(cand, nv, topk, idx + i * topk, val ? val + i * topk : NULL);
        free(cand);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------- HISA */

/* Mean-pool complete blocks: pooled [batch, n_k / block, dim] bf16 bits. */
int orc_pool(const orc_shape* S, const void* k, const float* k_scale, int32_t block,
             uint16_t* pooled) {
    if (check_shape(S) || block <= 0) return -1;
    const int64_t nb = S->n_k / block;
    const int64_t n = (int64_t)S->batch * nb;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        int64_t b = i / nb, j = i % nb;
        for (int64_t d = 0; d < S->dim; ++d) {
            double sum = 0.0;
            for (int64_t s = j * block; s < (j + 1) * block; ++s)
                sum += key_value(S, k, k_scale, b, s, d);
            pooled[i * S->dim + d] = orc_double_to_bf16(sum / (double)block);
        }
    }
    return 0;
}

/* Local block of query t (the block holding its last visible key), or -1. */
static int64_t local_block(const orc_shape* S, int64_t t, int32_t block) {
    int64_t nv = orc_n_visible(S, t);
    return nv > 0 ? (nv - 1) / block : -1;
}

/* Kept blocks of one row, ascending; returns the count (<= m_total). */
static int64_t select_blocks_row(const orc_shape* S, const uint16_t* qrow, const float* wrow,
                                 const uint16_t* pooled, int32_t block, int32_t m_scored,
                                 uint32_t flags, int64_t row, int64_t* kept, double* kept_val) {
    int64_t b = row / S->n_q, t = row % S->n_q;
    int64_t L = local_block(S, t, block);
    if (L < 0) return 0;
    const int64_t nb = S->n_k / block;
    int first_forced = (flags & ORC_FORCE_FIRST) && L > 0;
    /* scored candidates: complete blocks strictly before the local block */
    int64_t n_el = 0;
    orc_entry* cand = (orc_entry*)malloc(sizeof(orc_entry) * (size_t)(L > 0 ? L : 1));
    for (int64_t j = first_forced ? 1 : 0; j < L; ++j) {
        cand[n_el].score = score_pooled(S, qrow, wrow, pooled + (b * nb + j) * S->dim);
        cand[n_el].index = j;
        ++n_el;
    }
    qsort(cand, (size_t)n_el, sizeof(orc_entry), entry_before);
    int64_t take = n_el < m_scored ? n_el : m_scored;
    int64_t n = 0;
    if (first_forced) {
        kept[n] = 0;
        kept_val[n] = INFINITY;
        ++n;
    }
    for (int64_t i = 0; i < take; ++i) {
        kept[n] = cand[i].index;
        kept_val[n] = cand[i].score;
        ++n;
    }
    if (flags & ORC_FORCE_LOCAL) {
        kept[n] = L;
        kept_val[n] = INFINITY;
        ++n;
    }
    free(cand);
    /* ascending block order (insertion sort; n <= m_total) */
    for (int64_t i = 1; i < n; ++i) {
        int64_t kb = kept[i];
        double kv = kept_val[i];
        int64_t j = i - 1;
        while (j >= 0 && kept[j] > kb) {
            kept[j + 1] = kept[j];
            kept_val[j + 1] = kept_val[j];
            --j;
        }
        kept[j + 1] = kb;
        kept_val[j + 1] = kv;
    }
    return n;
}

static int popcount2(uint32_t f) { return (int)((f & 1u) + ((f >> 1) & 1u)); }

/* Block selection for the listed rows (q / w hold those rows only).
 * blk: [n_rows, m_total] ascending, -1 padded; blk_val (or NULL): block
 * scores, +inf for forced blocks. */
int orc_block_select(const orc_shape* S, const uint16_t* q, const float* w,
                     const uint16_t* pooled, int32_t block, int32_t m_scored, uint32_t flags,
                     const int64_t* rows, int64_t n_rows, int32_t m_total, int32_t* blk,
                     double* blk_val) {
    if (check_shape(S) || block <= 0 || m_scored < 0 || (flags & ~3u) ||
        m_total != m_scored + popcount2(flags) || m_total <= 0 || check_rows(S, rows, n_rows))
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t kept[m_total];
        double kv[m_total];
        int64_t n = select_blocks_row(S, q + i * S->heads * S->dim, w + i * S->heads, pooled,
                                      block, m_scored, flags, rows[i], kept, kv);
        for (int64_t j = 0; j < m_total; ++j) {
            blk[i * m_total + j] = j < n ? (int32_t)kept[j] : -1;
            if (blk_val) blk_val[i * m_total + j] = j < n ? kv[j] : NAN;
        }
    }
    return 0;
}

/* Token-level refinement inside the given blocks (blk: [n_rows, m_total],
 * entries -1 are ignored).  q / w / idx / val as for orc_topk_flat. */
int orc_refine(const orc_shape* S, const uint16_t* q, const float* w, const void* k,
               const float* k_scale, int32_t block, const int32_t* blk, int32_t m_total,
               int32_t topk, const int64_t* rows, int64_t n_rows, int32_t* idx, double* val) {
    if (check_shape(S) || block <= 0 || m_total <= 0 || topk <= 0 || check_rows(S, rows, n_rows))
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t b = rows[i] / S->n_q, t = rows[i] % S->n_q;
        int64_t nv = orc_n_visible(S, t);
        orc_entry* cand = (orc_entry*)malloc(sizeof(orc_entry) * (size_t)m_total * block + 1);
        if (!cand) {
            bad = 1;
            continue;
        }
        int64_t n = 0;
        for (int64_t j = 0; j < m_total; ++j) {
            int64_t bj = blk[i * m_total + j];
            if (bj < 0) continue;
            /* a block listed twice is scored once */
            int dup = 0;
            for (int64_t jj = 0; jj < j; ++jj)
                if (blk[i * m_total + jj] == bj) dup = 1;
            if (dup) continue;
            for (int64_t s = bj * block; s < (bj + 1) * block && s < nv; ++s) {
                cand[n].score = score_key(S, q + i * S->heads * S->dim, w + i * S->heads, k,
                                          k_scale, b, s);
                cand[n].index = s;
                ++n;
            }
        }
        emit_topk(cand, n, topk, idx + i * topk, val ? val + i * topk : NULL);
        free(cand);
    }
    return bad ? -2 : 0;
}

/* Whole HISA indexer for the listed rows (q / w hold those rows only):
 * pool, select, refine.  blk: [n_rows, m_scored + forced count]. */
int orc_hisa(const orc_shape* S, const uint16_t* q, const float* w, const void* k,
             const float* k_scale, int32_t block, int32_t m_scored, uint32_t flags,
             int32_t topk, const int64_t* rows, int64_t n_rows, int32_t* blk, int32_t* idx,
             double* val) {
    if (check_shape(S) || block <= 0) return -1;
    const int32_t m_total = m_scored + popcount2(flags);
    const int64_t nb = S->n_k / block;
    uint16_t* pooled = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(S->batch * nb * S->dim + 1));
    if (!pooled) return -2;
    int rc = orc_pool(S, k, k_scale, block, pooled);
    if (!rc)
        rc = orc_block_select(S, q, w, pooled, block, m_scored, flags, rows, n_rows, m_total,
                              blk, NULL);
    if (!rc)
        rc = orc_refine(S, q, w, k, k_scale, block, blk, m_total, topk, rows, n_rows, idx, val);
    free(pooled);
    return rc;
}

/* ------------------------------------------------------- key compression */

/* Compress raw bf16 keys [batch, n_raw, dim] (ratio m = S->causal_ratio):
 * the n_raw / m complete groups give keys 0 .. n_raw/m - 1 of the cache
 * k [batch, S->n_k, dim] (bf16 bits, or e4m3fn codes with k_scale
 * [batch, S->n_k] when S->key_fp8).  Cache slots past n_raw / m are not
 * written. */
int orc_compress_keys(const orc_shape* S, const uint16_t* raw, int64_t n_raw, void* k,
                      float* k_scale) {
    if (check_shape(S) || n_raw < 0 || n_raw / S->causal_ratio > S->n_k) return -1;
    const int64_t m = S->causal_ratio, D = S->dim;
    const int64_t nc = n_raw / m;
    const int64_t n = (int64_t)S->batch * nc;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const int64_t b = i / nc, j = i % nc;
        const int64_t out = b * S->n_k + j;
        uint16_t kc[D];
        for (int64_t d = 0; d < D; ++d) {
            double sum = 0.0;
            for (int64_t r = 0; r < m; ++r)
                sum += orc_bf16_to_double(raw[(b * n_raw + m * j + r) * D + d]);
            kc[d] = orc_double_to_bf16(sum / (double)m);
        }
        if (!S->key_fp8) {
            memcpy((uint16_t*)k + out * D, kc, sizeof(uint16_t) * (size_t)D);
            continue;
        }
        float amax = 0.0f;
        for (int64_t d = 0; d < D; ++d) {
            float v = fabsf((float)orc_bf16_to_double(kc[d]));
            if (v > amax) amax = v;
        }
        const float scale = amax / 448.0f;
        const float div = scale > 0.0f ? scale : 1.0f;
        for (int64_t d = 0; d < D; ++d)
            ((uint8_t*)k)[out * D + d] = orc_float_to_e4m3fn((float)orc_bf16_to_double(kc[d]) / div);
        k_scale[out] = scale;
    }
    return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
