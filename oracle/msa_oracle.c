/*
 * Plain CPU oracle for the decode-time sparse-attention block indexer
 * (score plane -> per-row Top16 select -> merge of split-column Top16 lists).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously-correct definition
 * that the HIP library is checked against. Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg load it. It shares no source, header, table
 * or helper with the HIP library, and the library never loads it.
 *
 * Sources (FlashInfer msa_ops API pages):
 *   [P1] "flashinfer.msa_ops.msa_icp_decode_index_score_sharded": description
 *        (written columns), index_q (token positions), index_k, block_table,
 *        seq_lens, score_out (cols limits), page_size limits.
 *   [P2] "flashinfer.msa_ops.prepare_msa_icp_indexer": decode chain
 *        (score plane -> Top16 select -> owner merge); the prefill chain
 *        (window plan -> per-chunk scoring and select -> merge);
 *        init_blocks/local_blocks (forced begin/end blocks, sum at most 16).
 *   [P3] "flashinfer.msa_ops.msa_icp_topk_select_publish": description (the
 *        row format: sixteen unscaled scores with increasing block ids; all
 *        rows are written on each call, padding rows too); scores (K limit);
 *        num_valid_pages (a count of global B128 blocks).
 *   OCP 8-bit Floating Point Specification (OFP8), E4M3 format: bias 7, no
 *        infinities, S.1111.111 is NaN, exponent field 0 is subnormal.
 *
 * Readings where the pages leave a step open (both the oracle and the GPU path
 * use them):
 *   - block score = max over the block's keys at positions <= the token's
 *     position of the raw q.k dot product; a block with no such key scores -inf;
 *   - ranking = score descending, then lower block id; -0 and +0 compare equal;
 *   - the Top16 row lists its entries by ascending id; unused slots hold
 *     (score -inf, id -1);
 *   - forced blocks of a row are [0, init) and [n - local, n) intersected with
 *     the row's valid ids [0, n), n = num_valid_pages of the token.
 *
 * Arithmetic: every finite e4m3fn value is an integer multiple of 2^-9 of
 * magnitude <= 448 = 229376 * 2^-9 < 2^18 * 2^-9. A product is then an integer
 * multiple of 2^-18 below 2^36 units and a 128-term sum stays below 2^43 units,
 * so dot products are accumulated exactly in int64 and rounded once to float32
 * (round to nearest even) at the end.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DIM 128   /* index head dimension [P1 index_q / index_k] */
#define ORACLE_HEADS 4   /* index heads [P1 index_q; P2 num_index_heads] */
#define ORACLE_BLOCK 128 /* keys per B128 block [P1 description; P3 num_valid_pages] */
#define ORACLE_TOPK 16   /* Top16 row width [P3 description] */

typedef struct {
    float score[ORACLE_TOPK];
    int32_t id[ORACLE_TOPK];
} oracle_row;

/* ------------------------------------------------------------------------ */
/* E4M3FN decode (OCP OFP8 E4M3), built once into a 256-entry table.          */
/* ------------------------------------------------------------------------ */

static int g_table_ready = 0;
static int64_t g_units[256];   /* value in units of 2^-9 (finite codes)      */
static double g_value[256];    /* value as a double (NaN for the NaN codes)  */
static int g_is_nan[256];

static void build_e4m3fn_table(void)
{
    for (int code = 0; code < 256; ++code) {
        int sign = (code >> 7) & 1;
        int exponent = (code >> 3) & 0xF;
        int mantissa = code & 0x7;
        int64_t magnitude_units;
        if (exponent == 0xF && mantissa == 0x7) {
            /* S.1111.111 is the only NaN encoding; there are no infinities. */
            g_is_nan[code] = 1;
            g_units[code] = 0;
            g_value[code] = NAN;
            continue;
        }
        if (exponent == 0) {
            /* subnormal: (mantissa / 8) * 2^(1 - 7) = mantissa * 2^-9 */
            magnitude_units = mantissa;
        } else {
            /* normal: (1 + mantissa / 8) * 2^(exponent - 7)
             *       = (8 + mantissa) * 2^(exponent - 10)
             *       = (8 + mantissa) * 2^(exponent - 1) units of 2^-9 */
            magnitude_units = (int64_t)(8 + mantissa) << (exponent - 1);
        }
        g_is_nan[code] = 0;
        g_units[code] = sign ? -magnitude_units : magnitude_units;
        g_value[code] = ldexp((double)magnitude_units, -9);
        if (sign)
            g_value[code] = -g_value[code];  /* keeps -0.0 for code 0x80 */
    }
    g_table_ready = 1;
}

static void ensure_table(void)
{
    if (!g_table_ready)
        build_e4m3fn_table();
}

/* Fills values[256] with the decoded e4m3fn value of every byte code. */
void oracle_e4m3fn_table(double* values)
{
    ensure_table();
    for (int c = 0; c < 256; ++c)
        values[c] = g_value[c];
}

/* ------------------------------------------------------------------------ */
/* One dot product, exact. [P1 index_q, index_k: fp8 e4m3fn rows of 128]     */
/* ------------------------------------------------------------------------ */

/* Returns sum_i q[i]*k[i] in units of 2^-18 (exact); *abs_units receives
 * sum_i |q[i]*k[i]| in the same units. Sets *has_nan if either row holds a
 * NaN code. */
static int64_t dot_units(const uint8_t* q, const uint8_t* k, int64_t* abs_units, int* has_nan)
{
    int64_t acc = 0, acc_abs = 0;
    int nan = 0;
    for (int i = 0; i < ORACLE_DIM; ++i) {
        int64_t prod = g_units[q[i]] * g_units[k[i]];
        acc += prod;
        acc_abs += prod < 0 ? -prod : prod;
        nan |= g_is_nan[q[i]] | g_is_nan[k[i]];
    }
    if (abs_units)
        *abs_units = acc_abs;
    if (has_nan)
        *has_nan = nan;
    return acc;
}

/* units of 2^-18 -> float32, rounded once (the double is exact: |x| < 2^53). */
static float units_to_float(int64_t units)
{
    return (float)ldexp((double)units, -18);
}

/* Batched single dot products: out_f32[i] = fp32(q_i . k_i) rounded once,
 * out_exact[i] = the exact value as a double (exact, see file header). */
void oracle_dots(const uint8_t* q, const uint8_t* k, int64_t n, float* out_f32, double* out_exact)
{
    ensure_table();
    for (int64_t i = 0; i < n; ++i) {
        int nan = 0;
        int64_t u = dot_units(q + i * ORACLE_DIM, k + i * ORACLE_DIM, NULL, &nan);
        out_f32[i] = nan ? NAN : units_to_float(u);
        out_exact[i] = nan ? NAN : ldexp((double)u, -18);
    }
}

/* Threads the plane functions may use (OpenMP), for reporting. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads later plane calls may use (OpenMP); n >= 1. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Score plane.                                                              */
/* ------------------------------------------------------------------------ */

/* Number of written columns of a request: its ceil(seq_len / 128) B128 blocks
 * rounded up to a multiple of four [P1 description]. With every page's full
 * rows on one device, a column is one global B128 block at both page sizes;
 * at page_size 256 each page holds two blocks and
 * roundup4(ceil(s/128)) == roundup4(2*ceil(s/256)) for every s, so counting
 * two blocks per page of the request gives the same padded count. */
int64_t oracle_written_columns(int64_t seq_len)
{
    if (seq_len <= 0)
        return 0;
    int64_t blocks = (seq_len + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    return (blocks + 3) / 4 * 4;
}

/* Key p is visible to a token at position pos of a request of seq_len keys
 * when p < seq_len and p <= pos [P1 index_q: the token's position]. */
static int key_visible(int64_t p, int64_t seq_len, int64_t pos)
{
    return p < seq_len && p <= pos;
}

/* Folds one visible key into a block's running maximum: best holds the max
 * exact dot product, best_abs the max sum |q_i k_i| (both in 2^-18 units). */
static void take_key(const uint8_t* q_row, const uint8_t* key, int* have, int64_t* best,
                     int64_t* best_abs)
{
    int64_t abs_units = 0;
    int64_t u = dot_units(q_row, key, &abs_units, NULL);
    if (!*have || u > *best)
        *best = u;
    if (!*have || abs_units > *best_abs)
        *best_abs = abs_units;
    *have = 1;
}

/* Score of one plane element [P1 description, index_q, index_k, block_table]:
 * q_row is the token's 128-byte head row, pos its position
 * (seq_len - decode_query_len + j). Column c covers keys [128c, 128c + 128);
 * key p lives at index_k[block_table_row[p / page_size], p % page_size, :].
 * Visible keys: p < seq_len and p <= pos.
 * *score = fp32(max visible dot) or -inf if no key is visible;
 * *amax  = max over visible keys of sum_i |q_i k_i| (0 if none).
 * Returns 0, or -1 if a needed block_table entry is outside [0, num_pages). */
int oracle_score_element(const uint8_t* q_row, const uint8_t* index_k, int64_t num_pages,
                         int32_t page_size, const int32_t* block_table_row, int64_t seq_len,
                         int64_t pos, int64_t c, float* score, double* amax)
{
    ensure_table();
    int have = 0, bad = 0;
    int64_t best = 0, best_abs = 0;
    for (int64_t p = c * ORACLE_BLOCK; p < (c + 1) * ORACLE_BLOCK; ++p) {
        if (!key_visible(p, seq_len, pos))
            continue;
        int64_t page = block_table_row[p / page_size];
        if (page < 0 || page >= num_pages) {
            bad = 1;
            continue;
        }
        take_key(q_row, index_k + ((page * page_size) + (p % page_size)) * ORACLE_DIM, &have,
                 &best, &best_abs);
    }
    *score = have ? units_to_float(best) : -INFINITY;
    if (amax)
        *amax = have ? ldexp((double)best_abs, -18) : 0.0;
    return bad ? -1 : 0;
}

/* The whole plane [P1]: for request b, token j, head h, column
 * c < min(written_columns(seq_len[b]), cols):
 *   score_out[(b*dql + j), h, c] = oracle_score_element(...)
 * Other columns are left as they are. amax_out (nullable) has the plane's
 * shape and receives the per-element amax for written columns.
 * Returns the number of elements that met an out-of-range block_table entry. */
int64_t oracle_score_decode(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                            const int32_t* block_table, int64_t block_table_stride,
                            const int32_t* seq_lens, int32_t batch, int32_t page_size,
                            int32_t decode_query_len, float* score_out, int32_t cols,
                            double* amax_out)
{
    ensure_table();
    int64_t bad = 0;
    int64_t rows = (int64_t)batch * decode_query_len * ORACLE_HEADS;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t row = 0; row < rows; ++row) {
        int64_t t = row / ORACLE_HEADS;
        int64_t b = t / decode_query_len;
        int64_t j = t % decode_query_len;
        int64_t seq_len = seq_lens[b];
        int64_t pos = seq_len - decode_query_len + j;
        int64_t written = oracle_written_columns(seq_len);
        if (written > cols)
            written = cols;
        const uint8_t* q_row = index_q + row * ORACLE_DIM;
        for (int64_t c = 0; c < written; ++c) {
            float s;
            double a;
            if (oracle_score_element(q_row, index_k, num_pages, page_size,
                                     block_table + b * block_table_stride, seq_len, pos, c,
                                     &s, &a) != 0)
                ++bad;
            score_out[row * cols + c] = s;
            if (amax_out)
                amax_out[row * cols + c] = a;
        }
    }
    return bad;
}

/* Sampled elements: for each i, element (row[i], col[i]) of the plane
 * (row = (b*dql + j)*4 + h). Same definition as oracle_score_decode. */
int64_t oracle_score_sampled(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                             const int32_t* block_table, int64_t block_table_stride,
                             const int32_t* seq_lens, int32_t page_size, int32_t decode_query_len,
                             const int64_t* sample_rows, const int64_t* sample_cols,
                             int64_t n_samples, float* score_out, double* amax_out)
{
    ensure_table();
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad)
    for (int64_t i = 0; i < n_samples; ++i) {
        int64_t row = sample_rows[i];
        int64_t t = row / ORACLE_HEADS;
        int64_t b = t / decode_query_len;
        int64_t j = t % decode_query_len;
        int64_t seq_len = seq_lens[b];
        int64_t pos = seq_len - decode_query_len + j;
        float s;
        double a;
        if (oracle_score_element(index_q + row * ORACLE_DIM, index_k, num_pages, page_size,
                                 block_table + b * block_table_stride, seq_len, pos,
                                 sample_cols[i], &s, &a) != 0)
            ++bad;
        score_out[i] = s;
        if (amax_out)
            amax_out[i] = a;
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Prefill score plane [P2 prefill chain; element definition of P1].         */
/* ------------------------------------------------------------------------ */

/* The prefill chain of [P2] scores a chunk of query tokens per request: the
 * query tokens of request b are rows [qo_indptr[b], qo_indptr[b+1]) of
 * index_q, q_len_b of them, and (as for decode tokens, [P1 index_q]) token j
 * of the chunk sits at position seq_len[b] - q_len_b + j, its own key being
 * the chunk's key at that position. Each element is the decode element:
 * column c of a token's head row is the maximum over the block's keys
 * p <= pos (p < seq_len) of the exact dot product, -inf if none, written for
 * c < min(written_columns(seq_len[b]), cols). With q_len_b = decode_query_len
 * for every request this is oracle_score_decode.
 *
 * tokens (nullable): the query-token rows to score, n_tokens of them; the
 * output then holds those tokens' rows [n_tokens, 4, cols] in that order.
 * With tokens == NULL every token of the chunk is scored (n_tokens ignored)
 * into [qo_indptr[batch], 4, cols]. Columns a token does not write are left
 * as they are. Returns the number of elements that met an out-of-range
 * block_table entry, or -1 if a token row is outside [0, qo_indptr[batch]) or
 * qo_indptr decreases. */
int64_t oracle_score_prefill(const uint8_t* index_q, const uint8_t* index_k, int64_t num_pages,
                             const int32_t* block_table, int64_t block_table_stride,
                             const int32_t* qo_indptr, const int32_t* seq_lens, int32_t batch,
                             int32_t page_size, const int64_t* tokens, int64_t n_tokens,
                             float* score_out, int32_t cols, double* amax_out)
{
    ensure_table();
    for (int32_t b = 0; b < batch; ++b)
        if (qo_indptr[b + 1] < qo_indptr[b] || qo_indptr[0] != 0)
            return -1;
    int64_t total = qo_indptr[batch];
    int64_t n_out = tokens ? n_tokens : total;
    for (int64_t i = 0; tokens && i < n_out; ++i)
        if (tokens[i] < 0 || tokens[i] >= total)
            return -1;
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t i = 0; i < n_out; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        int64_t b = 0;
        while (qo_indptr[b + 1] <= t)  /* the request whose chunk holds row t */
            ++b;
        int64_t q_len = qo_indptr[b + 1] - qo_indptr[b];
        int64_t j = t - qo_indptr[b];
        int64_t seq_len = seq_lens[b];
        int64_t pos = seq_len - q_len + j;
        int64_t written = oracle_written_columns(seq_len);
        if (written > cols)
            written = cols;
        for (int h = 0; h < ORACLE_HEADS; ++h) {
            const uint8_t* q_row = index_q + (t * ORACLE_HEADS + h) * ORACLE_DIM;
            int64_t out_row = i * ORACLE_HEADS + h;
            for (int64_t c = 0; c < written; ++c) {
                float sc;
                double a;
                if (oracle_score_element(q_row, index_k, num_pages, page_size,
                                         block_table + b * block_table_stride, seq_len, pos, c,
                                         &sc, &a) != 0)
                    ++bad;
                score_out[out_row * cols + c] = sc;
                if (amax_out)
                    amax_out[out_row * cols + c] = a;
            }
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Top16 select and merge [P3 description; P2 init_blocks/local_blocks].     */
/* ------------------------------------------------------------------------ */

typedef struct {
    float score;
    int32_t id;
} entry;

/* Ranking: higher score first; equal scores (-0 == +0 as floats) -> lower id. */
static int rank_cmp(const void* pa, const void* pb)
{
    const entry* a = (const entry*)pa;
    const entry* b = (const entry*)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->id > b->id) - (a->id < b->id);
}

static int id_cmp(const void* pa, const void* pb)
{
    const entry* a = (const entry*)pa;
    const entry* b = (const entry*)pb;
    return (a->id > b->id) - (a->id < b->id);
}

/* Forced begin/end blocks of a row with n valid blocks: [0, init) and
 * [n - local, n), both inside [0, n). */
static int is_forced(int64_t id, int64_t n, int32_t init_blocks, int32_t local_blocks)
{
    if (id < 0 || id >= n)
        return 0;
    return id < init_blocks || id >= n - local_blocks;
}

/* Keeps the forced entries and the best (16 - n_forced_total) of the others
 * by (score desc, id asc); writes them by ascending id, then pads with
 * (-inf, -1). `cand` is sorted in place. */
static void emit_row(entry* forced, int n_forced, int budget, entry* cand, int64_t n_cand,
                     oracle_row* out)
{
    entry chosen[ORACLE_TOPK];
    int m = 0;
    for (int i = 0; i < n_forced; ++i)
        chosen[m++] = forced[i];
    qsort(cand, (size_t)n_cand, sizeof(entry), rank_cmp);
    int64_t take = budget < n_cand ? budget : n_cand;
    for (int64_t i = 0; i < take; ++i)
        chosen[m++] = cand[i];
    qsort(chosen, (size_t)m, sizeof(entry), id_cmp);
    for (int i = 0; i < ORACLE_TOPK; ++i) {
        out->score[i] = i < m ? chosen[i].score : -INFINITY;
        out->id[i] = i < m ? chosen[i].id : -1;
    }
}

/* Columns per select range: w = ceil(cols / num_ranges). */
static int64_t range_width(int32_t cols, int32_t num_ranges)
{
    return ((int64_t)cols + num_ranges - 1) / num_ranges;
}

/* Top16 select of every (token, head, range) row [P3 description]:
 * scores [T, 4, cols]; range r covers columns [r*w, min((r+1)*w, cols)),
 * w = ceil(cols / num_ranges). Valid ids are [0, n), n = num_valid_pages[t]
 * clamped to [0, cols]. Forced ids of the range are kept, the rest ranked.
 * out: [T, 4, num_ranges] rows. Returns the number of tokens whose
 * num_valid_pages was outside [0, cols], or -1 for invalid arguments. */
int64_t oracle_top16_select(const float* scores, int32_t num_tokens, int32_t cols,
                            const int32_t* num_valid_pages, int32_t init_blocks,
                            int32_t local_blocks, int32_t num_ranges, oracle_row* out)
{
    if (init_blocks < 0 || local_blocks < 0 || init_blocks + local_blocks > ORACLE_TOPK ||
        num_ranges < 1 || cols < 1)
        return -1;
    int64_t width = range_width(cols, num_ranges);
    int64_t bad = 0;
    entry* cand = (entry*)malloc(sizeof(entry) * (size_t)(width > 0 ? width : 1));
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t n = num_valid_pages[t];
        if (n < 0 || n > cols) {
            ++bad;
            n = n < 0 ? 0 : cols;
        }
        for (int h = 0; h < ORACLE_HEADS; ++h) {
            const float* srow = scores + (t * ORACLE_HEADS + h) * (int64_t)cols;
            for (int32_t r = 0; r < num_ranges; ++r) {
                int64_t lo = r * width;
                int64_t hi = lo + width < cols ? lo + width : cols;
                int64_t valid_hi = hi < n ? hi : n;
                entry forced[ORACLE_TOPK];
                int n_forced = 0;
                int64_t n_cand = 0;
                for (int64_t id = lo; id < valid_hi; ++id) {
                    entry e = {srow[id], (int32_t)id};
                    if (is_forced(id, n, init_blocks, local_blocks))
                        forced[n_forced++] = e;
                    else
                        cand[n_cand++] = e;
                }
                emit_row(forced, n_forced, ORACLE_TOPK - n_forced, cand, n_cand,
                         out + (t * ORACLE_HEADS + h) * num_ranges + r);
            }
        }
    }
    free(cand);
    return bad;
}

/* Merge of R partial Top16 rows per (token, head) [P2 decode: owner merge]:
 * the union of the rows' entries (id >= 0; an id met twice keeps its higher
 * score), forced ids of [0, n) recomputed, the rest ranked as in select with
 * budget 16 - |forced of [0, n)|. partial: [T, 4, R]; out: [T, 4].
 * Returns the number of (token, head) rows in which a forced id was missing
 * from the union, or -1 for invalid arguments. */
int64_t oracle_top16_merge(const oracle_row* partial, int32_t num_tokens, int32_t num_ranges,
                           const int32_t* num_valid_pages, int32_t init_blocks,
                           int32_t local_blocks, oracle_row* out)
{
    if (init_blocks < 0 || local_blocks < 0 || init_blocks + local_blocks > ORACLE_TOPK ||
        num_ranges < 1)
        return -1;
    int64_t cap = (int64_t)num_ranges * ORACLE_TOPK;
    entry* all = (entry*)malloc(sizeof(entry) * (size_t)cap);
    entry* cand = (entry*)malloc(sizeof(entry) * (size_t)cap);
    int64_t missing_rows = 0;
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t n = num_valid_pages[t] < 0 ? 0 : num_valid_pages[t];
        for (int h = 0; h < ORACLE_HEADS; ++h) {
            const oracle_row* rows = partial + (t * ORACLE_HEADS + h) * num_ranges;
            int64_t n_all = 0;
            for (int32_t r = 0; r < num_ranges; ++r) {
                for (int s = 0; s < ORACLE_TOPK; ++s) {
                    if (rows[r].id[s] < 0)
                        continue;
                    int64_t k;
                    for (k = 0; k < n_all; ++k)
                        if (all[k].id == rows[r].id[s])
                            break;
                    if (k < n_all) {
                        if (rows[r].score[s] > all[k].score)
                            all[k].score = rows[r].score[s];
                    } else {
                        all[n_all].id = rows[r].id[s];
                        all[n_all].score = rows[r].score[s];
                        ++n_all;
                    }
                }
            }
            int64_t expected_forced = 0;
            for (int64_t id = 0; id < n; ++id)
                expected_forced += is_forced(id, n, init_blocks, local_blocks);
            entry forced[ORACLE_TOPK];
            int n_forced = 0;
            int64_t n_cand = 0;
            for (int64_t k = 0; k < n_all; ++k) {
                if (is_forced(all[k].id, n, init_blocks, local_blocks))
                    forced[n_forced++] = all[k];
                else
                    cand[n_cand++] = all[k];
            }
            if (n_forced != expected_forced)
                ++missing_rows;
            emit_row(forced, n_forced, ORACLE_TOPK - (int)expected_forced, cand, n_cand,
                     out + t * ORACLE_HEADS + h);
        }
    }
    free(all);
    free(cand);
    return missing_rows;
}

/* ------------------------------------------------------------------------ */
/* Row-sharded scoring and the column -> global id mapping                   */
/* [P1 description, index_k, rank/world_size, Layout].                        */
/* ------------------------------------------------------------------------ */

/* Written columns of a request on one rank of a row-sharded cache: the
 * request's ceil(seq_len / page_size) pages rounded up to a multiple of four
 * [P1 description]. */
int64_t oracle_written_columns_sharded(int64_t seq_len, int32_t page_size)
{
    if (seq_len <= 0)
        return 0;
    int64_t pages = (seq_len + page_size - 1) / page_size;
    return (pages + 3) / 4 * 4;
}

/* One element of rank `rank`'s plane. The rank holds rows
 * [rank * R, rank * R + R) of every page, R = page_size / world_size, as
 * index_k_shard [num_pages, R, 128] [P1 index_k]. Column c is page c of the
 * request (at page_size 128 that page is global B128 block c; at 256 the
 * rank's rows lie in global block 2c + rank * 2 / world_size [P1
 * description]), so its keys here are p = c * page_size + rank * R + i,
 * i < R, read from index_k_shard[block_table_row[c], i, :]. Visible keys,
 * value and amax as in oracle_score_element. */
int oracle_score_element_sharded(const uint8_t* q_row, const uint8_t* index_k_shard,
                                 int64_t num_pages, int32_t page_size, int32_t rank,
                                 int32_t world_size, const int32_t* block_table_row,
                                 int64_t seq_len, int64_t pos, int64_t c, float* score,
                                 double* amax)
{
    ensure_table();
    const int64_t rows = page_size / world_size;
    int have = 0, bad = 0;
    int64_t best = 0, best_abs = 0;
    for (int64_t i = 0; i < rows; ++i) {
        int64_t p = c * page_size + (int64_t)rank * rows + i;
        if (!key_visible(p, seq_len, pos))
            continue;
        int64_t page = block_table_row[c];
        if (page < 0 || page >= num_pages) {
            bad = 1;
            continue;
        }
        take_key(q_row, index_k_shard + (page * rows + i) * ORACLE_DIM, &have, &best,
                 &best_abs);
    }
    *score = have ? units_to_float(best) : -INFINITY;
    if (amax)
        *amax = have ? ldexp((double)best_abs, -18) : 0.0;
    return bad ? -1 : 0;
}

/* Rank `rank`'s whole plane: columns c < min(written_columns_sharded, cols)
 * of every (token, head) row, others untouched. Returns the number of
 * elements that met an out-of-range block_table entry, or -1 for invalid
 * arguments (world_size must divide page_size, 0 <= rank < world_size). */
int64_t oracle_score_decode_sharded(const uint8_t* index_q, const uint8_t* index_k_shard,
                                    int64_t num_pages, const int32_t* block_table,
                                    int64_t block_table_stride, const int32_t* seq_lens,
                                    int32_t batch, int32_t page_size, int32_t decode_query_len,
                                    int32_t rank, int32_t world_size, float* score_out,
                                    int32_t cols, double* amax_out)
{
    if (world_size < 1 || page_size % world_size != 0 || rank < 0 || rank >= world_size)
        return -1;
    ensure_table();
    int64_t bad = 0;
    int64_t rows = (int64_t)batch * decode_query_len * ORACLE_HEADS;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t row = 0; row < rows; ++row) {
        int64_t t = row / ORACLE_HEADS;
        int64_t b = t / decode_query_len;
        int64_t j = t % decode_query_len;
        int64_t seq_len = seq_lens[b];
        int64_t pos = seq_len - decode_query_len + j;
        int64_t written = oracle_written_columns_sharded(seq_len, page_size);
        if (written > cols)
            written = cols;
        const uint8_t* q_row = index_q + row * ORACLE_DIM;
        for (int64_t c = 0; c < written; ++c) {
            float s;
            double a;
            if (oracle_score_element_sharded(q_row, index_k_shard, num_pages, page_size, rank,
                                             world_size, block_table + b * block_table_stride,
                                             seq_len, pos, c, &s, &a) != 0)
                ++bad;
            score_out[row * cols + c] = s;
            if (amax_out)
                amax_out[row * cols + c] = a;
        }
    }
    return bad;
}

/* Top16 select with plane column c standing for global block id
 * index_scale * c + index_offset (index_scale >= 1, index_offset >= 0): the
 * select rule of oracle_top16_select applied to the global ids, so validity
 * (id < n), the forced ids and the tie order are all taken on global ids and
 * the rows list global ids. n outside [0, index_scale * cols + index_offset]
 * is counted and clamped. With index_scale 1 and index_offset 0 this is
 * oracle_top16_select. Returns the count, or -1 for invalid arguments. */
int64_t oracle_top16_select_mapped(const float* scores, int32_t num_tokens, int32_t cols,
                                   const int32_t* num_valid_pages, int32_t init_blocks,
                                   int32_t local_blocks, int32_t num_ranges, int32_t index_scale,
                                   int32_t index_offset, oracle_row* out)
{
    if (init_blocks < 0 || local_blocks < 0 || init_blocks + local_blocks > ORACLE_TOPK ||
        num_ranges < 1 || cols < 1 || index_scale < 1 || index_offset < 0)
        return -1;
    int64_t width = range_width(cols, num_ranges);
    int64_t n_max = (int64_t)index_scale * cols + index_offset;
    int64_t bad = 0;
    entry* cand = (entry*)malloc(sizeof(entry) * (size_t)(width > 0 ? width : 1));
    for (int64_t t = 0; t < num_tokens; ++t) {
        int64_t n = num_valid_pages[t];
        if (n < 0 || n > n_max) {
            ++bad;
            n = n < 0 ? 0 : n_max;
        }
        for (int h = 0; h < ORACLE_HEADS; ++h) {
            const float* srow = scores + (t * ORACLE_HEADS + h) * (int64_t)cols;
            for (int32_t r = 0; r < num_ranges; ++r) {
                int64_t lo = r * width;
                int64_t hi = lo + width < cols ? lo + width : cols;
                entry forced[ORACLE_TOPK];
                int n_forced = 0;
                int64_t n_cand = 0;
                for (int64_t c = lo; c < hi; ++c) {
                    int64_t id = (int64_t)index_scale * c + index_offset;
                    if (id >= n)
                        continue;
                    entry e = {srow[c], (int32_t)id};
                    if (is_forced(id, n, init_blocks, local_blocks))
                        forced[n_forced++] = e;
                    else
                        cand[n_cand++] = e;
                }
                emit_row(forced, n_forced, ORACLE_TOPK - n_forced, cand, n_cand,
                         out + (t * ORACLE_HEADS + h) * num_ranges + r);
            }
        }
    }
    free(cand);
    return bad;
}
