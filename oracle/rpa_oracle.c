/*
 * CPU oracle for ragged paged attention.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The GPU library never links, includes or calls it, and the
 * two share no code: no headers, helpers, tables or constants.
 *
 * Everything below is the plain definition written out with scalar loops and
 * fp64 arithmetic.  Cache, query and new-token values are bfloat16 bit patterns
 * held in uint16_t; widening bf16 to double is exact.
 *
 *   oracle_write_kv       scatter of each new token's K/V row into its page slot
 *                         (ONNX Runtime PR 31727 "[WebGPU] Optimized PagedAttention
 *                         implementation (2/n)", commit note of Phase 1b.1, the
 *                         scatter program; causal alignment from the same page's
 *                         note on the seqlens_q input of FlashAttention).
 *   oracle_attention      per query row: gather the visible keys through the block
 *                         table, then softmax attention (Ragged Paged Attention card,
 *                         "Key ideas": causal GQA over ragged paged KV; the same PR's
 *                         "What's shipped" for packed varlen Q and past-aware masking).
 *   oracle_union_tables   Q-block union, then intra-group union, then ascending
 *                         compaction into per-KV-head tables (CompactAttention page,
 *                         "Core claim" and Figure 3; KV-head-major pages, Figure 4).
 *   oracle_rotary_qkv     rotary embedding of new Q and K rows taken from packed or
 *                         separate Q/K/V, then the K/V scatter (ONNX Runtime PR, the rotary
 *                         program of Phase 1b.2: rotate Q and K before the scatter,
 *                         position = past + local token, dims from rotary_dim on copied,
 *                         V not rotated, interleaved or split pairs; and the packed-QKV
 *                         commit: per token, columns [0, Hq*D) are Q, then Hkv*D of K, then
 *                         Hkv*D of V).  Pair (x1, x2) at position p and pair index i becomes
 *                         (x1 cos - x2 sin, x2 cos + x1 sin) with cos = cos_cache[p][i],
 *                         sin = sin_cache[p][i] (fp32 tables [max_position][rotary_dim/2]);
 *                         interleaved pairs are dims (2i, 2i+1), split pairs (i, i + rd/2).
 *                         Each output is fmaf(x1, cos, -(x2 * sin)), resp.
 *                         fmaf(x2, cos, x1 * sin), in fp32, rounded to bf16 (nearest even).
 *   oracle_fp8_encode, oracle_fp8_decode, oracle_write_kv_fp8, oracle_attention_fp8
 *                         the quantized KV cache that the ONNX Runtime PR lists among
 *                         its deferred items ("Quantized KV cache (T_CACHE)") without
 *                         fixing a format.  Reading taken here: FP8 E4M3 of the OCP
 *                         8-bit floating point specification (bias 7, no infinities,
 *                         S.1111.111 is NaN, largest finite 448), one scale per cache
 *                         tensor: stored value = code value * scale.  A new K/V value x
 *                         (bf16) is stored as encode(float(x) * float(1 / scale)), the
 *                         product and the reciprocal rounded to fp32, the result
 *                         clamped to +-448 and rounded to nearest, ties to even.
 *
 * Layouts (all row-major):
 *   layout 0, sequence-major:  cache [P][S][Hkv][D]; tables [B][max_pages];
 *                              kv_lens [B].
 *   layout 1, KV-head-major:   cache [P][S][D] (one page holds one KV head);
 *                              tables [B][Hkv][max_pages]; kv_lens [B][Hkv].
 *   q and out: [T][Hq][D];  k_new, v_new: [T][Hkv][D];  cu_q_lens: [B+1].
 *
 * kv_len counts every key of the sequence including the new tokens; the new
 * tokens are the last q_len positions, so token t of sequence b sits at position
 * past_b + t with past_b = kv_len_b - q_len_b and sees keys 0 .. past_b + t.
 * Query head h reads KV head h / (Hq / Hkv).
 *
 * Return codes: 0 ok, 1 bad argument, 2 a block table entry outside [0, P).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* FP8 E4M3 code -> value: exponent field E, mantissa field M; E == 0 is subnormal
 * (M * 2^-9), otherwise (1 + M/8) * 2^(E-7); E == 15 with M == 7 is NaN. */
static double fp8_to_double(uint8_t c)
{
    int E = (c >> 3) & 15, M = c & 7;
    double v;
    if (E == 15 && M == 7)
        v = NAN;
    else if (E == 0)
        v = ldexp((double)M, -9);
    else
        v = ldexp(8.0 + M, E - 10);
    return (c & 0x80) ? -v : v;
}

/* value -> FP8 E4M3 code, clamped to +-448, rounded to nearest, ties to even.
 * Every scaling below is by a power of two, hence exact; nearbyint rounds ties to even
 * in the default rounding mode. */
static uint8_t fp8_from_float(float y)
{
    if (isnan(y))
        return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0;
    double a = fabs((double)y);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {                 /* subnormal range: steps of 2^-9 */
        int m = (int)nearbyint(ldexp(a, 9));   /* 0 .. 8; 8 is the smallest normal */
        return sign | (uint8_t)m;
    }
    int e2;
    frexp(a, &e2);                             /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                            /* a in [2^e, 2^(e+1)) */
    int r = (int)nearbyint(ldexp(a, 3 - e));   /* 8 .. 16 */
    if (r == 16) {
        r = 8;
        e += 1;
    }
    return sign | (uint8_t)(((e + 7) << 3) | (r - 8));
}

int oracle_fp8_encode(const float *y, uint8_t *codes, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        codes[i] = fp8_from_float(y[i]);
    return 0;
}

int oracle_fp8_decode(const uint8_t *codes, double *y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = fp8_to_double(codes[i]);
    return 0;
}

static float bf16_to_float(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Sequence index b with cu_q_lens[b] <= token < cu_q_lens[b+1] (linear scan). */
static int seq_of_token(int B, const int32_t *cu_q_lens, int64_t token)
{
    for (int b = 0; b < B; ++b)
        if (token >= cu_q_lens[b] && token < cu_q_lens[b + 1])
            return b;
    return -1;
}

static int32_t kv_len_of(const int32_t *kv_lens, int layout, int Hkv, int b, int g)
{
    return layout == 0 ? kv_lens[b] : kv_lens[(int64_t)b * Hkv + g];
}

static int32_t table_entry(const int32_t *tables, int layout, int Hkv, int max_pages,
                           int b, int g, int64_t logical_block)
{
    if (layout == 0)
        return tables[(int64_t)b * max_pages + logical_block];
    return tables[((int64_t)b * Hkv + g) * max_pages + logical_block];
}

/* Element offset of (page, slot, kv head) row start in the cache. */
static int64_t cache_row(int layout, int S, int Hkv, int D, int64_t page, int64_t slot, int g)
{
    if (layout == 0)
        return ((page * S + slot) * Hkv + g) * (int64_t)D;
    return (page * S + slot) * (int64_t)D;
}

/* kv8 == 0: caches of bf16, rows copied.  kv8 == 1: caches of FP8 codes, each value
 * stored as fp8_from_float(float(x) * inv_scale). */
static int write_kv_impl(int B, const int32_t *cu_q_lens, const int32_t *kv_lens,
                         int Hkv, int D, int S, int layout, int max_pages, int num_pages,
                         const int32_t *tables, const uint16_t *k_new, const uint16_t *v_new,
                         void *k_cache, void *v_cache, int kv8, float k_inv, float v_inv)
{
    if (B < 0 || Hkv <= 0 || D <= 0 || S <= 0 || (layout != 0 && layout != 1))
        return 1;
    for (int b = 0; b < B; ++b) {
        int q_len = cu_q_lens[b + 1] - cu_q_lens[b];
        for (int g = 0; g < Hkv; ++g) {
            int kv_len = kv_len_of(kv_lens, layout, Hkv, b, g);
            int past = kv_len - q_len;
            if (past < 0)
                return 1;
            for (int t = 0; t < q_len; ++t) {
                int64_t pos = (int64_t)past + t;
                int64_t logical = pos / S;
                if (logical >= max_pages)
                    return 1;
                int32_t page = table_entry(tables, layout, Hkv, max_pages, b, g, logical);
                if (page < 0 || page >= num_pages)
                    return 2;
                int64_t slot = pos % S;
                int64_t dst = cache_row(layout, S, Hkv, D, page, slot, g);
                int64_t src = ((int64_t)(cu_q_lens[b] + t) * Hkv + g) * D;
                for (int d = 0; d < D; ++d) {
                    if (kv8) {
                        ((uint8_t *)k_cache)[dst + d] = fp8_from_float(bf16_to_float(k_new[src + d]) * k_inv);
                        ((uint8_t *)v_cache)[dst + d] = fp8_from_float(bf16_to_float(v_new[src + d]) * v_inv);
                    } else {
                        ((uint16_t *)k_cache)[dst + d] = k_new[src + d];
                        ((uint16_t *)v_cache)[dst + d] = v_new[src + d];
                    }
                }
            }
        }
    }
    return 0;
}

int oracle_write_kv(int B, const int32_t *cu_q_lens, const int32_t *kv_lens,
                    int Hkv, int D, int S, int layout, int max_pages, int num_pages,
                    const int32_t *tables, const uint16_t *k_new, const uint16_t *v_new,
                    uint16_t *k_cache, uint16_t *v_cache)
{
    return write_kv_impl(B, cu_q_lens, kv_lens, Hkv, D, S, layout, max_pages, num_pages, tables,
                         k_new, v_new, k_cache, v_cache, 0, 1.0f, 1.0f);
}

/* FP8 caches: k_scale, v_scale > 0 are the caches' scales; the reciprocals are taken in fp32. */
int oracle_write_kv_fp8(int B, const int32_t *cu_q_lens, const int32_t *kv_lens,
                        int Hkv, int D, int S, int layout, int max_pages, int num_pages,
                        const int32_t *tables, const uint16_t *k_new, const uint16_t *v_new,
                        uint8_t *k_cache, uint8_t *v_cache, float k_scale, float v_scale)
{
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f))
        return 1;
    return write_kv_impl(B, cu_q_lens, kv_lens, Hkv, D, S, layout, max_pages, num_pages, tables,
                         k_new, v_new, k_cache, v_cache, 1, 1.0f / k_scale, 1.0f / v_scale);
}

/* Value d of a cache row: bf16, or FP8 code times the cache's scale. */
static double cache_value(const void *cache, int kv8, double scale, int64_t idx)
{
    if (kv8)
        return fp8_to_double(((const uint8_t *)cache)[idx]) * scale;
    return bf16_to_double(((const uint16_t *)cache)[idx]);
}

/* One query row (token, head): gather, scores, softmax, weighted sum of V. */
static int attend_row(int B, const int32_t *cu_q_lens, const int32_t *kv_lens,
                      int Hq, int Hkv, int D, int S, int layout, int max_pages, int num_pages,
                      const int32_t *tables, const uint16_t *q, const void *k_cache,
                      const void *v_cache, int kv8, double k_scale, double v_scale,
                      double scale, const uint8_t *block_allowed,
                      int64_t token, int h, double *o)
{
    int b = seq_of_token(B, cu_q_lens, token);
    if (b < 0 || h < 0 || h >= Hq)
        return 1;
    int G = Hq / Hkv;
    int g = h / G;
    int q_len = cu_q_lens[b + 1] - cu_q_lens[b];
    int t = (int)(token - cu_q_lens[b]);
    int kv_len = kv_len_of(kv_lens, layout, Hkv, b, g);
    int past = kv_len - q_len;
    if (past < 0)
        return 1;
    int64_t n_vis = (int64_t)past + t + 1; /* keys 0 .. past + t */

    double *score = (double *)malloc(sizeof(double) * (size_t)n_vis);
    unsigned char *use = (unsigned char *)malloc((size_t)n_vis);
    if (!score || !use) {
        free(score);
        free(use);
        return 1;
    }
    const uint16_t *qrow = q + (token * Hq + h) * (int64_t)D;
    int rc = 0;
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j) {
        int64_t logical = j / S;
        use[j] = 1;
        if (block_allowed && !block_allowed[((int64_t)b * Hkv + g) * max_pages + logical])
            use[j] = 0;
        if (!use[j])
            continue;
        int32_t page = table_entry(tables, layout, Hkv, max_pages, b, g, logical);
        if (page < 0 || page >= num_pages) {
            rc = 2;
            break;
        }
        const int64_t krow = cache_row(layout, S, Hkv, D, page, j % S, g);
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += bf16_to_double(qrow[d]) * cache_value(k_cache, kv8, k_scale, krow + d);
        score[j] = scale * dot;
        if (score[j] > m)
            m = score[j];
    }
    if (rc == 0) {
        double l = 0.0;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        for (int64_t j = 0; j < n_vis; ++j) {
            if (!use[j])
                continue;
            double e = exp(score[j] - m);
            l += e;
            int32_t page = table_entry(tables, layout, Hkv, max_pages, b, g, j / S);
            const int64_t vrow = cache_row(layout, S, Hkv, D, page, j % S, g);
            for (int d = 0; d < D; ++d)
                o[d] += e * cache_value(v_cache, kv8, v_scale, vrow + d);
        }
        /* l > 0 whenever a key is visible; with none, the row is defined as 0. */
        for (int d = 0; d < D; ++d)
            o[d] = l > 0.0 ? o[d] / l : 0.0;
    }
    free(score);
    free(use);
    return rc;
}

/*
 * rows == NULL: every (token, head) row, out[(token * Hq + h) * D + d].
 * rows != NULL: nrows pairs (token, head) in rows[2i], rows[2i+1]; out[i * D + d].
 * block_allowed (nullable, [B][Hkv][max_pages]): a key at position j is visible
 * only if its logical block j / S is allowed for the row's KV head.
 * nthreads <= 0 uses the OpenMP default.
 */
static int attention_impl(int B, const int32_t *cu_q_lens, const int32_t *kv_lens,
                          int Hq, int Hkv, int D, int S, int layout, int max_pages, int num_pages,
                          const int32_t *tables, const uint16_t *q, const void *k_cache,
                          const void *v_cache, int kv8, double k_scale, double v_scale,
                          double scale, const uint8_t *block_allowed,
                          int64_t nrows, const int32_t *rows, double *out, int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || S <= 0 ||
        (layout != 0 && layout != 1))
        return 1;
    int64_t T = cu_q_lens[B];
    int64_t n = rows ? nrows : T * Hq;
    int rc = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(max : rc)
#endif
    for (int64_t i = 0; i < n; ++i) {
        int64_t token = rows ? rows[2 * i] : i / Hq;
        int h = rows ? rows[2 * i + 1] : (int)(i % Hq);
        int r = attend_row(B, cu_q_lens, kv_lens, Hq, Hkv, D, S, layout, max_pages, num_pages,
                           tables, q, k_cache, v_cache, kv8, k_scale, v_scale, scale,
                           block_allowed, token, h, out + i * D);
        if (r > rc)
            rc = r;
    }
    return rc;
}

int oracle_attention(int B, const int32_t *cu_q_lens, const int32_t *kv_lens,
                     int Hq, int Hkv, int D, int S, int layout, int max_pages, int num_pages,
                     const int32_t *tables, const uint16_t *q, const uint16_t *k_cache,
                     const uint16_t *v_cache, double scale, const uint8_t *block_allowed,
                     int64_t nrows, const int32_t *rows, double *out, int nthreads)
{
    return attention_impl(B, cu_q_lens, kv_lens, Hq, Hkv, D, S, layout, max_pages, num_pages,
                          tables, q, k_cache, v_cache, 0, 1.0, 1.0, scale, block_allowed, nrows,
                          rows, out, nthreads);
}

/* The same over FP8 caches: every cached K value is code value * k_scale, V likewise. */
int oracle_attention_fp8(int B, const int32_t *cu_q_lens, const int32_t *kv_lens,
                         int Hq, int Hkv, int D, int S, int layout, int max_pages, int num_pages,
                         const int32_t *tables, const uint16_t *q, const uint8_t *k_cache,
                         const uint8_t *v_cache, double k_scale, double v_scale, double scale,
                         const uint8_t *block_allowed, int64_t nrows, const int32_t *rows,
                         double *out, int nthreads)
{
    return attention_impl(B, cu_q_lens, kv_lens, Hq, Hkv, D, S, layout, max_pages, num_pages,
                          tables, q, k_cache, v_cache, 1, k_scale, v_scale, scale, block_allowed,
                          nrows, rows, out, nthreads);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Block-union tables for one sequence's chunk [past, kv_len).
 *   mask:        [Hq][nQB][nKB] uint8, nonzero = query block qb of head h selects KV block kb
 *   base_tables: [Hkv][nKB] physical page of each logical block of each KV head
 * Steps, in the page's order: union over query blocks per head, then union over the
 * G heads of each group; the chunk's own blocks [past/S, (kv_len-1)/S] are always
 * kept; only blocks below ceil(kv_len/S) are considered.  The selected blocks are
 * listed in ascending order and mapped to physical pages.
 * Outputs: out_tables [Hkv][nKB] (-1 after the count), out_counts [Hkv],
 * out_kv_lens [Hkv] = keys of the compacted sequence, out_selected [Hkv][nKB]
 * (nullable) = the selected set before compaction.
 */
int oracle_union_tables(const uint8_t *mask, int Hq, int Hkv, int nQB, int nKB,
                        const int32_t *base_tables, int past, int kv_len, int S,
                        int32_t *out_tables, int32_t *out_counts, int32_t *out_kv_lens,
                        uint8_t *out_selected)
{
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || nQB <= 0 || nKB <= 0 || S <= 0 ||
        past < 0 || kv_len <= past)
        return 1;
    int G = Hq / Hkv;
    int64_t n_valid = ((int64_t)kv_len + S - 1) / S;
    if (n_valid > nKB)
        return 1;
    int first_chunk = past / S;
    int last_chunk = (kv_len - 1) / S;
    unsigned char *sel = (unsigned char *)calloc((size_t)Hkv * nKB, 1);
    if (!sel)
        return 1;

    /* Q-block union per head, then union over the heads of each group. */
    for (int h = 0; h < Hq; ++h) {
        int g = h / G;
        for (int kb = 0; kb < n_valid; ++kb) {
            int any = 0;
            for (int qb = 0; qb < nQB; ++qb)
                if (mask[((int64_t)h * nQB + qb) * nKB + kb])
                    any = 1;
            if (any)
                sel[(int64_t)g * nKB + kb] = 1;
        }
    }
    for (int g = 0; g < Hkv; ++g)
        for (int kb = first_chunk; kb <= last_chunk; ++kb)
            sel[(int64_t)g * nKB + kb] = 1;

    /* Ascending compaction. */
    for (int g = 0; g < Hkv; ++g) {
        int count = 0;
        for (int kb = 0; kb < nKB; ++kb) {
            if (out_selected)
                out_selected[(int64_t)g * nKB + kb] = sel[(int64_t)g * nKB + kb];
            if (sel[(int64_t)g * nKB + kb])
                out_tables[(int64_t)g * nKB + count++] = base_tables[(int64_t)g * nKB + kb];
        }
        for (int i = count; i < nKB; ++i)
            out_tables[(int64_t)g * nKB + i] = -1;
        out_counts[g] = count;
        int n_chunk_blocks = last_chunk - first_chunk + 1;
        out_kv_lens[g] = (count - n_chunk_blocks) * S + (kv_len - first_chunk * S);
    }
    free(sel);
    return 0;
}

/* fp32 -> bf16 bits, round to nearest even (finite values). */
static uint16_t float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* One row of D values (bf16 bits) rotated at position pos; dims >= rd are copied. */
static void rotate_row(const uint16_t *x, uint16_t *y, int D, int rd, int interleaved,
                       const float *cos_row, const float *sin_row)
{
    for (int d = 0; d < D; ++d) {
        if (d >= rd) {
            y[d] = x[d];
            continue;
        }
        int half = rd / 2;
        int i, first, partner;
        if (interleaved) {
            i = d / 2;
            first = (d % 2) == 0;
            partner = first ? d + 1 : d - 1;
        } else {
            i = d < half ? d : d - half;
            first = d < half;
            partner = first ? d + half : d - half;
        }
        float c = cos_row[i], s = sin_row[i];
        float xd = (float)bf16_to_double(x[d]);
        float xp = (float)bf16_to_double(x[partner]);
        float out = first ? fmaf(xd, c, -(xp * s)) : fmaf(xd, c, xp * s);
        y[d] = float_to_bf16(out);
    }
}

/*
 * q, k, v: the new rows; row t of head h at q + t * q_stride + h * D (likewise k, v with
 * kv_stride); packed QKV is q = qkv, k = qkv + Hq*D, v = qkv + (Hq+Hkv)*D with both strides
 * (Hq + 2 Hkv) * D.  Writes q_out [T][Hq][D] (rotated) and scatters rotated K and V into the
 * caches exactly as oracle_write_kv / oracle_write_kv_fp8 do (kv8, scales).  rd == 0 rotates
 * nothing.  The position of token t of sequence b is kv_len(b, KV head 0) - q_len_b + t.
 * Returns 1 on a bad argument (odd or too large rd, a position >= max_position).
 */
int oracle_rotary_qkv(int B, const int32_t *cu_q_lens, const int32_t *kv_lens,
                      int Hq, int Hkv, int D, int S, int layout, int max_pages, int num_pages,
                      const int32_t *tables, const uint16_t *q, const uint16_t *k,
                      const uint16_t *v, int64_t q_stride, int64_t kv_stride,
                      const float *cos_cache, const float *sin_cache, int max_position,
                      int rd, int interleaved, uint16_t *q_out, void *k_cache, void *v_cache,
                      int kv8, float k_scale, float v_scale)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || rd < 0 || rd > D || rd % 2 != 0)
        return 1;
    int64_t T = cu_q_lens[B];
    uint16_t *kn = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(T * Hkv * D + 1));
    uint16_t *vn = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(T * Hkv * D + 1));
    if (!kn || !vn) {
        free(kn);
        free(vn);
        return 1;
    }
    int rc = 0;
    for (int b = 0; b < B && rc == 0; ++b) {
        int q_len = cu_q_lens[b + 1] - cu_q_lens[b];
        int past = kv_len_of(kv_lens, layout, Hkv, b, 0) - q_len;
        for (int t = 0; t < q_len && rc == 0; ++t) {
            int64_t tok = cu_q_lens[b] + t;
            int pos = past + t;
            if (rd > 0 && (pos < 0 || pos >= max_position)) {
                rc = 1;
                break;
            }
            const float *cr = rd > 0 ? cos_cache + (int64_t)pos * (rd / 2) : NULL;
            const float *sr = rd > 0 ? sin_cache + (int64_t)pos * (rd / 2) : NULL;
            for (int h = 0; h < Hq; ++h)
                rotate_row(q + tok * q_stride + (int64_t)h * D, q_out + (tok * Hq + h) * D, D,
                           rd, interleaved, cr, sr);
            for (int g = 0; g < Hkv; ++g) {
                rotate_row(k + tok * kv_stride + (int64_t)g * D, kn + (tok * Hkv + g) * D, D, rd,
                           interleaved, cr, sr);
                memcpy(vn + (tok * Hkv + g) * D, v + tok * kv_stride + (int64_t)g * D,
                       sizeof(uint16_t) * (size_t)D);
            }
        }
    }
    if (rc == 0) {
        if (kv8)
            rc = oracle_write_kv_fp8(B, cu_q_lens, kv_lens, Hkv, D, S, layout, max_pages,
                                     num_pages, tables, kn, vn, (uint8_t *)k_cache,
                                     (uint8_t *)v_cache, k_scale, v_scale);
        else
            rc = oracle_write_kv(B, cu_q_lens, kv_lens, Hkv, D, S, layout, max_pages, num_pages,
                                 tables, kn, vn, (uint16_t *)k_cache, (uint16_t *)v_cache);
    }
    free(kn);
    free(vn);
    return rc;
}
