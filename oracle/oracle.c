/*
 * CPU oracle for causal grouped-query attention over an fp32 or Q4_0 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * bench's CPU-baseline leg, never by the HIP library. See oracle.h for the
 * sources and the contract of every function. Built with plain gcc, no
 * fast-math and no FP contraction, so the fp32 quantiser steps round exactly
 * as written.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- binary16 */

/* IEEE 754 binary32 -> binary16, round to nearest, ties to even.
 * A binary16 value has 10 stored significand bits; its quantum is 2^(e-25)
 * for biased exponent e >= 1 and 2^-24 for subnormals. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, sizeof x);
    const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    const int exp32 = (int)((x >> 23) & 0xffu);
    const uint32_t man32 = x & 0x7fffffu;

    if (exp32 == 0xff)                       /* inf / nan */
        return (uint16_t)(sign | 0x7c00u | (man32 ? 0x200u | (man32 >> 13) : 0u));
    if (exp32 == 0)                          /* zero or fp32 subnormal: below 2^-25 */
        return sign;

    const int e16 = exp32 - 127 + 15;        /* unbiased-to-binary16 bias */
    const int e_eff = e16 >= 1 ? e16 : 1;
    const uint32_t sig = man32 | 0x800000u;  /* 24-bit significand, value sig*2^(exp32-150) */
    const int shift = 125 + e_eff - exp32;   /* sig / quantum = sig >> shift */
    if (shift >= 26)                         /* below a quarter quantum: rounds to zero */
        return sign;

    uint32_t q = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;

    uint32_t h;
    if (e16 >= 1)
        h = ((uint32_t)e16 << 10) + q - 0x400u;  /* a carry out of q bumps the exponent */
    else
        h = q;                                    /* subnormal (0x400 = smallest normal) */
    if (h >= 0x7c00u)
        h = 0x7c00u;                              /* overflow to infinity */
    return (uint16_t)(sign | h);
}

float oracle_f16_to_f32(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int m = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* ------------------------------------------------------------------- Q4_0 */

enum { Q4_BLK = 32, Q4_BLK_BYTES = 18 };

/* Code of one element: rint(x * id) clamped to [-8, 7], plus 8. The clamp
 * is done on the float before converting, so that products outside the int
 * range have a defined code (C leaves the conversion undefined there): a NaN
 * product (NaN element, or 0 * inf when 1/d overflows) is taken as 0, i.e.
 * code 8, and +-inf clamp to codes 15 / 0. For finite in-range products this
 * is clamp(int(rint(x * id)) + 8, 0, 15). */
static int q4_code(float x, float id)
{
    float r = rintf(x * id);
    if (isnan(r))
        return 8;
    if (r < -8.0f)
        r = -8.0f;
    if (r > 7.0f)
        r = 7.0f;
    return (int)r + 8;
}

/* One 32-element block of the Q4_0 format, whose definition fixes the
 * bytes and the order of the steps ([FA] "4-bit KV cache (Q4_0 blocks)"
 * section, fc_kvq4_quant_block). Steps, all in fp32:
 *  1. amax: fmaxf fold of |x_j| starting from 0
 *  2. d = amax / -8  (the stored scale is negative)
 *  3. id = 1/d, or 0 when d is zero
 *  4. code_j = clamp(int(rint(x_j * id)) + 8, 0, 15), the clamp taken on the
 *     float (q4_code) so non-finite products are defined
 *  5. bytes 0-1: binary16(d) little-endian; byte 2+j: code_j | code_{j+16} << 4 */
static void q4_block(const float *xb, uint8_t *blk)
{
    float amax = 0.0f;
    for (int j = 0; j < Q4_BLK; j++)
        amax = fmaxf(amax, fabsf(xb[j]));
    const float d = amax / -8.0f;
    const float id = (d != 0.0f) ? 1.0f / d : 0.0f;

    const uint16_t dh = oracle_f32_to_f16(d);
    blk[0] = (uint8_t)(dh & 0xffu);
    blk[1] = (uint8_t)(dh >> 8);
    for (int j = 0; j < Q4_BLK / 2; j++) {
        const int lo = q4_code(xb[j], id);
        const int hi = q4_code(xb[j + Q4_BLK / 2], id);
        blk[2 + j] = (uint8_t)(lo | (hi << 4));
    }
}

void oracle_q4_quantize_row(const float *x, int head_dim, uint8_t *row)
{
    for (int b = 0; b < head_dim / Q4_BLK; b++)
        q4_block(x + (size_t)b * Q4_BLK, row + (size_t)b * Q4_BLK_BYTES);
}

void oracle_q4_dequantize_row(const uint8_t *row, int head_dim, float *x)
{
    for (int e = 0; e < head_dim; e++) {
        const uint8_t *blk = row + (size_t)(e / Q4_BLK) * Q4_BLK_BYTES;
        const float d = oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
        const int local = e % Q4_BLK;
        const int byte = blk[2 + (local % (Q4_BLK / 2))];
        const int code = local < Q4_BLK / 2 ? (byte & 0xf) : (byte >> 4);
        x[e] = (float)(code - 8) * d;
    }
}

void oracle_q4_quantize_rows(const float *x, int64_t n_rows, int head_dim, uint8_t *rows)
{
    const size_t rb = (size_t)(head_dim / Q4_BLK) * Q4_BLK_BYTES;
    for (int64_t r = 0; r < n_rows; r++)
        oracle_q4_quantize_row(x + (size_t)r * head_dim, head_dim, rows + (size_t)r * rb);
}

void oracle_q4_dequantize_rows(const uint8_t *rows, int64_t n_rows, int head_dim, float *x)
{
    const size_t rb = (size_t)(head_dim / Q4_BLK) * Q4_BLK_BYTES;
    for (int64_t r = 0; r < n_rows; r++)
        oracle_q4_dequantize_row(rows + (size_t)r * rb, head_dim, x + (size_t)r * head_dim);
}

/* -------------------------------------------------------------- attention */

int oracle_key_in_set(int j, int p, int attn_sink, int attn_win)
{
    if (j < 0 || j > p)
        return 0;                       /* causal: only keys at or before the query */
    if (attn_win <= 0)
        return 1;                       /* full causal attention */
    return j < attn_sink || j >= p - attn_win + 1;
}

/* softmax_j(scale * q.k_j) over the key set, applied to v; global max first. */
static void attend_one(const float *qv, const float *kb, const float *vb,
                       int head_dim, int p, int attn_sink, int attn_win,
                       double scale, double *sc, double *out)
{
    double m = -INFINITY;
    for (int j = 0; j <= p; j++) {
        if (!oracle_key_in_set(j, p, attn_sink, attn_win))
            continue;
        const float *kj = kb + (size_t)j * head_dim;
        double dot = 0.0;
        for (int e = 0; e < head_dim; e++)
            dot += (double)qv[e] * (double)kj[e];
        sc[j] = scale * dot;
        if (sc[j] > m)
            m = sc[j];
    }
    double sum = 0.0;
    for (int e = 0; e < head_dim; e++)
        out[e] = 0.0;
    for (int j = 0; j <= p; j++) {
        if (!oracle_key_in_set(j, p, attn_sink, attn_win))
            continue;
        const double w = exp(sc[j] - m);
        const float *vj = vb + (size_t)j * head_dim;
        sum += w;
        for (int e = 0; e < head_dim; e++)
            out[e] += w * (double)vj[e];
    }
    for (int e = 0; e < head_dim; e++)
        out[e] /= sum;
}

int oracle_gqa_rows(const float *q, const int *q_pos, int n_q,
                    const float *k, const float *v, int kv_rows,
                    int n_head, int n_kv_head, int head_dim,
                    int attn_sink, int attn_win, double scale,
                    const int64_t *sel, int64_t n_sel, double *out)
{
    if (n_q < 0 || n_head <= 0 || n_kv_head <= 0 || head_dim <= 0 ||
        n_head % n_kv_head != 0)
        return -1;
    const int group = n_head / n_kv_head;
    const int64_t total = sel ? n_sel : (int64_t)n_q * n_head;
    int max_p = -1;
    for (int i = 0; i < n_q; i++) {
        if (q_pos[i] < 0 || q_pos[i] >= kv_rows)
            return -1;
        if (q_pos[i] > max_p)
            max_p = q_pos[i];
    }
    double *sc = (double *)malloc(sizeof(double) * (size_t)(max_p + 1 > 0 ? max_p + 1 : 1));
    if (!sc)
        return -1;
    for (int64_t r = 0; r < total; r++) {
        const int64_t flat = sel ? sel[r] : r;
        if (flat < 0 || flat >= (int64_t)n_q * n_head) {
            free(sc);
            return -1;
        }
        const int qi = (int)(flat / n_head);
        const int h = (int)(flat % n_head);
        const int kvh = h / group;      /* consecutive q heads share a kv head */
        const size_t kv_off = (size_t)kvh * kv_rows * head_dim;
        attend_one(q + (size_t)flat * head_dim, k + kv_off, v + kv_off, head_dim,
                   q_pos[qi], attn_sink, attn_win, scale, sc,
                   out + (size_t)r * head_dim);
    }
    free(sc);
    return 0;
}

/* ------------------------------------------------------- plans and tiles */

int oracle_key_is_fp16(int s, int p, int shadow_sink, int shadow_win, int live_lo)
{
    if (s < shadow_sink)
        return 1;
    return shadow_win > 0 && s > p - shadow_win && s > live_lo;
}

/* attend_one with the K/V row of key j taken from the shadow (k16/v16) or
 * the Q4_0 body (k/v) by oracle_key_is_fp16. */
static void attend_one_shadow(const float *qv, const float *kb, const float *vb,
                              const float *kb16, const float *vb16, int head_dim, int p,
                              int attn_sink, int attn_win, int shadow_sink,
                              int shadow_win, int live_lo, double scale, double *sc,
                              double *out)
{
    double m = -INFINITY;
    for (int j = 0; j <= p; j++) {
        if (!oracle_key_in_set(j, p, attn_sink, attn_win))
            continue;
        const int f16 = oracle_key_is_fp16(j, p, shadow_sink, shadow_win, live_lo);
        const float *kj = (f16 ? kb16 : kb) + (size_t)j * head_dim;
        double dot = 0.0;
        for (int e = 0; e < head_dim; e++)
            dot += (double)qv[e] * (double)kj[e];
        sc[j] = scale * dot;
        if (sc[j] > m)
            m = sc[j];
    }
    double sum = 0.0;
    for (int e = 0; e < head_dim; e++)
        out[e] = 0.0;
    for (int j = 0; j <= p; j++) {
        if (!oracle_key_in_set(j, p, attn_sink, attn_win))
            continue;
        const int f16 = oracle_key_is_fp16(j, p, shadow_sink, shadow_win, live_lo);
        const double w = exp(sc[j] - m);
        const float *vj = (f16 ? vb16 : vb) + (size_t)j * head_dim;
        sum += w;
        for (int e = 0; e < head_dim; e++)
            out[e] += w * (double)vj[e];
    }
    for (int e = 0; e < head_dim; e++)
        out[e] /= sum;
}

int oracle_gqa_rows_shadow(const float *q, const int *q_pos, int n_q,
                           const float *k, const float *v,
                           const float *k16, const float *v16, int kv_rows,
                           int n_head, int n_kv_head, int head_dim,
                           int attn_sink, int attn_win, double scale,
                           int shadow_sink, int shadow_win, int live_lo,
                           const int64_t *sel, int64_t n_sel, double *out)
{
    if (n_q < 0 || n_head <= 0 || n_kv_head <= 0 || head_dim <= 0 ||
        n_head % n_kv_head != 0)
        return -1;
    const int group = n_head / n_kv_head;
    const int64_t total = sel ? n_sel : (int64_t)n_q * n_head;
    int max_p = -1;
    for (int i = 0; i < n_q; i++) {
        if (q_pos[i] < 0 || q_pos[i] >= kv_rows)
            return -1;
        if (q_pos[i] > max_p)
            max_p = q_pos[i];
    }
    double *sc = (double *)malloc(sizeof(double) * (size_t)(max_p + 1 > 0 ? max_p + 1 : 1));
    if (!sc)
        return -1;
    for (int64_t r = 0; r < total; r++) {
        const int64_t flat = sel ? sel[r] : r;
        if (flat < 0 || flat >= (int64_t)n_q * n_head) {
            free(sc);
            return -1;
        }
        const int qi = (int)(flat / n_head);
        const int h = (int)(flat % n_head);
        const int kvh = h / group;
        const size_t kv_off = (size_t)kvh * kv_rows * head_dim;
        attend_one_shadow(q + (size_t)flat * head_dim, k + kv_off, v + kv_off, k16 + kv_off,
                          v16 + kv_off, head_dim, q_pos[qi], attn_sink, attn_win,
                          shadow_sink, shadow_win, live_lo, scale, sc,
                          out + (size_t)r * head_dim);
    }
    free(sc);
    return 0;
}

int oracle_gqa_lse(const float *q, const int *q_pos, int n_q,
                   const float *k, int kv_rows, int n_head, int n_kv_head, int head_dim,
                   int attn_sink, int attn_win, double scale,
                   const int64_t *sel, int64_t n_sel, double *lse)
{
    if (n_q < 0 || n_head <= 0 || n_kv_head <= 0 || head_dim <= 0 ||
        n_head % n_kv_head != 0)
        return -1;
    const int group = n_head / n_kv_head;
    const int64_t total = sel ? n_sel : (int64_t)n_q * n_head;
    for (int i = 0; i < n_q; i++)
        if (q_pos[i] < 0 || q_pos[i] >= kv_rows)
            return -1;
    for (int64_t r = 0; r < total; r++) {
        const int64_t flat = sel ? sel[r] : r;
        if (flat < 0 || flat >= (int64_t)n_q * n_head)
            return -1;
        const int p = q_pos[flat / n_head];
        const float *qv = q + (size_t)flat * head_dim;
        const float *kb = k + (size_t)((flat % n_head) / group) * kv_rows * head_dim;
        /* max first, then ln sum exp(s - max) + max */
        double m = -INFINITY;
        for (int j = 0; j <= p; j++) {
            if (!oracle_key_in_set(j, p, attn_sink, attn_win))
                continue;
            double dot = 0.0;
            for (int e = 0; e < head_dim; e++)
                dot += (double)qv[e] * (double)kb[(size_t)j * head_dim + e];
            if (scale * dot > m)
                m = scale * dot;
        }
        double sum = 0.0;
        for (int j = 0; j <= p; j++) {
            if (!oracle_key_in_set(j, p, attn_sink, attn_win))
                continue;
            double dot = 0.0;
            for (int e = 0; e < head_dim; e++)
                dot += (double)qv[e] * (double)kb[(size_t)j * head_dim + e];
            sum += exp(scale * dot - m);
        }
        lse[r] = m + log(sum);
    }
    return 0;
}

int oracle_decode_plan(int seq_len, int kps, int cap, int tile,
                       int *n_splits, int *split_len)
{
    if (seq_len < 1 || kps < 1 || cap < 1 || tile < 1)
        return -1;
    int n = (seq_len + kps - 1) / kps;
    if (n < 1)
        n = 1;
    if (n > cap)
        n = cap;
    int len = (seq_len + n - 1) / n;
    len = (len + tile - 1) / tile * tile;
    *n_splits = n;
    *split_len = len;
    return (seq_len + len - 1) / len;
}

void oracle_tile_walk(int q0, int q1, int lo, int hi, int attn_sink,
                      int attn_win, int bk, uint64_t *visited,
                      uint64_t *skipped)
{
    for (int j0 = lo; j0 < hi && j0 <= q1; j0 += bk) {
        int e = j0 + bk - 1;            /* last key of the tile the block can see */
        if (e > hi - 1)
            e = hi - 1;
        if (e > q1)
            e = q1;
        if (attn_win > 0 && j0 >= attn_sink && e < q0 - attn_win + 1)
            (*skipped)++;
        else
            (*visited)++;
    }
}

void oracle_prefill_tile_counts(int n, int pos0, int n_kv_head, int attn_sink,
                                int attn_win, int bq, int bk,
                                uint64_t *visited, uint64_t *skipped)
{
    uint64_t vis = 0, skp = 0;
    for (int b = 0; (int64_t)b * bq < n; b++) {
        const int q0 = pos0 + b * bq;
        int q1 = q0 + bq - 1;
        if (q1 > pos0 + n - 1)
            q1 = pos0 + n - 1;
        oracle_tile_walk(q0, q1, 0, q1 + 1, attn_sink, attn_win, bk, &vis, &skp);
    }
    *visited = vis * (uint64_t)n_kv_head;
    *skipped = skp * (uint64_t)n_kv_head;
}

void oracle_decode_tile_counts(const int *pos, int n_slots, int n_kv_head,
                               int kps, int cap, int attn_sink, int attn_win,
                               int bk, uint64_t *visited, uint64_t *skipped)
{
    uint64_t vis = 0, skp = 0;
    for (int s = 0; s < n_slots; s++) {
        const int len = pos[s] + 1;
        int n_splits, split_len;
        const int live = oracle_decode_plan(len, kps, cap, bk, &n_splits, &split_len);
        for (int sp = 0; sp < live; sp++) {
            const int lo = sp * split_len;
            int hi = lo + split_len;
            if (hi > len)
                hi = len;
            oracle_tile_walk(pos[s], pos[s], lo, hi, attn_sink, attn_win, bk, &vis, &skp);
        }
    }
    *visited = vis * (uint64_t)n_kv_head;
    *skipped = skp * (uint64_t)n_kv_head;
}
