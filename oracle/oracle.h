/*
 * CPU oracle for causal grouped-query attention over an fp32 or Q4_0 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library. It shares no code, header, table or
 * helper with the HIP library: everything here is written from the pages'
 * definitions, in plain C, double precision for the attention math, and
 * single-threaded per call.
 *
 * Sources (cited by page title and section):
 *   [FA]  Foundry cuda_kernels/attention.cu
 *         - file header (online softmax contract; StreamingLLM sink + recent
 *           window key set)
 *         - "4-bit KV cache (Q4_0 blocks)" section (row/block byte layout)
 *         - fc_kvq4_quant_block / fc_kvq4_dequant_elem comments (quantiser
 *           steps, negative scale, convert -> +8 -> clamp order)
 *         - fc_attn_tile_in_window comment (tile predicate)
 *         - "Decode-mode flash attention" section and fc_attn_dec_plan comment
 *           (split plan, partial layout)
 *   [VT]  vllm-cpp-sys include/vt/ops.h
 *         - vt::Attention comment (dense causal GQA definition, q head h reads
 *           kv head h / (Hq/Hk))
 *         - AttentionWindow comment ((W-1, 0) is a causal window of W tokens)
 *
 * Every function here is pinned by tests/test_oracle_*.py against hand-built
 * values, closed forms, invariants, library routines or brute force.
 */
#ifndef CGQA_ORACLE_H
#define CGQA_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE 754 binary16 <-> binary32, round-to-nearest-even on the way down. */
uint16_t oracle_f32_to_f16(float f);
float oracle_f16_to_f32(uint16_t h);

/* Q4_0 row of head_dim floats (head_dim % 32 == 0) -> (head_dim/32)*18 bytes.
 * [FA] fc_kvq4_quant_block + the Q4_0 section. Arithmetic in IEEE fp32. */
void oracle_q4_quantize_row(const float *x, int head_dim, uint8_t *row);

/* Inverse: element e = (c - 8) * fp32(half(d)). [FA] fc_kvq4_dequant_elem. */
void oracle_q4_dequantize_row(const uint8_t *row, int head_dim, float *x);

/* Many rows at once (n_rows rows, each head_dim floats / row bytes). */
void oracle_q4_quantize_rows(const float *x, int64_t n_rows, int head_dim, uint8_t *rows);
void oracle_q4_dequantize_rows(const uint8_t *rows, int64_t n_rows, int head_dim, float *x);

/* 1 if key position j is in the key set of a query at position p. [FA] header:
 * win <= 0 -> every j <= p; else j <= p and (j < sink or j >= p - win + 1). */
int oracle_key_in_set(int j, int p, int attn_sink, int attn_win);

/* Output rows of causal GQA attention, global-max softmax in double.
 *   q:     [n_q][n_head][head_dim] fp32
 *   q_pos: [n_q] absolute position of each query row
 *   k, v:  [n_kv_head][kv_rows][head_dim] fp32 (already dequantised if Q4)
 *   sel:   NULL for every (query, head) row, else n_sel flat indices
 *          qi * n_head + h
 *   out:   [n_sel or n_q*n_head][head_dim] double
 * Returns 0, or -1 on bad arguments (position beyond kv_rows, bad heads). */
int oracle_gqa_rows(const float *q, const int *q_pos, int n_q,
                    const float *k, const float *v, int kv_rows,
                    int n_head, int n_kv_head, int head_dim,
                    int attn_sink, int attn_win, double scale,
                    const int64_t *sel, int64_t n_sel, double *out);

/* fp16 shadow of a Q4_0 cache ([FA] "fp16 sink + recent-window exemption",
 * fc_kvq4_is_fp16, and the win_live_lo guard of fc_attn_flash_prefill_q4):
 * a query at position p reads key s at fp16 iff s < shadow_sink, or
 * shadow_win > 0 and s > p - shadow_win and s > live_lo, where live_lo is the
 * highest position appended so far minus the ring size (older ring rows were
 * overwritten). Otherwise it reads the Q4_0 body. */
int oracle_key_is_fp16(int s, int p, int shadow_sink, int shadow_win, int live_lo);

/* oracle_gqa_rows with that choice per (query, key): k, v hold the Q4_0 body
 * (dequantised) and k16, v16 the fp16 shadow values (as fp32), both
 * [n_kv_head][kv_rows][head_dim]. */
int oracle_gqa_rows_shadow(const float *q, const int *q_pos, int n_q,
                           const float *k, const float *v,
                           const float *k16, const float *v16, int kv_rows,
                           int n_head, int n_kv_head, int head_dim,
                           int attn_sink, int attn_win, double scale,
                           int shadow_sink, int shadow_win, int live_lo,
                           const int64_t *sel, int64_t n_sel, double *out);

/* Log-sum-exp of each row's scaled scores over its key set (natural log):
 * lse = ln sum_j exp(scale * q.k_j), the state [VT] MergeAttnStates combines.
 * Same arguments and row selection as oracle_gqa_rows; lse[r] per row. */
int oracle_gqa_lse(const float *q, const int *q_pos, int n_q,
                   const float *k, int kv_rows, int n_head, int n_kv_head, int head_dim,
                   int attn_sink, int attn_win, double scale,
                   const int64_t *sel, int64_t n_sel, double *lse);

/* Decode split plan. [FA] fc_attn_dec_plan: n = clamp(ceil(L/kps), 1, cap);
 * split_len = ceil(L/n) rounded up to a multiple of `tile`; returns the live
 * split count ceil(L/split_len). */
int oracle_decode_plan(int seq_len, int kps, int cap, int tile,
                       int *n_splits, int *split_len);

/* Tile accounting for one block of query positions [q0, q1] walking key tiles
 * of `bk` keys that start at lo and stop before hi (and after q1). A tile is
 * window-skipped when it meets neither [0, sink) nor the union of the rows'
 * windows; every other walked tile is visited. [FA] fc_attn_tile_in_window. */
void oracle_tile_walk(int q0, int q1, int lo, int hi, int attn_sink,
                      int attn_win, int bk, uint64_t *visited,
                      uint64_t *skipped);

/* Totals over a prefill call: query blocks of bq positions from pos0, one walk
 * per block and kv head. */
void oracle_prefill_tile_counts(int n, int pos0, int n_kv_head, int attn_sink,
                                int attn_win, int bq, int bk,
                                uint64_t *visited, uint64_t *skipped);

/* Totals over a multi-slot decode: per slot, the plan of L = pos[s] + 1 with
 * (kps, cap, bk), one walk per live split and kv head. */
void oracle_decode_tile_counts(const int *pos, int n_slots, int n_kv_head,
                               int kps, int cap, int attn_sink, int attn_win,
                               int bk, uint64_t *visited, uint64_t *skipped);

#ifdef __cplusplus
}
#endif

#endif /* CGQA_ORACLE_H */
