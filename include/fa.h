/*
 * libfa: causal grouped-query flash attention for AMD Instinct MI355X (gfx950)
 * over a device-resident KV cache stored as fp32 or as 4-bit Q4_0 blocks.
 *
 * Sources cited below:
 *   [FA] Foundry cuda_kernels/attention.cu (the kernel file this method
 *        comes from): file header, "4-bit KV cache (Q4_0 blocks)" section,
 *        fc_kvq4_quant_block, fc_attn_tile_in_window, fc_attn_kv_append,
 *        fc_attn_flash_prefill, "Decode-mode flash attention" section,
 *        fc_attn_dec_plan, fc_attn_flash_decode_combine, "Multi-user decode
 *        attention (slots)" section.
 *   [VT] vllm-cpp-sys include/vt/ops.h: vt::Attention, AttentionWindow,
 *        MlaDecodeAttention (split determinism), PagedAttentionArgs
 *        (host-known max_seq_len hint), ReshapeAndCache, PagedAttention,
 *        MergeAttnStates, kernel registration contract (unsupported inputs
 *        fail loudly).
 *
 * Conventions shared by every entry point:
 *   - Pointers named k, v, k_new, v_new, q, out, d_pos, ws, tile_stats are
 *     DEVICE pointers owned by the caller. The library never allocates,
 *     frees or keeps them after the call returns, and never synchronises.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream. All work is enqueued on it, in call order.
 *   - Every argument is validated on the host before anything is enqueued.
 *     A rejected call returns a negative FA_E* code and enqueues nothing;
 *     fa_strerror() names the code. A launch the runtime refuses returns
 *     FA_EHIP. No C++ exception crosses this interface.
 *   - Layouts are row-major with the last index fastest.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- codes */
#define FA_OK            0
#define FA_EINVAL       -1  /* a size, index or scalar is out of its valid range */
#define FA_ENULL        -2  /* a required pointer is NULL */
#define FA_EUNSUPPORTED -3  /* valid but not built: head_dim, group size or format */
#define FA_EWORKSPACE   -4  /* workspace smaller than the call needs (or than the fixed
                               decode scratch of fa_decode_noalloc can hold) */
#define FA_EHIP         -5  /* the HIP runtime refused a launch or query */
#define FA_ERANGE       -6  /* positions past the cache (pos0 + n > max_seq) */
#define FA_EDEVICE      -7  /* current device is not a gfx950 GPU */

/* ----------------------------------------------------------- KV formats */
/* fp32 rows of head_dim floats. [FA] fc_attn_kv_append. */
#define FA_KV_F32   0
/* Q4_0 rows of head_dim/32 blocks of 18 bytes: bytes 0-1 the binary16 scale
 * d (little-endian, stored negative: d = amax / -8), byte 2+j element j in
 * the low nibble and element j+16 in the high nibble; code c decodes to
 * (c - 8) * d. [FA] "4-bit KV cache (Q4_0 blocks)" and fc_kvq4_quant_block. */
#define FA_KV_Q4_0  1

/* Capacity of the optional fp16 shadow of a Q4_0 cache ([FA] "fp16 sink +
 * recent-window exemption": the first positions and a ring of recent rows per
 * (slot, kv head) are also kept at fp16). The ring laps at
 * FA_SHADOW_WIN_MAX rows whatever the window width. */
#define FA_SHADOW_SINK_MAX 8
#define FA_SHADOW_WIN_MAX  256

/* A KV cache of n_slots independent sequences.
 * k and v each hold [n_slots][n_kv_head][max_seq][row] where row is
 * fa_cache_row_bytes(format, head_dim) bytes ([FA] slots section: one ring
 * per slot, each slot's slice laid out like the single-user cache).
 *
 * fp16 shadow (Q4_0 only; all zero / NULL = none). [FA] "fp16 sink +
 * recent-window exemption" and fc_kvq4_is_fp16: every appended row also goes,
 * rounded to binary16 (round-to-nearest-even), to
 *   k_sink/v_sink [n_slots][n_kv_head][FA_SHADOW_SINK_MAX][head_dim] if its
 *     position p < shadow_sink;
 *   k_win/v_win   [n_slots][n_kv_head][FA_SHADOW_WIN_MAX][head_dim] at ring
 *     row p % FA_SHADOW_WIN_MAX if shadow_win > 0, with win_pos
 *     [n_slots][FA_SHADOW_WIN_MAX] (int32) recording the position each ring
 *     row holds (the caller fills win_pos with -1 before first use).
 * Attention for a query at position p then reads key s from the shadow
 * instead of the Q4_0 body iff s < shadow_sink, or shadow_win > 0 and
 * s > p - shadow_win and win_pos holds s (the row was not overwritten by a
 * later position); otherwise from the Q4_0 body, which holds every row. */
typedef struct fa_cache {
    int format;      /* FA_KV_F32 or FA_KV_Q4_0 */
    int n_slots;     /* >= 1 */
    int n_kv_head;   /* >= 1 */
    int head_dim;    /* 64, 128 or 256 */
    int max_seq;     /* rows per (slot, kv head), >= 1 */
    void *k;         /* device, fa_cache_bytes() bytes */
    void *v;         /* device, fa_cache_bytes() bytes */
    int shadow_sink; /* 0 .. FA_SHADOW_SINK_MAX */
    int shadow_win;  /* 0 .. FA_SHADOW_WIN_MAX */
    void *k_sink, *v_sink;   /* device fp16, required if shadow_sink > 0 */
    void *k_win, *v_win;     /* device fp16, required if shadow_win > 0 */
    int *win_pos;            /* device int32, required if shadow_win > 0 */
} fa_cache;

/* Bytes of one cache row (head_dim*4 for fp32, head_dim/32*18 for Q4_0);
 * 0 if format or head_dim is invalid. */
size_t fa_cache_row_bytes(int format, int head_dim);

/* Bytes of the k (or v) tensor of a cache; 0 if a field is invalid. */
size_t fa_cache_bytes(const fa_cache *cache);

/* Checks that the current HIP device is gfx950. FA_OK or FA_EDEVICE/FA_EHIP.
 * Every compute entry point calls it once per device. */
int fa_init(void);

/* ------------------------------------------------------------ KV append */
/* Writes n new K/V rows of one slot into the cache at positions
 * pos0 .. pos0+n-1. [FA] fc_attn_kv_append (fp32 copy) and
 * fc_attn_kv_append_q4 + fc_kvq4_quant_block (Q4_0: per 32-element block,
 * amax fold, d = amax/-8, id = 1/d or 0, code = clamp(rint(x*id)+8, 0, 15),
 * binary16 scale), all in IEEE fp32 so the bytes are exactly determined.
 * The clamp is taken on the rounded product as a float, so non-finite
 * products have defined codes: a NaN product (a NaN element, or 0 * inf when
 * a block's amax is below 2^-125 and 1/d overflows) gives code 8, +-inf give
 * codes 15 / 0; the amax fold skips quiet NaN elements (fmaxf). A scale
 * beyond binary16 range is stored as -inf.
 *   k_new, v_new: device [n][n_kv_head][head_dim] fp32.
 *   slot in [0, n_slots); pos0 >= 0; n >= 0; pos0 + n <= max_seq (the
 *   cache never wraps: FA_ERANGE otherwise). n == 0 enqueues nothing. */
int fa_kv_append(const fa_cache *cache, int slot, int pos0, int n,
                 const float *k_new, const float *v_new, void *stream);

/* One new row per slot at a position held in device memory ([FA] "Multi-user
 * decode attention (slots)" section, fc_attn_kv_append_slots and the per-slot
 * Q4_0 append; the device-resident position of fc_attn_kv_append_dev). For
 * every slot s in [0, n_slots), row s of k_new/v_new is written to cache
 * position d_pos[s] of slot s, converted exactly as fa_kv_append converts it
 * (fp32 copy, or the same Q4_0 block quantisation, byte for byte). The
 * positions are read on the device, so the enqueued work does not depend on
 * them: with fa_decode (which also reads d_pos on the device) and a device-
 * side position increment, one captured HIP graph replays a decode step at
 * every position.
 *   k_new, v_new: device [n_slots][n_kv_head][head_dim] fp32 (finite values).
 *   d_pos: device int32[n_slots]. A slot whose d_pos[s] is outside
 *   [0, max_seq) is left unchanged (the cache never wraps; fa_decode returns
 *   NaN rows for such a slot). 0 <= n_slots <= cache->n_slots; n_slots == 0
 *   enqueues nothing. One launch on `stream`. */
int fa_kv_append_slots(const fa_cache *cache, const int *d_pos, int n_slots,
                       const float *k_new, const float *v_new, void *stream);

/* -------------------------------------------------------------- prefill */
/* Causal GQA attention for n query rows of one slot at absolute positions
 * pos0 .. pos0+n-1, against cache rows [0, pos0+n) of that slot, which must
 * already be appended. [VT] vt::Attention: for q head h (kv head h/G,
 * G = n_head / n_kv_head) and query position p,
 *     s_j = scale * (q . k_j) for j in K(p);  out = sum_j softmax(s)_j v_j
 * with the key set of the [FA] file header:
 *     K(p) = {0..p}                                   if attn_win <= 0
 *     K(p) = {j <= p : j < attn_sink or j >= p-attn_win+1}  otherwise
 * (attn_win = W is the causal window (W-1, 0) of [VT] AttentionWindow).
 * The N x N score matrix is never formed: key tiles are folded into a
 * running max and running sum ([FA] file header), and key tiles that meet
 * neither the sink nor any row's window are skipped before they are loaded
 * ([FA] fc_attn_tile_in_window).
 *   q:   device [n][n_head][head_dim] fp32.  out: device, same shape.
 *   n_head % n_kv_head == 0, G in {1,2,4,8}; head_dim in {64,128,256};
 *   scale finite and > 0 (applied to q.k); attn_sink < 0 acts as 0.
 *   ws, ws_bytes: device scratch of at least fa_prefill_workspace_bytes().
 *   tile_stats: NULL, or device uint64[2] to which the call ADDS the number
 *   of key tiles it visited ([0]) and window-skipped ([1]); tile geometry
 *   from fa_prefill_tile_shape(). Tiles past the causal bound are neither.
 * With an fp16 shadow, the shadow keys of every query block are folded
 * first, by a launch of the same kernel over the shadow buffers, and each
 * row's pass over the Q4_0 body starts from that partial.
 * Rows of q and out must not overlap. Two launches on `stream` (four with a
 * shadow); nothing in them depends on host reads of device data, so a
 * captured HIP graph replays the call.
 * The work-groups split the visited key tiles by a schedule of 4 units per
 * tile and 5 per query block of fa_prefill_tile_shape() positions, summed
 * over kv heads and counted in 32 bits: a call whose total exceeds 2^31 - 1
 * (a full-causal prefill of about 2^19 positions at 8 kv heads) returns
 * FA_EUNSUPPORTED, checked before the workspace size. */
int fa_prefill(const fa_cache *cache, int slot, const float *q, int pos0, int n,
               int n_head, int attn_sink, int attn_win, float scale, float *out,
               void *ws, size_t ws_bytes, unsigned long long *tile_stats, void *stream);

/* Workspace fa_prefill needs for n query rows: when a query block's key
 * tiles are spread over several work-groups (the schedule balances the
 * causal triangle across CUs), each part leaves a partial {m, l, acc} per
 * row ([FA] decode partial form) that a second launch merges; plus the list
 * of such cut blocks (fewer than the work-groups), and, for a cache with an
 * fp16 shadow, each row's shadow-key m and l. Independent of pos0 and of the
 * data. 0 if an argument is invalid. */
size_t fa_prefill_workspace_bytes(int n, int n_head, int n_kv_head, int head_dim);

/* Tile geometry fa_prefill uses for a shape: each work-group owns
 * *q_positions consecutive query positions (from pos0) of one kv head and
 * walks key tiles of *key_tile keys from key 0. FA_OK or FA_EUNSUPPORTED. */
int fa_prefill_tile_shape(int n_head, int n_kv_head, int head_dim,
                          int *q_positions, int *key_tile);

/* --------------------------------------------------------------- decode */
/* Split plan of one slot with seq_len = pos + 1 keys. [FA] fc_attn_dec_plan:
 *   n = clamp(ceil(seq_len / kps), 1, cap); split_len = ceil(seq_len / n)
 *   rounded up to a multiple of the decode key tile; returns the live split
 *   count ceil(seq_len / split_len) (or FA_EINVAL if seq_len < 1).
 * kps, cap and the key tile are the library's constants
 * (fa_decode_plan_params); the device computes the same plan per slot. */
int fa_decode_plan(int seq_len, int *n_splits, int *split_len);
void fa_decode_plan_params(int *kps, int *cap, int *key_tile);

/* Workspace for fa_decode: partials {m, l, acc[head_dim]} fp32 ([FA]
 * "Decode-mode flash attention": running max, running sum and unnormalised
 * accumulator of the keys a partial folded) plus a per-(slot, kv head) table
 * of where each one's partials start. The size depends on n_slots, the head
 * counts and max_ctx (which fixes how many work-groups the partial pass
 * uses), not on the device positions. 0 if an argument is invalid. */
size_t fa_decode_workspace_bytes(const fa_cache *cache, int n_slots, int n_head,
                                 int max_ctx);

/* One decode step for slots 0..n_slots-1: the query row of slot s sits at
 * position d_pos[s] and attends K(d_pos[s]) of that slot's cache (its own
 * row already appended). Two launches on `stream` ([FA] "Decode-mode flash
 * attention" and slots sections):
 *   1. partial pass: every slot's keys [0, d_pos[s]] are cut into splits by
 *      fa_decode_plan, computed on the device from d_pos[s]. The splits of
 *      all (slot, kv head) pairs form one work list that a fixed grid of
 *      single-wave work-groups divides into equal contiguous runs; a wave
 *      folds the splits of one (slot, kv head) in its run into one partial.
 *   2. combine per (slot, head): M = max_r m_r, out = sum_r w_r acc_r /
 *      sum_r w_r l_r with w_r = exp(m_r - M), partials in ascending key
 *      order, no atomics, so a fixed launch gives bit-identical results
 *      ([VT] MlaDecodeAttention determinism).
 *   q, out: device [n_slots][n_head][head_dim] fp32.
 *   d_pos:  device int32[n_slots]. A value outside [0, max_seq) reads no
 *           memory and makes that slot's output rows NaN.
 *   max_ctx_hint: host upper bound on d_pos[s]+1, 1..max_seq ([VT]
 *           PagedAttentionArgs max_seq_len: sizes the launch without a device
 *           read). A slot with more keys than the hint is still computed
 *           exactly.
 *   ws, ws_bytes: device scratch of at least
 *           fa_decode_workspace_bytes(cache, n_slots, n_head, max_ctx_hint),
 *           16-byte aligned (FA_EINVAL otherwise).
 *   tile_stats: as in fa_prefill, key tiles of the plan's tile size walked
 *           split by split.
 * n_slots == 0 enqueues nothing. Other rules as fa_prefill. The work items
 * (at most the plan's cap per slot and kv head) are counted in 32 bits:
 * n_slots * n_kv_head beyond (2^31 - 1) / cap returns FA_EUNSUPPORTED. */
int fa_decode(const fa_cache *cache, const float *q, const int *d_pos, int n_slots,
              int max_ctx_hint, int n_head, int attn_sink, int attn_win, float scale,
              float *out, void *ws, size_t ws_bytes, unsigned long long *tile_stats,
              void *stream);

/* fa_decode over a Q4_0 cache with the two tile contractions on fp16 matrix
 * cores (v_mfma_f32_16x16x32_f16, fp32 accumulate) instead of fp32 ones: an
 * opt-in lane that departs from fp32 operands, in the way of [FA]'s
 * "NARROW-STAGING prefill variants" note (fp16-narrowed K staging) and of
 * the two-pass hi/lo activation lane of the logicaffeine
 * codegen_cuda/qwen38_batched.rs page, so that a decode over 4-bit keys and
 * values is no longer bound by the fp32 matrix rate. Q4_0 codes are exact
 * binary16 values; q, and p times each key's block scale, are carried as an
 * fp16 high part plus an fp16 low part (their rounding error), so every
 * product is exact and sums are fp32: results agree with fa_decode to about
 * fp32 rounding (the oracle bar of the Q4_0 cache applies), not bit for bit.
 * Same arguments, workspace (fa_decode_workspace_bytes), schedule, partials
 * and combine as fa_decode. The cache must be FA_KV_Q4_0 without an fp16
 * shadow (FA_EUNSUPPORTED otherwise); other rules as fa_decode. */
int fa_decode_q4_hilo(const fa_cache *cache, const float *q, const int *d_pos, int n_slots,
                      int max_ctx_hint, int n_head, int attn_sink, int attn_win, float scale,
                      float *out, void *ws, size_t ws_bytes, unsigned long long *tile_stats,
                      void *stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * call as fa_decode (same kernels, same results bit for bit) without the
 * workspace argument: the partials live in a scratch array the library
 * holds on every GPU it runs on, FA_DECODE_SCRATCH_BYTES per GPU, for the
 * life of the process. Nothing is allocated, freed or cleared per call
 * (every scratch byte the combine reads is written earlier in the same call).
 * A call whose fa_decode_workspace_bytes(cache, n_slots, n_head,
 * max_ctx_hint) exceeds FA_DECODE_SCRATCH_BYTES returns FA_EWORKSPACE. All
 * calls on one GPU share its scratch: calls that overlap in time on one GPU
 * (other streams, other host threads) race and corrupt each other's
 * results; calls on one stream are ordered and safe. Arguments and other
 * rules as fa_decode. */
#define FA_DECODE_SCRATCH_BYTES (32u << 20)
int fa_decode_noalloc(const fa_cache *cache, const float *q, const int *d_pos, int n_slots,
                      int max_ctx_hint, int n_head, int attn_sink, int attn_win, float scale,
                      float *out, unsigned long long *tile_stats, void *stream);

/* ------------------------------------------------ paged KV, varlen batch */
/* A paged fp32 KV cache in the NHD layout of [VT] ReshapeAndCache and
 * PagedAttention: k and v each hold num_blocks pages of block_size rows, and
 * row o of page b for kv head g is the head_dim floats starting at float
 *     b * block_stride + (o * n_kv_head + g) * head_dim
 * of k (or v). block_stride 0 means block_size * n_kv_head * head_dim, i.e.
 * k and v are [num_blocks][block_size][n_kv_head][head_dim]; the two halves
 * of one [num_blocks][2][block_size][n_kv_head][head_dim] allocation are
 * k = base, v = base + block_size * n_kv_head * head_dim with block_stride
 * 2 * block_size * n_kv_head * head_dim. */
typedef struct fa_paged_cache {
    int num_blocks;          /* >= 1 */
    int block_size;          /* rows per page, >= 1 */
    int n_kv_head;           /* >= 1 */
    int head_dim;            /* 64, 128 or 256 */
    long long block_stride;  /* floats between pages: 0, or a multiple of 4 that is
                                at least block_size * n_kv_head * head_dim */
    float *k, *v;            /* device, 16-byte aligned */
} fa_paged_cache;

/* Paged KV write ([VT] ReshapeAndCache). For token t < num_slots with slot
 * s = slot_mapping[t]: k[t] and v[t] (all kv heads) are copied verbatim to row
 * s % block_size of page s / block_size. A slot < 0 skips its token (the
 * padding convention); so does a slot >= num_blocks * block_size. Tokens at
 * or past num_slots are not read (graph padding).
 *   k, v: device [>= num_slots][n_kv_head][head_dim] fp32, 16-byte aligned.
 *   slot_mapping: device int64[num_slots]. Two tokens mapped to one slot
 *   race (either may win). num_slots == 0 enqueues nothing. One launch. */
int fa_paged_append(const fa_paged_cache *cache, const float *k, const float *v,
                    const int64_t *slot_mapping, int num_slots, void *stream);

/* Workspace fa_paged_attention needs (independent of the batch); 0 if
 * head_dim is invalid. */
size_t fa_paged_workspace_bytes(int head_dim);

/* Causal GQA attention of a varlen batch over a paged cache ([VT]
 * PagedAttention, causal path; the key rows of every query, its own
 * included, must already be written, e.g. by fa_paged_append). Request r
 * owns query tokens t in [query_start_loc[r], query_start_loc[r+1]); with
 * query_len = query_start_loc[r+1] - query_start_loc[r], token t sits at
 * absolute position p = seq_lens[r] - query_len + (t - query_start_loc[r])
 * (bottom-right alignment: seq_lens[r] counts the context including this
 * chunk). Query head h reads kv head h / G; its key j <= p is row j % bs of
 * page block_table[r * max_blocks_per_seq + j / bs] (bs = block_size).
 *     s_j = scale * (q[t][h] . k_j);  out[t][h] = sum_j softmax(s)_j v_j
 * over j in [0, p], or over [p - window_left, p] when window_left >= 0
 * ([VT] AttentionWindow (left, right), bottom-right aligned: window_right,
 * which must then be >= 0, admits no key past p under the causal bound).
 * window_left < 0 is full causal attention. One query block of one request
 * and kv head is the unit of work, and the blocks of all requests share one
 * stream-K launch (key tiles outside the window are skipped) that needs no
 * device-to-host read: the batch metadata stays on the device.
 *   q, out: device [num_tokens][n_head][head_dim] fp32, 16-byte aligned.
 *   lse:    NULL, or device [n_head][num_tokens] fp32 receiving
 *           ln sum_j exp(s_j) per query row (the state fa_merge_attn_states
 *           combines).
 *   query_start_loc: device int32[num_reqs + 1], non-decreasing, within
 *           [0, num_tokens]. seq_lens: device int32[num_reqs], with
 *           query_len <= seq_lens[r] <= max_blocks_per_seq * block_size.
 *   block_table: device int32[num_reqs][max_blocks_per_seq], entries in
 *           [0, num_blocks).
 *   0 <= num_reqs <= 1024; num_tokens == 0 or num_reqs == 0 enqueue nothing.
 *   ws, ws_bytes: device scratch of at least fa_paged_workspace_bytes().
 * The device metadata is not checked against those rules on the host (it is
 * never read there); out-of-rule values are clamped on the device so that no
 * access leaves the buffers, and the rows they touch are unspecified.
 * Tokens outside every request's range are not written. Head dims, group
 * sizes and the scale rule as fa_prefill. Two launches on `stream`.
 * The kernel counts its schedule in 32 bits (as fa_prefill); since the batch
 * is not read on the host, the host bounds it by n_kv_head * (num_tokens / BQ
 * + num_reqs) query blocks of at most max_blocks_per_seq * block_size / 32 + 1
 * tiles (BQ from fa_prefill_tile_shape) and returns FA_EUNSUPPORTED when that
 * bound exceeds 2^31 - 1 schedule units (4 per tile, 5 per block). */
int fa_paged_attention(const fa_paged_cache *cache, const float *q, int num_tokens,
                       int n_head, const int *query_start_loc, const int *seq_lens,
                       int num_reqs, const int *block_table, int max_blocks_per_seq,
                       int window_left, int window_right, float scale, float *out,
                       float *lse, void *ws, size_t ws_bytes, void *stream);

/* Workspace fa_paged_decode needs: the split-KV partials of fa_decode's
 * scheme, sized by the request count, head counts and max_seq_len_hint; 0 if
 * an argument is invalid. */
size_t fa_paged_decode_workspace_bytes(int num_reqs, int n_head, int n_kv_head, int head_dim,
                                       int max_seq_len_hint);

/* Decode step over a paged cache: request r has exactly one query token, row
 * r of q, at position p = seq_lens[r] - 1, and attends keys [0, p] (or
 * [p - window_left, p] when window_left >= 0, with window_right >= 0 and
 * otherwise unused, as in fa_paged_attention), read through the block table
 * as in fa_paged_attention ([VT] PagedAttention on a batch of decode tokens).
 * The same computation as fa_paged_attention on such a batch, with
 * fa_decode's split-KV schedule ([FA] "Decode-mode flash attention"): every
 * request's keys are cut into splits by fa_decode_plan, all requests' splits
 * share one work list, and a combine pass merges the partials in ascending
 * order, so a fixed launch is bit-reproducible.
 *   cache->block_size must be a multiple of 16 (FA_EUNSUPPORTED otherwise):
 *       16 aligned rows then share a page, so a 16-key group needs one
 *       block-table lookup.
 *   q, out: device [num_reqs][n_head][head_dim] fp32, 16-byte aligned.
 *   lse: NULL, or device [n_head][num_reqs] fp32 (ln sum_j exp(s_j)).
 *   seq_lens: device int32[num_reqs]; values are clamped on the device to
 *       max_blocks_per_seq * block_size, and a request with seq_lens < 1
 *       gets NaN rows (no key).
 *   block_table: device int32[num_reqs][max_blocks_per_seq] (entries
 *       clamped on the device into [0, num_blocks)).
 *   max_seq_len_hint: host upper bound on seq_lens, 1..max_blocks_per_seq *
 *       block_size ([VT] PagedAttentionArgs max_seq_len); sizes the launch.
 *       Longer requests are still computed exactly.
 *   ws, ws_bytes: at least fa_paged_decode_workspace_bytes(...), 16-byte
 *       aligned.
 * No device metadata is read on the host. num_reqs == 0 enqueues nothing.
 * Two launches on `stream`. The 32-bit item limit of fa_decode applies to
 * num_reqs * n_kv_head. */
int fa_paged_decode(const fa_paged_cache *cache, const float *q, int num_reqs, int n_head,
                    const int *seq_lens, const int *block_table, int max_blocks_per_seq,
                    int max_seq_len_hint, int window_left, int window_right, float scale,
                    float *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/* LSE merge of two attention results over disjoint key sets ([VT]
 * MergeAttnStates), in fp32. Per (token t, head h), with L_p, L_s the two
 * log-sum-exps (a +inf read as -inf):
 *   m = max(L_p, L_s); w_p = exp(L_p - m); w_s = exp(L_s - m);
 *   out = (w_p out_p + w_s out_s) / (w_p + w_s); out_lse = m + ln(w_p + w_s)
 * and when L_p = L_s = -inf (neither side saw a key): out = out_p and
 * out_lse = -inf. Tokens t >= prefill_tokens_with_context (when that is
 * >= 0) take out_s and L_s unchanged.
 *   out, prefix_out, suffix_out: device [num_tokens][n_head][head_dim] fp32,
 *       16-byte aligned; out may be either input.
 *   out_lse (NULL: not written), prefix_lse, suffix_lse: device
 *       [n_head][num_tokens] fp32; out_lse may be either input LSE.
 *   head_dim a multiple of 4 in [4, 4096]. One launch. */
int fa_merge_attn_states(float *out, float *out_lse, const float *prefix_out,
                         const float *prefix_lse, const float *suffix_out,
                         const float *suffix_lse, int num_tokens, int n_head, int head_dim,
                         int prefill_tokens_with_context, void *stream);

/* Message for a return code (static storage). */
const char *fa_strerror(int code);

/* Name of the HIP runtime error behind the calling thread's most recent
 * FA_EHIP return ("hipSuccess" if there was none); static storage. */
const char *fa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
