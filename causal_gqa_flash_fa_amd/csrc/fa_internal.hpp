// Internal launcher interface between the C-ABI layer (fa_api.cpp) and the
// kernel translation units. Arguments reaching these functions have already
// been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Capacity of the fp16 shadow of a Q4_0 cache (equal to FA_SHADOW_*_MAX).
constexpr int kShadowSinkMax = 8;
constexpr int kShadowWinMax = 256;

// fp16 shadow of a Q4_0 cache; sink == win == 0 means none. Buffers hold
// [n_slots][n_kv][kShadowSinkMax | kShadowWinMax][hd] binary16 values and
// win_pos [n_slots][kShadowWinMax] the position held by each ring row.
struct ShadowArgs {
    uint16_t *k_sink, *v_sink, *k_win, *v_win;
    int *win_pos;
    int sink, win;
};

// Key s of a query at position p is read from the shadow (not the Q4_0
// body): sink rows always, ring rows while recent and not overwritten.
__device__ __forceinline__ bool shadow_key(const ShadowArgs &sh, const int *win_pos, int s,
                                           int p) {
    if (s < sh.sink) return true;
    return sh.win > 0 && s > p - sh.win && win_pos[s % kShadowWinMax] == s;
}

// Decode shadow work items (fa_shadow.hpp): the softmax partial of each
// query row over its fp16 shadow keys. Work item = (query i, kv head) x chunk
// group; query i sits at d_pos[i] (one per slot, shadow buffers of slot i;
// d_pos NULL: at pos0 + i, shadow buffers of one slot). Partial of head g of
// item it, chunk group cg: row (it * chunk_groups + cg) * G + g of m_out,
// l_out, acc_out.
struct ShadowPassArgs {
    const float *q;               // [n_q][n_head][hd]
    const int *d_pos;             // decode positions, or NULL
    int pos0, n_q, n_head, n_kv, max_seq;
    int sink, win;                // key set
    float qscale;                 // scale * log2(e)
    ShadowArgs sh;
    int chunk_groups;             // work-groups per (query, kv head)
    int chunks_per_group;         // 64-key chunks folded by each
    float *m_out, *l_out, *acc_out;
};

struct AppendArgs {
    const float *k_new, *v_new;   // [n][n_kv][hd]
    void *k, *v;                  // slot base of the cache: [n_kv][max_seq][row]
    int n, n_kv, head_dim, max_seq, pos0;
    // NULL: input row t goes to position pos0 + t of the slot at k/v.
    // Else input row t belongs to slot t (base k/v + t * slot_bytes) and goes
    // to position d_pos[t], read on the device; out-of-range positions skip.
    const int *d_pos;
    size_t slot_bytes;
    ShadowArgs sh;                // Q4_0 only: mirror rows into the fp16 shadow
};

// Geometry of the prefill work-group: 8 waves of 16 (position, head) rows,
// two waves per SIMD (one work-group per CU), on 16x16x4 fp32 MFMAs; the
// same 128 rows as 4 waves of 32 on 32x32x2 MFMAs, which timed 3.5% slower
// on the 8k Q4_0 prefill (one wave per SIMD exposes its waits and barriers).
constexpr int kPrefillWaves = 8;
constexpr int kPrefillRowsPerWave = 16;
constexpr int kPrefillKeyTile = 32;
// Stream-K prefill grid: at most one work-group per CU of a 256-CU MI355X.
constexpr int kPrefillMaxWorkGroups = 256;
// Decode: single-wave work-groups folding tiles of 64 keys (one per lane).
constexpr int kDecodeKeyTile = 64;
// Split plan constants: about kDecodeKps keys per split, at most
// kDecodeSplitCap splits per slot. Splits are the schedulable work items, so
// they set how evenly the stream-K runs cut the keys: one key tile per split
// timed ~1.3% faster than two on the 64-slot fp32-cache decode (the same on
// Q4_0), four tiles 2-6% slower.
constexpr int kDecodeKps = 64;
constexpr int kDecodeSplitCap = 512;
// Work-groups of the decode partial pass: 8 waves per CU of a 256-CU MI355X
// for Q4_0 tiles (bound by issue: two waves per SIMD hide each other's
// latencies; one wave per SIMD was 46% slower). fp32 tiles are bound by HBM,
// and one wave per SIMD (4 per CU) streams them ~0.6% faster than two, with
// half the run boundaries and partials.
constexpr int kDecodeMaxWaves = 2048;
constexpr int kDecodeMaxWavesF32 = 1024;
// The fp16 hi/lo Q4_0 decode: two waves per SIMD as well (its MFMA results
// then stay in VGPRs; at one wave per SIMD the compiler moved them through
// AGPRs every tile).
constexpr int kDecodeMaxWavesHilo = 2048;
// SIMDs of a 256-CU MI355X, and the run weights of the first- and
// second-dispatched wave of a SIMD when a decode grid holds two per SIMD:
// for the fp32-MFMA Q4_0 tiles (bound by instruction issue, where the
// arbiter's preference for the older wave weighs most) and for the fp16
// hi/lo tiles. Set by timing the 64-slot decode over a sweep of ratios.
constexpr int kDecodeSimds = 1024;
constexpr int kDecodeWeightFirst = 5;
constexpr int kDecodeWeightSecond = 3;
constexpr int kDecodeWeightFirstHilo = 3;
constexpr int kDecodeWeightSecondHilo = 2;

// Requests of one paged prefill launch (their table sits in LDS).
constexpr int kPagedMaxReqs = 1024;

// A query block cut between work-groups: its pieces and where its rows go
// (position p of the block is query token p + tok). Filled by the prefill
// kernel, read by its combine launch.
struct CutSeg {
    int piece0, n_pieces, q0, q1, kvh, tok, pad0, pad1;
};
// Cut segments of one prefill launch: every cut sits at a run boundary, so
// there are fewer than kPrefillMaxWorkGroups of them.
struct CutList {
    int count;
    int pad[7];
    CutSeg seg[kPrefillMaxWorkGroups];
};

struct PrefillArgs {
    const float *q;               // [n][n_head][hd]
    float *out;                   // [n][n_head][hd]
    float *lse;                   // NULL or [n_head][n]: ln sum_j exp(scale q.k_j)
    const void *k, *v;            // slot base: [n_kv][max_seq][row]; paged: page 0
    unsigned long long *stats;    // NULL or [2]
    float *ws_m, *ws_l, *ws_acc;  // pieces of cut segments: [piece][rows](+[hd])
    CutList *cuts;
    int n, pos0, n_head, n_kv, max_seq;
    int sink, win;
    float qscale;                 // scale * log2(e)
    int n_qblocks;
    int n_wg;                     // work-groups of the stream-K grid
    // Paged varlen batch (paged instances; n = total query tokens): request
    // r holds query tokens [qsl[r], qsl[r+1]) at positions
    // seq_lens[r] - qlen_r + i, and its key row j sits in page
    // block_table[r * bt_stride + j / block_size], row j % block_size, at
    // float page * blk_stride + (row * n_kv + kv head) * hd of k / v.
    const int *qsl, *seq_lens, *block_table;
    int n_req, bt_stride, block_size, num_blocks;
    long long blk_stride;
    // fp16 shadow (Q4_0): buffers of this slot. Its keys are skipped here;
    // the shadow-mode launch left each row's partial in sh_m, sh_l
    // ([n][n_head]) and out (acc), and the first piece of every segment
    // starts from it. The shadow mode itself writes them.
    ShadowArgs sh;
    const float *sh_m, *sh_l;
};

struct DecodeArgs {
    const float *q;               // [n_slots][n_head][hd]
    const int *pos;               // device [n_slots]
    const void *k, *v;            // cache base: [n_slots_cache][n_kv][max_seq][row]
    float *ws_m, *ws_l, *ws_acc;  // partials [n_partials][G] (+[hd])
    int *seg_table;               // [n_slots * n_kv][2]: first partial, partial count
    float *out;                   // [n_slots][n_head][hd]
    unsigned long long *stats;
    int n_slots, n_head, n_kv, max_seq;
    int sink, win;
    float qscale;
    int kps, cap;                 // split plan constants
    // fp16 shadow (Q4_0): buffers of slot 0; its keys are skipped here and
    // folded by the shadow pass into sh_groups partials per segment, rows
    // (seg * sh_groups + c) * G + g of sh_m, sh_l, sh_acc.
    ShadowArgs sh;
    const float *sh_m, *sh_l, *sh_acc;
    int sh_groups;
    // The shadow pass's work items run as the first sh_waves work-groups of
    // the partial launch (shp.m_out/l_out/acc_out = sh_m/sh_l/sh_acc).
    ShadowPassArgs shp;
    int sh_waves;
    // Paged batch (paged fp32 instances): slot s is request s, whose query
    // sits at position seq_lens[s] - 1 (pos is unused) and whose key row j
    // is row j % block_size of page block_table[s * bt_stride + j /
    // block_size], at float page * blk_stride + (row * n_kv + kv head) * hd.
    // block_size is a multiple of 16, so 16 aligned rows share a page.
    const int *seq_lens, *block_table;
    int bt_stride, block_size, num_blocks;
    long long blk_stride;
    float *lse;                   // NULL or [n_head][n_slots]: ln sum_j exp(scale q.k_j)
};

// Visited key tiles of the query block [q0, q1] ([FA] fc_attn_tile_in_window
// over the union of the block's key sets): the causal walk has q1/bk + 1
// tiles; with a window, tiles below the sink or reaching the union window
// [q0 - win + 1, q1] are visited and the rest are skipped. The host sizes
// the stream-K grid and checks the schedule's range with this function and
// the kernel walks its tiles with it, so the two cannot disagree.
struct SegTiles {
    int walked, nsink, wt, count;       // visited tile i -> i < nsink ? i : wt + i - nsink
    __host__ __device__ int tile(int i) const { return i < nsink ? i : wt + i - nsink; }
};

__host__ __device__ inline SegTiles seg_tiles(int q0, int q1, int sink, int win, int bk) {
    SegTiles t;
    t.walked = q1 / bk + 1;
    t.nsink = t.walked;
    t.wt = t.walked;
    t.count = t.walked;
    if (win > 0) {
        const int win_lo = q0 - win + 1;
        const int wt = win_lo > 0 ? win_lo / bk : 0;
        int nsink = ((sink > 0 ? sink : 0) + bk - 1) / bk;
        if (nsink > t.walked) nsink = t.walked;
        if (wt > nsink) {
            t.nsink = nsink;
            t.wt = wt;
            t.count = nsink + (t.walked - wt);
        }
    }
    return t;
}

// Stream-K prefill schedule units: a visited tile is kTileUnits units and
// starting a segment costs kSegUnits more (measured: a segment switch,
// output stores plus the next Q load and first-tile latency, costs about one
// ~9 us tile; 4, 5 and 6 units time the same within noise). The kernel
// counts units in 32-bit integers, so the host refuses a launch whose total
// exceeds kMaxScheduleUnits.
constexpr int kTileUnits = 4;
constexpr int kSegUnits = 5;
constexpr long long kMaxScheduleUnits = 0x7fffffffLL;

inline int prefill_q_positions(int group) {
    return kPrefillWaves * kPrefillRowsPerWave / group;
}

hipError_t launch_append(int format, const AppendArgs &a, hipStream_t s);
hipError_t launch_prefill(int format, int head_dim, int group, const PrefillArgs &a,
                          hipStream_t s);
hipError_t launch_paged_prefill(int head_dim, int group, const PrefillArgs &a, hipStream_t s);
// fp16-shadow keys of a Q4_0 slot cache on the prefill MFMA path: leaves each
// row's partial in sh_m, sh_l (m, l) and out (acc, unnormalised).
hipError_t launch_shadow_prefill(int head_dim, int group, const PrefillArgs &a, hipStream_t s);

// Paged KV append ([VT] ReshapeAndCache): token t < n goes to slot
// slot_mapping[t] (page slot / block_size, row slot % block_size); slots < 0
// or past the cache are skipped.
struct PagedAppendArgs {
    const float *k_new, *v_new;   // [n][n_kv][hd]
    float *k, *v;
    const long long *slot_mapping;
    int n, n_kv, head_dim, block_size, num_blocks;
    long long blk_stride;
};
hipError_t launch_paged_append(const PagedAppendArgs &a, hipStream_t s);

// LSE merge of two attention states ([VT] MergeAttnStates).
struct MergeArgs {
    float *out, *out_lse;         // [T][H][D], [H][T] or NULL
    const float *p_out, *p_lse, *s_out, *s_lse;
    int T, H, D, prefill_tokens_with_context;
};
hipError_t launch_merge(const MergeArgs &a, hipStream_t s);
hipError_t launch_decode(int format, int head_dim, int group, const DecodeArgs &a, int waves,
                         hipStream_t s);
hipError_t launch_paged_decode(int head_dim, int group, const DecodeArgs &a, int waves,
                               hipStream_t s);
// The combine pass of fa_decode alone (decode partials already written).
hipError_t launch_decode_combine(int head_dim, int group, const DecodeArgs &a, hipStream_t s);
// Q4_0 decode on fp16 MFMA with hi/lo-split operands (fa_decode_q4_hilo):
// partial pass over a Q4_0 cache without fp16 shadow, then the combine.
hipError_t launch_decode_hilo(int head_dim, int group, const DecodeArgs &a, int waves,
                              hipStream_t s);

// Host copy of the device plan ([FA] fc_attn_dec_plan).
__host__ __device__ inline int decode_plan(int seq_len, int kps, int cap, int tile, int *n_splits,
                       int *split_len) {
    int n = (seq_len + kps - 1) / kps;
    if (n < 1) n = 1;
    if (n > cap) n = cap;
    int len = (seq_len + n - 1) / n;
    len = (len + tile - 1) / tile * tile;
    *n_splits = n;
    *split_len = len;
    return (seq_len + len - 1) / len;
}

}  // namespace fa
