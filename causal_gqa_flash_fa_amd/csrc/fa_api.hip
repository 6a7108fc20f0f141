// C-ABI layer of libfa: argument validation, geometry, and dispatch to the
// kernel launchers. Nothing here allocates device memory or synchronises.
// Unsupported or inconsistent arguments are refused with a code before any
// launch ([VT] kernel registration contract: fail loudly, never truncate).
#include <math.h>
#include <string.h>

#include "../../include/fa.h"
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;
int g_device_ok[kMaxDevices];   // 0 unknown, 1 gfx950, -1 other
int g_device_cus[kMaxDevices];  // compute units of each checked device

bool dim_ok(int head_dim) { return head_dim == 64 || head_dim == 128 || head_dim == 256; }
bool group_ok(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

int check_cache(const fa_cache *c) {
    if (!c) return FA_ENULL;
    if (c->format != FA_KV_F32 && c->format != FA_KV_Q4_0) return FA_EUNSUPPORTED;
    if (!dim_ok(c->head_dim)) return FA_EUNSUPPORTED;
    if (c->n_slots < 1 || c->n_kv_head < 1 || c->max_seq < 1) return FA_EINVAL;
    if (!c->k || !c->v) return FA_ENULL;
    if (c->shadow_sink < 0 || c->shadow_sink > FA_SHADOW_SINK_MAX || c->shadow_win < 0 ||
        c->shadow_win > FA_SHADOW_WIN_MAX)
        return FA_EINVAL;
    if (c->shadow_sink > 0 || c->shadow_win > 0) {
        if (c->format != FA_KV_Q4_0) return FA_EUNSUPPORTED;   // the shadow exempts Q4_0 rows
        if (c->shadow_sink > 0 && (!c->k_sink || !c->v_sink)) return FA_ENULL;
        if (c->shadow_win > 0 && (!c->k_win || !c->v_win || !c->win_pos)) return FA_ENULL;
    }
    return FA_OK;
}

int check_heads(const fa_cache *c, int n_head) {
    if (n_head < 1 || n_head % c->n_kv_head != 0) return FA_EINVAL;
    if (!group_ok(n_head / c->n_kv_head)) return FA_EUNSUPPORTED;
    return FA_OK;
}

int check_scale(float scale) {
    return (isfinite(scale) && scale > 0.0f) ? FA_OK : FA_EINVAL;
}

static_assert(fa::kShadowSinkMax == FA_SHADOW_SINK_MAX && fa::kShadowWinMax == FA_SHADOW_WIN_MAX,
              "shadow capacity");

// The cache's fp16 shadow with its buffers offset to `slot` (all zero if the
// cache has none).
fa::ShadowArgs shadow_args(const fa_cache *c, int slot) {
    fa::ShadowArgs sh{};
    if (c->shadow_sink <= 0 && c->shadow_win <= 0) return sh;
    const size_t hd = (size_t)c->head_dim, nkv = (size_t)c->n_kv_head;
    sh.sink = c->shadow_sink;
    sh.win = c->shadow_win;
    if (sh.sink > 0) {
        const size_t off = (size_t)slot * nkv * fa::kShadowSinkMax * hd;
        sh.k_sink = (uint16_t *)c->k_sink + off;
        sh.v_sink = (uint16_t *)c->v_sink + off;
    }
    if (sh.win > 0) {
        const size_t off = (size_t)slot * nkv * fa::kShadowWinMax * hd;
        sh.k_win = (uint16_t *)c->k_win + off;
        sh.v_win = (uint16_t *)c->v_win + off;
        sh.win_pos = c->win_pos + (size_t)slot * fa::kShadowWinMax;
    }
    return sh;
}

size_t slot_stride_bytes(const fa_cache *c) {
    return (size_t)c->n_kv_head * c->max_seq * fa_cache_row_bytes(c->format, c->head_dim);
}

// The HIP error behind this thread's most recent FA_EHIP.
thread_local hipError_t g_last_hip_error = hipSuccess;

// Decode scratch owned by the library, for fa_decode_noalloc: every GPU holds
// its own copy of this array for the life of the process. Its name is a
// host-side stand-in in host code, never a device address: fa_init resolves
// each device's address once (hipGetSymbolAddress, with that device current)
// into g_scratch, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_SCRATCH_BYTES];
void *g_scratch[kMaxDevices];

int hip_rc(hipError_t e) {
    if (e == hipSuccess) return FA_OK;
    g_last_hip_error = e;
    return FA_EHIP;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

size_t fa_cache_row_bytes(int format, int head_dim) {
    if (!dim_ok(head_dim)) return 0;
    if (format == FA_KV_F32) return (size_t)head_dim * 4;
    if (format == FA_KV_Q4_0) return (size_t)fa::q4_row_bytes(head_dim);
    return 0;
}

size_t fa_cache_bytes(const fa_cache *c) {
    if (!c || c->n_slots < 1 || c->n_kv_head < 1 || c->max_seq < 1) return 0;
    const size_t rb = fa_cache_row_bytes(c->format, c->head_dim);
    return (size_t)c->n_slots * slot_stride_bytes(c) * (rb ? 1 : 0);
}

int fa_init(void) {
    int dev = 0;
    if (hip_rc(hipGetDevice(&dev))) return FA_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return FA_EDEVICE;
    if (g_device_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hip_rc(hipGetDeviceProperties(&prop, dev))) return FA_EHIP;
        const bool gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        if (gfx950) {
            // this device's copy of the decode scratch (the device is current)
            void *p = nullptr;
            if (hip_rc(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))) return FA_EHIP;
            if (!p) return FA_EHIP;
            g_scratch[dev] = p;
        }
        g_device_cus[dev] = prop.multiProcessorCount;
        g_device_ok[dev] = gfx950 ? 1 : -1;
    }
    return g_device_ok[dev] == 1 ? FA_OK : FA_EDEVICE;
}

int fa_kv_append(const fa_cache *cache, int slot, int pos0, int n, const float *k_new,
                 const float *v_new, void *stream) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if (slot < 0 || slot >= cache->n_slots || pos0 < 0 || n < 0) return FA_EINVAL;
    if ((long long)pos0 + n > cache->max_seq) return FA_ERANGE;
    if (n == 0) return FA_OK;
    if (!k_new || !v_new) return FA_ENULL;
    if ((rc = fa_init())) return rc;
    fa::AppendArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k = (uint8_t *)cache->k + (size_t)slot * slot_stride_bytes(cache);
    a.v = (uint8_t *)cache->v + (size_t)slot * slot_stride_bytes(cache);
    a.n = n;
    a.n_kv = cache->n_kv_head;
    a.head_dim = cache->head_dim;
    a.max_seq = cache->max_seq;
    a.pos0 = pos0;
    a.d_pos = nullptr;
    a.slot_bytes = 0;
    a.sh = shadow_args(cache, slot);
    return hip_rc(fa::launch_append(cache->format, a, (hipStream_t)stream));
}

int fa_kv_append_slots(const fa_cache *cache, const int *d_pos, int n_slots, const float *k_new,
                       const float *v_new, void *stream) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if (n_slots < 0 || n_slots > cache->n_slots) return FA_EINVAL;
    if (n_slots == 0) return FA_OK;
    if (!d_pos || !k_new || !v_new) return FA_ENULL;
    if ((rc = fa_init())) return rc;
    fa::AppendArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k = cache->k;
    a.v = cache->v;
    a.n = n_slots;
    a.n_kv = cache->n_kv_head;
    a.head_dim = cache->head_dim;
    a.max_seq = cache->max_seq;
    a.pos0 = 0;
    a.d_pos = d_pos;
    a.slot_bytes = slot_stride_bytes(cache);
    a.sh = shadow_args(cache, 0);
    return hip_rc(fa::launch_append(cache->format, a, (hipStream_t)stream));
}

int fa_prefill_tile_shape(int n_head, int n_kv_head, int head_dim, int *q_positions,
                          int *key_tile) {
    if (n_kv_head < 1 || n_head < 1 || n_head % n_kv_head) return FA_EINVAL;
    if (!group_ok(n_head / n_kv_head) || !dim_ok(head_dim)) return FA_EUNSUPPORTED;
    if (q_positions) *q_positions = fa::prefill_q_positions(n_head / n_kv_head);
    if (key_tile) *key_tile = fa::kPrefillKeyTile;
    return FA_OK;
}

namespace {
// Stream-K prefill layout: the list of cut segments and their pieces.
struct PrefillLayout {
    int n_qblocks;
    size_t pieces, table_bytes, m_off, l_off, acc_off;
    size_t sh_m_off, sh_l_off;    // fp16-shadow partial of every row: m, l ([n][n_head])
    size_t total;
};

PrefillLayout prefill_layout(int n, int n_head, int n_kv_head, int head_dim) {
    PrefillLayout p;
    const int bq = fa::prefill_q_positions(n_head / n_kv_head);
    const size_t rows = (size_t)fa::kPrefillWaves * fa::kPrefillRowsPerWave;
    (void)n_kv_head;
    p.n_qblocks = (n + bq - 1) / bq;
    // cut segments own at most 2 * (work-groups - 1) pieces in total
    p.pieces = 2 * (size_t)fa::kPrefillMaxWorkGroups;
    p.table_bytes = align256(sizeof(fa::CutList));
    p.m_off = p.table_bytes;
    p.l_off = p.m_off + align256(p.pieces * rows * sizeof(float));
    p.acc_off = p.l_off + align256(p.pieces * rows * sizeof(float));
    const size_t qrows = (size_t)n * n_head;
    p.sh_m_off = align256(p.acc_off + p.pieces * rows * (size_t)head_dim * sizeof(float));
    p.sh_l_off = p.sh_m_off + align256(qrows * sizeof(float));
    p.total = p.sh_l_off + qrows * sizeof(float);
    return p;
}

// Visited key tiles of a prefill call per kv head (the stream-K grid never
// needs more work-groups than that) and the schedule units the kernel counts
// for them, both from the kernel's own tile walk.
struct PrefillWork {
    long long tiles, units;
};

PrefillWork prefill_work(int n, int pos0, int bq, int sink, int win) {
    PrefillWork w{0, 0};
    const long long end = (long long)pos0 + n;
    for (long long b0 = pos0; b0 < end; b0 += bq) {
        const int q0 = (int)b0;
        const int q1 = (int)(b0 + bq - 1 < end - 1 ? b0 + bq - 1 : end - 1);
        const int c = fa::seg_tiles(q0, q1, sink, win, fa::kPrefillKeyTile).count;
        w.tiles += c;
        w.units += c > 0 ? (long long)c * fa::kTileUnits + fa::kSegUnits : 0;
    }
    return w;
}

// The same for the fp16-shadow launch: per query block, its shadow keys in
// 32-key tiles (the sink positions, then every position a row's ring window
// reaches).
PrefillWork shadow_work(int n, int pos0, int bq, int sh_sink, int sh_win) {
    PrefillWork w{0, 0};
    const long long end = (long long)pos0 + n;
    for (long long b0 = pos0; b0 < end; b0 += bq) {
        const long long q0 = b0, q1 = b0 + bq - 1 < end - 1 ? b0 + bq - 1 : end - 1;
        const long long n_sk = sh_sink < q1 + 1 ? sh_sink : q1 + 1;
        const long long wlo = sh_sink > q0 - sh_win + 1 ? sh_sink : q0 - sh_win + 1;
        const long long nk = n_sk + (sh_win > 0 && q1 >= wlo ? q1 - wlo + 1 : 0);
        const long long c = (nk + fa::kPrefillKeyTile - 1) / fa::kPrefillKeyTile;
        w.tiles += c;
        w.units += c > 0 ? c * fa::kTileUnits + fa::kSegUnits : 0;
    }
    return w;
}
}  // namespace

size_t fa_prefill_workspace_bytes(int n, int n_head, int n_kv_head, int head_dim) {
    if (n < 0 || n_head < 1 || n_kv_head < 1 || n_head % n_kv_head ||
        !group_ok(n_head / n_kv_head) || !dim_ok(head_dim))
        return 0;
    return prefill_layout(n, n_head, n_kv_head, head_dim).total;
}

int fa_prefill(const fa_cache *cache, int slot, const float *q, int pos0, int n, int n_head,
               int attn_sink, int attn_win, float scale, float *out, void *ws, size_t ws_bytes,
               unsigned long long *tile_stats, void *stream) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = check_heads(cache, n_head))) return rc;
    if ((rc = check_scale(scale))) return rc;
    if (slot < 0 || slot >= cache->n_slots || pos0 < 0 || n < 0) return FA_EINVAL;
    if ((long long)pos0 + n > cache->max_seq) return FA_ERANGE;
    if (n == 0) return FA_OK;
    if (!q || !out || !ws) return FA_ENULL;
    const int group = n_head / cache->n_kv_head;
    const int bq = fa::prefill_q_positions(group);
    const int sink = attn_sink < 0 ? 0 : attn_sink;
    const bool shadowed = cache->shadow_sink > 0 || cache->shadow_win > 0;
    // the stream-K schedule counts its units in 32 bits: refuse what does not fit
    const PrefillWork wk = prefill_work(n, pos0, bq, sink, attn_win);
    if (wk.units > fa::kMaxScheduleUnits / cache->n_kv_head) return FA_EUNSUPPORTED;
    const PrefillWork swk = shadowed ? shadow_work(n, pos0, bq, cache->shadow_sink,
                                                   cache->shadow_win)
                                     : PrefillWork{0, 0};
    if (swk.units > fa::kMaxScheduleUnits / cache->n_kv_head) return FA_EUNSUPPORTED;
    const PrefillLayout lay = prefill_layout(n, n_head, cache->n_kv_head, cache->head_dim);
    if (ws_bytes < lay.total) return FA_EWORKSPACE;
    if ((rc = fa_init())) return rc;
    int dev = 0;
    if (hip_rc(hipGetDevice(&dev))) return FA_EHIP;
    long long n_wg = g_device_cus[dev] < fa::kPrefillMaxWorkGroups ? g_device_cus[dev]
                                                                   : fa::kPrefillMaxWorkGroups;
    const long long tiles = (long long)cache->n_kv_head * wk.tiles;
    if (tiles < n_wg) n_wg = tiles;
    if (n_wg < 1) n_wg = 1;
    uint8_t *wsb = (uint8_t *)ws;
    fa::PrefillArgs a{};
    a.q = q;
    a.out = out;
    a.lse = nullptr;
    a.k = (const uint8_t *)cache->k + (size_t)slot * slot_stride_bytes(cache);
    a.v = (const uint8_t *)cache->v + (size_t)slot * slot_stride_bytes(cache);
    a.stats = tile_stats;
    a.cuts = (fa::CutList *)wsb;
    a.ws_m = (float *)(wsb + lay.m_off);
    a.ws_l = (float *)(wsb + lay.l_off);
    a.ws_acc = (float *)(wsb + lay.acc_off);
    a.n = n;
    a.pos0 = pos0;
    a.n_head = n_head;
    a.n_kv = cache->n_kv_head;
    a.max_seq = cache->max_seq;
    a.sink = sink;
    a.win = attn_win;
    a.qscale = scale * fa::kLog2e;
    a.n_qblocks = lay.n_qblocks;
    a.n_wg = (int)n_wg;
    a.sh = shadow_args(cache, slot);
    a.sh_m = (const float *)(wsb + lay.sh_m_off);
    a.sh_l = (const float *)(wsb + lay.sh_l_off);
    if (shadowed) {
        // each row's shadow-key partial (m, l to the workspace, acc to out),
        // from the same kernel in its shadow mode: per query block, the
        // union of its rows' shadow keys in 32-key tiles
        fa::PrefillArgs sa = a;
        sa.stats = nullptr;
        sa.lse = nullptr;
        const long long sh_tiles = swk.tiles * cache->n_kv_head;
        long long sh_wg = g_device_cus[dev] < fa::kPrefillMaxWorkGroups ? g_device_cus[dev]
                                                                        : fa::kPrefillMaxWorkGroups;
        if (sh_tiles < sh_wg) sh_wg = sh_tiles;
        sa.n_wg = sh_wg < 1 ? 1 : (int)sh_wg;
        if ((rc = hip_rc(fa::launch_shadow_prefill(cache->head_dim, group, sa,
                                                   (hipStream_t)stream))))
            return rc;
    }
    return hip_rc(fa::launch_prefill(cache->format, cache->head_dim, group, a,
                                     (hipStream_t)stream));
}

void fa_decode_plan_params(int *kps, int *cap, int *key_tile) {
    if (kps) *kps = fa::kDecodeKps;
    if (cap) *cap = fa::kDecodeSplitCap;
    if (key_tile) *key_tile = fa::kDecodeKeyTile;
}

int fa_decode_plan(int seq_len, int *n_splits, int *split_len) {
    if (seq_len < 1) return FA_EINVAL;
    int n, len;
    const int live = fa::decode_plan(seq_len, fa::kDecodeKps, fa::kDecodeSplitCap,
                                     fa::kDecodeKeyTile, &n, &len);
    if (n_splits) *n_splits = n;
    if (split_len) *split_len = len;
    return live;
}

namespace {
// Decode work distribution for a launch: waves and the workspace layout.
struct DecodeLayout {
    int waves;
    size_t max_partials, table_bytes, m_off, l_off, acc_off;
    int sh_groups;                // fp16-shadow partials per segment (0: no shadow)
    size_t sh_m_off, sh_l_off, sh_acc_off, total;
};

// Shadow-pass work-groups per (query, kv head) in decode: one per 64-key chunk
// of the largest shadow key set.
int shadow_groups(const fa_cache *c) {
    if (c->shadow_sink <= 0 && c->shadow_win <= 0) return 0;
    return (c->shadow_sink + c->shadow_win + 63) / 64;
}

DecodeLayout decode_layout_of(int format, int n_kv_head, int head_dim, int sh_groups, int n_slots,
                              int n_head, int max_ctx) {
    DecodeLayout d;
    const size_t nsegs = (size_t)n_slots * n_kv_head;
    const int group = n_head / n_kv_head;
    const size_t items = nsegs * (size_t)fa_decode_plan(max_ctx, nullptr, nullptr);
    const size_t max_waves =
        (size_t)(format == FA_KV_F32 ? fa::kDecodeMaxWavesF32 : fa::kDecodeMaxWaves);
    d.waves = (int)(items < max_waves ? (items ? items : 1) : max_waves);
    d.max_partials = nsegs + (size_t)d.waves;   // each run boundary adds at most one partial
    d.table_bytes = align256(nsegs * 2 * sizeof(int));
    d.m_off = d.table_bytes;
    d.l_off = d.m_off + align256(d.max_partials * group * sizeof(float));
    d.acc_off = d.l_off + align256(d.max_partials * group * sizeof(float));
    size_t end = d.acc_off + d.max_partials * group * (size_t)head_dim * sizeof(float);
    d.sh_groups = sh_groups;
    const size_t sh_rows = nsegs * (size_t)d.sh_groups * group;
    d.sh_m_off = align256(end);
    d.sh_l_off = d.sh_m_off + align256(sh_rows * sizeof(float));
    d.sh_acc_off = d.sh_l_off + align256(sh_rows * sizeof(float));
    d.total = d.sh_groups ? d.sh_acc_off + sh_rows * (size_t)head_dim * sizeof(float) : end;
    return d;
}

// The decode kernels count work items (at most kDecodeSplitCap per slot and
// kv head) in 32 bits.
bool decode_items_fit(int n_slots, int n_kv_head) {
    return (long long)n_slots * n_kv_head <= fa::kMaxScheduleUnits / fa::kDecodeSplitCap;
}

DecodeLayout decode_layout(const fa_cache *c, int n_slots, int n_head, int max_ctx) {
    return decode_layout_of(c->format, c->n_kv_head, c->head_dim, shadow_groups(c), n_slots, n_head,
                            max_ctx);
}
}  // namespace

size_t fa_decode_workspace_bytes(const fa_cache *cache, int n_slots, int n_head, int max_ctx) {
    if (!cache || !dim_ok(cache->head_dim) || cache->n_kv_head < 1 || n_slots < 0 ||
        n_head < 1 || n_head % cache->n_kv_head || max_ctx < 1)
        return 0;
    return decode_layout(cache, n_slots, n_head, max_ctx).total;
}

}  // extern "C"

namespace {
// fa_decode with the caller's workspace, or (use_scratch) with this GPU's
// library-owned scratch.
// The decode's tile contractions: fp32 MFMA (fa_decode), or fp16 MFMA with
// hi/lo-split operands over a Q4_0 cache (fa_decode_q4_hilo).
enum class DecodeLane { kFp32, kHilo };

int decode_entry(const fa_cache *cache, const float *q, const int *d_pos, int n_slots,
                 int max_ctx_hint, int n_head, int attn_sink, int attn_win, float scale,
                 float *out, void *ws, size_t ws_bytes, bool use_scratch,
                 unsigned long long *tile_stats, void *stream,
                 DecodeLane lane = DecodeLane::kFp32) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if (lane == DecodeLane::kHilo &&
        (cache->format != FA_KV_Q4_0 || cache->shadow_sink > 0 || cache->shadow_win > 0))
        return FA_EUNSUPPORTED;
    if ((rc = check_heads(cache, n_head))) return rc;
    if ((rc = check_scale(scale))) return rc;
    if (n_slots < 0 || n_slots > cache->n_slots) return FA_EINVAL;
    if (max_ctx_hint < 1 || max_ctx_hint > cache->max_seq) return FA_EINVAL;
    if (n_slots == 0) return FA_OK;
    if (!q || !d_pos || !out || (!use_scratch && !ws)) return FA_ENULL;
    if (!use_scratch && (uintptr_t)ws % 16 != 0) return FA_EINVAL;
    if (!decode_items_fit(n_slots, cache->n_kv_head)) return FA_EUNSUPPORTED;
    const DecodeLayout lay = decode_layout(cache, n_slots, n_head, max_ctx_hint);
    if (use_scratch ? lay.total > (size_t)FA_DECODE_SCRATCH_BYTES : ws_bytes < lay.total)
        return FA_EWORKSPACE;
    if ((rc = fa_init())) return rc;
    if (use_scratch) {
        int dev = 0;
        if (hip_rc(hipGetDevice(&dev))) return FA_EHIP;
        ws = g_scratch[dev];
    }
    uint8_t *wsb = (uint8_t *)ws;
    fa::DecodeArgs a{};
    a.q = q;
    a.pos = d_pos;
    a.k = cache->k;
    a.v = cache->v;
    a.seg_table = (int *)wsb;
    a.ws_m = (float *)(wsb + lay.m_off);
    a.ws_l = (float *)(wsb + lay.l_off);
    a.ws_acc = (float *)(wsb + lay.acc_off);
    a.out = out;
    a.stats = tile_stats;
    a.n_slots = n_slots;
    a.n_head = n_head;
    a.n_kv = cache->n_kv_head;
    a.max_seq = cache->max_seq;
    a.sink = attn_sink < 0 ? 0 : attn_sink;
    a.win = attn_win;
    a.qscale = scale * fa::kLog2e;
    a.kps = fa::kDecodeKps;
    a.cap = fa::kDecodeSplitCap;
    a.sh = shadow_args(cache, 0);
    a.sh_groups = lay.sh_groups;
    a.sh_m = (float *)(wsb + lay.sh_m_off);
    a.sh_l = (float *)(wsb + lay.sh_l_off);
    a.sh_acc = (float *)(wsb + lay.sh_acc_off);
    const int group = n_head / cache->n_kv_head;
    a.sh_waves = 0;
    if (lay.sh_groups) {
        fa::ShadowPassArgs &sp = a.shp;
        sp.q = q;
        sp.d_pos = d_pos;
        sp.pos0 = 0;
        sp.n_q = n_slots;
        sp.n_head = n_head;
        sp.n_kv = cache->n_kv_head;
        sp.max_seq = cache->max_seq;
        sp.sink = a.sink;
        sp.win = a.win;
        sp.qscale = a.qscale;
        sp.sh = a.sh;
        sp.chunk_groups = lay.sh_groups;
        sp.chunks_per_group = 1;
        sp.m_out = (float *)a.sh_m;
        sp.l_out = (float *)a.sh_l;
        sp.acc_out = (float *)a.sh_acc;
        a.sh_waves = n_slots * cache->n_kv_head * lay.sh_groups;   // run inside the partial launch
    }
    if (lane == DecodeLane::kHilo)
        return hip_rc(fa::launch_decode_hilo(cache->head_dim, group, a,
                                             lay.waves < fa::kDecodeMaxWavesHilo
                                                 ? lay.waves : fa::kDecodeMaxWavesHilo,
                                             (hipStream_t)stream));
    return hip_rc(fa::launch_decode(cache->format, cache->head_dim, group, a, lay.waves,
                                    (hipStream_t)stream));
}
}  // namespace

extern "C" {

int fa_decode(const fa_cache *cache, const float *q, const int *d_pos, int n_slots,
              int max_ctx_hint, int n_head, int attn_sink, int attn_win, float scale,
              float *out, void *ws, size_t ws_bytes, unsigned long long *tile_stats,
              void *stream) {
    return decode_entry(cache, q, d_pos, n_slots, max_ctx_hint, n_head, attn_sink, attn_win,
                        scale, out, ws, ws_bytes, false, tile_stats, stream);
}

int fa_decode_q4_hilo(const fa_cache *cache, const float *q, const int *d_pos, int n_slots,
                      int max_ctx_hint, int n_head, int attn_sink, int attn_win, float scale,
                      float *out, void *ws, size_t ws_bytes, unsigned long long *tile_stats,
                      void *stream) {
    return decode_entry(cache, q, d_pos, n_slots, max_ctx_hint, n_head, attn_sink, attn_win,
                        scale, out, ws, ws_bytes, false, tile_stats, stream, DecodeLane::kHilo);
}

int fa_decode_noalloc(const fa_cache *cache, const float *q, const int *d_pos, int n_slots,
                      int max_ctx_hint, int n_head, int attn_sink, int attn_win, float scale,
                      float *out, unsigned long long *tile_stats, void *stream) {
    return decode_entry(cache, q, d_pos, n_slots, max_ctx_hint, n_head, attn_sink, attn_win,
                        scale, out, nullptr, 0, true, tile_stats, stream);
}

// ---------------------------------------------------------------- paged
namespace {
int check_paged_cache(const fa_paged_cache *c) {
    if (!c) return FA_ENULL;
    if (!dim_ok(c->head_dim)) return FA_EUNSUPPORTED;
    if (c->num_blocks < 1 || c->block_size < 1 || c->n_kv_head < 1) return FA_EINVAL;
    if (!c->k || !c->v) return FA_ENULL;
    const long long page = (long long)c->block_size * c->n_kv_head * c->head_dim;
    if (c->block_stride != 0 && (c->block_stride < page || c->block_stride % 4 != 0))
        return FA_EINVAL;
    if (((uintptr_t)c->k | (uintptr_t)c->v) % 16 != 0) return FA_EINVAL;
    return FA_OK;
}

long long paged_block_stride(const fa_paged_cache *c) {
    return c->block_stride ? c->block_stride
                           : (long long)c->block_size * c->n_kv_head * c->head_dim;
}

struct PagedLayout {
    size_t table_bytes, m_off, l_off, acc_off, total;
};

PagedLayout paged_layout(int head_dim) {
    PagedLayout p;
    const size_t rows = (size_t)fa::kPrefillWaves * fa::kPrefillRowsPerWave;
    const size_t pieces = 2 * (size_t)fa::kPrefillMaxWorkGroups;
    p.table_bytes = align256(sizeof(fa::CutList));
    p.m_off = p.table_bytes;
    p.l_off = p.m_off + align256(pieces * rows * sizeof(float));
    p.acc_off = p.l_off + align256(pieces * rows * sizeof(float));
    p.total = p.acc_off + pieces * rows * (size_t)head_dim * sizeof(float);
    return p;
}
}  // namespace

int fa_paged_append(const fa_paged_cache *cache, const float *k, const float *v,
                    const int64_t *slot_mapping, int num_slots, void *stream) {
    int rc = check_paged_cache(cache);
    if (rc) return rc;
    if (num_slots < 0) return FA_EINVAL;
    if (num_slots == 0) return FA_OK;
    if (!k || !v || !slot_mapping) return FA_ENULL;
    if (((uintptr_t)k | (uintptr_t)v) % 16 != 0) return FA_EINVAL;
    if ((rc = fa_init())) return rc;
    fa::PagedAppendArgs a;
    a.k_new = k;
    a.v_new = v;
    a.k = cache->k;
    a.v = cache->v;
    a.slot_mapping = (const long long *)slot_mapping;
    a.n = num_slots;
    a.n_kv = cache->n_kv_head;
    a.head_dim = cache->head_dim;
    a.block_size = cache->block_size;
    a.num_blocks = cache->num_blocks;
    a.blk_stride = paged_block_stride(cache);
    return hip_rc(fa::launch_paged_append(a, (hipStream_t)stream));
}

size_t fa_paged_workspace_bytes(int head_dim) {
    if (!dim_ok(head_dim)) return 0;
    return paged_layout(head_dim).total;
}

int fa_paged_attention(const fa_paged_cache *cache, const float *q, int num_tokens, int n_head,
                       const int *query_start_loc, const int *seq_lens, int num_reqs,
                       const int *block_table, int max_blocks_per_seq, int window_left,
                       int window_right, float scale, float *out, float *lse, void *ws,
                       size_t ws_bytes, void *stream) {
    int rc = check_paged_cache(cache);
    if (rc) return rc;
    if (n_head < 1 || n_head % cache->n_kv_head != 0) return FA_EINVAL;
    if (!group_ok(n_head / cache->n_kv_head)) return FA_EUNSUPPORTED;
    if ((rc = check_scale(scale))) return rc;
    if (num_tokens < 0 || num_reqs < 0 || num_reqs > fa::kPagedMaxReqs) return FA_EINVAL;
    if (max_blocks_per_seq < 1 ||
        (long long)max_blocks_per_seq * cache->block_size > 0x7fffffffLL)
        return FA_EINVAL;
    if (window_left >= 0 && window_right < 0) return FA_EINVAL;
    if (num_tokens == 0 || num_reqs == 0) return FA_OK;
    if (!q || !out || !query_start_loc || !seq_lens || !block_table || !ws) return FA_ENULL;
    if (((uintptr_t)q | (uintptr_t)out) % 16 != 0) return FA_EINVAL;
    {
        // The batch is described on the device, so bound the schedule the
        // kernel will count in 32 bits: at most num_tokens / BQ + num_reqs
        // query blocks per kv head, each walking at most cap / 32 + 1 tiles.
        const int bq = fa::prefill_q_positions(n_head / cache->n_kv_head);
        const long long segs =
            (long long)cache->n_kv_head * ((num_tokens + (long long)bq - 1) / bq + num_reqs);
        const long long seg_units =
            ((long long)max_blocks_per_seq * cache->block_size / fa::kPrefillKeyTile + 1) *
                fa::kTileUnits + fa::kSegUnits;
        if (segs > fa::kMaxScheduleUnits / seg_units) return FA_EUNSUPPORTED;
    }
    const PagedLayout lay = paged_layout(cache->head_dim);
    if (ws_bytes < lay.total) return FA_EWORKSPACE;
    if ((rc = fa_init())) return rc;
    int dev = 0;
    if (hip_rc(hipGetDevice(&dev))) return FA_EHIP;
    uint8_t *wsb = (uint8_t *)ws;
    fa::PrefillArgs a{};
    a.q = q;
    a.out = out;
    a.lse = lse;
    a.k = cache->k;
    a.v = cache->v;
    a.stats = nullptr;
    a.cuts = (fa::CutList *)wsb;
    a.ws_m = (float *)(wsb + lay.m_off);
    a.ws_l = (float *)(wsb + lay.l_off);
    a.ws_acc = (float *)(wsb + lay.acc_off);
    a.n = num_tokens;
    a.pos0 = 0;
    a.n_head = n_head;
    a.n_kv = cache->n_kv_head;
    a.max_seq = 0;
    // causal window (left, right): keys [p - left, p]; right adds nothing
    // under the causal bound. A window wider than any context is none.
    const long long cap = (long long)max_blocks_per_seq * cache->block_size;
    a.sink = 0;
    a.win = window_left < 0 || window_left >= cap ? 0 : window_left + 1;
    a.qscale = scale * fa::kLog2e;
    a.n_qblocks = 1;
    a.n_wg = g_device_cus[dev] < fa::kPrefillMaxWorkGroups ? g_device_cus[dev]
                                                           : fa::kPrefillMaxWorkGroups;
    a.qsl = query_start_loc;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.n_req = num_reqs;
    a.bt_stride = max_blocks_per_seq;
    a.block_size = cache->block_size;
    a.num_blocks = cache->num_blocks;
    a.blk_stride = paged_block_stride(cache);
    return hip_rc(fa::launch_paged_prefill(cache->head_dim, n_head / cache->n_kv_head, a,
                                           (hipStream_t)stream));
}

size_t fa_paged_decode_workspace_bytes(int num_reqs, int n_head, int n_kv_head, int head_dim,
                                       int max_seq_len_hint) {
    if (num_reqs < 0 || n_kv_head < 1 || n_head < 1 || n_head % n_kv_head ||
        !group_ok(n_head / n_kv_head) || !dim_ok(head_dim) || max_seq_len_hint < 1)
        return 0;
    return decode_layout_of(FA_KV_F32, n_kv_head, head_dim, 0, num_reqs, n_head, max_seq_len_hint)
        .total;
}

int fa_paged_decode(const fa_paged_cache *cache, const float *q, int num_reqs, int n_head,
                    const int *seq_lens, const int *block_table, int max_blocks_per_seq,
                    int max_seq_len_hint, int window_left, int window_right, float scale,
                    float *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_paged_cache(cache);
    if (rc) return rc;
    if (cache->block_size % 16 != 0) return FA_EUNSUPPORTED;
    if (n_head < 1 || n_head % cache->n_kv_head != 0) return FA_EINVAL;
    if (!group_ok(n_head / cache->n_kv_head)) return FA_EUNSUPPORTED;
    if ((rc = check_scale(scale))) return rc;
    if (num_reqs < 0 || max_blocks_per_seq < 1 ||
        (long long)max_blocks_per_seq * cache->block_size > 0x7fffffffLL)
        return FA_EINVAL;
    const long long cap = (long long)max_blocks_per_seq * cache->block_size;
    if (max_seq_len_hint < 1 || max_seq_len_hint > cap) return FA_EINVAL;
    if (window_left >= 0 && window_right < 0) return FA_EINVAL;
    if (num_reqs == 0) return FA_OK;
    if (!q || !out || !seq_lens || !block_table || !ws) return FA_ENULL;
    if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)ws) % 16 != 0) return FA_EINVAL;
    if (!decode_items_fit(num_reqs, cache->n_kv_head)) return FA_EUNSUPPORTED;
    const int group = n_head / cache->n_kv_head;
    const DecodeLayout lay =
        decode_layout_of(FA_KV_F32, cache->n_kv_head, cache->head_dim, 0, num_reqs, n_head,
                         max_seq_len_hint);
    if (ws_bytes < lay.total) return FA_EWORKSPACE;
    if ((rc = fa_init())) return rc;
    uint8_t *wsb = (uint8_t *)ws;
    fa::DecodeArgs a{};
    a.q = q;
    a.pos = nullptr;
    a.k = cache->k;
    a.v = cache->v;
    a.seg_table = (int *)wsb;
    a.ws_m = (float *)(wsb + lay.m_off);
    a.ws_l = (float *)(wsb + lay.l_off);
    a.ws_acc = (float *)(wsb + lay.acc_off);
    a.out = out;
    a.stats = nullptr;
    a.n_slots = num_reqs;
    a.n_head = n_head;
    a.n_kv = cache->n_kv_head;
    a.max_seq = (int)cap;              // positions past a request's table row are invalid
    a.sink = 0;
    a.win = window_left < 0 || window_left >= cap ? 0 : window_left + 1;
    a.qscale = scale * fa::kLog2e;
    a.kps = fa::kDecodeKps;
    a.cap = fa::kDecodeSplitCap;
    a.sh_groups = 0;
    a.sh_waves = 0;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.bt_stride = max_blocks_per_seq;
    a.block_size = cache->block_size;
    a.num_blocks = cache->num_blocks;
    a.blk_stride = paged_block_stride(cache);
    a.lse = lse;
    return hip_rc(fa::launch_paged_decode(cache->head_dim, group, a, lay.waves, (hipStream_t)stream));
}

int fa_merge_attn_states(float *out, float *out_lse, const float *prefix_out,
                         const float *prefix_lse, const float *suffix_out,
                         const float *suffix_lse, int num_tokens, int n_head, int head_dim,
                         int prefill_tokens_with_context, void *stream) {
    if (num_tokens < 0 || n_head < 1 || head_dim < 4 || head_dim % 4 != 0 || head_dim > 4096)
        return FA_EINVAL;
    if (num_tokens == 0) return FA_OK;
    if (!out || !prefix_out || !prefix_lse || !suffix_out || !suffix_lse) return FA_ENULL;
    if (((uintptr_t)out | (uintptr_t)prefix_out | (uintptr_t)suffix_out) % 16 != 0)
        return FA_EINVAL;
    int rc;
    if ((rc = fa_init())) return rc;
    fa::MergeArgs a;
    a.out = out;
    a.out_lse = out_lse;
    a.p_out = prefix_out;
    a.p_lse = prefix_lse;
    a.s_out = suffix_out;
    a.s_lse = suffix_lse;
    a.T = num_tokens;
    a.H = n_head;
    a.D = head_dim;
    a.prefill_tokens_with_context = prefill_tokens_with_context;
    return hip_rc(fa::launch_merge(a, (hipStream_t)stream));
}

const char *fa_last_hip_error(void) { return hipGetErrorName(g_last_hip_error); }

const char *fa_strerror(int code) {
    switch (code) {
    case FA_OK: return "ok";
    case FA_EINVAL: return "invalid argument value";
    case FA_ENULL: return "required pointer is NULL";
    case FA_EUNSUPPORTED: return "unsupported head_dim, group size or KV format";
    case FA_EWORKSPACE: return "workspace too small (caller's, or the fixed decode scratch)";
    case FA_EHIP: return "HIP runtime error";
    case FA_ERANGE: return "positions beyond the cache (pos0 + n > max_seq)";
    case FA_EDEVICE: return "current device is not gfx950";
    }
    return "unknown error code";
}

}  // extern "C"
