// Causal GQA flash-attention prefill on fp32 MFMA (gfx950).
//
// Method ([FA] file header and fc_attn_flash_prefill): key tiles are folded
// into a running max m, running sum l and an unnormalised accumulator, so the
// score matrix never exists; the K/V tile is loaded once and serves every q
// head of the GQA group; tiles outside the sink U recent-window key set are
// skipped before any load or barrier ([FA] fc_attn_tile_in_window).
//
// MI355X layout of the work:
//   * A work-group of 8 waves (two per SIMD, one work-group per CU) owns
//     BQ = 128/G consecutive query positions of one kv head; each wave owns
//     16 (position, head) rows, row R -> position q0 + R/G, head
//     kvh*G + R%G. One 32-key K tile and V tile (fp32, padded rows) sit in
//     LDS and are shared by all 128 rows of the group. The second wave of a
//     SIMD issues its MFMAs while the first waits (LDS reads, the QK chain's
//     drain, the barrier).
//   * S^T = K Q^T with v_mfma_f32_16x16x4_f32, over the tile's two 16-key
//     sets: K rows come from LDS, Q^T is held in registers (pre-scaled by
//     scale*log2 e). The contraction order of each group of 4 MFMAs is
//     chosen so that a lane's K operands are one 16-byte read. The
//     accumulator gives lane l 8 keys of query row l&15, so a row's scores
//     sit in its 4 lane groups and the softmax needs two cross-lane steps
//     (lane ^ 16, ^ 32).
//   * O^T = V^T P^T, also 16x16x4: P^T is exactly the S^T accumulator after
//     the exponentials (the key order of each contraction step is chosen to
//     match the accumulator layout). Output block b of O^T holds dims
//     64 (b/4) + 4 m + b%4, so that a lane's V operands of one key are 16
//     contiguous floats (four 16-byte reads, contiguous across the 16 lanes
//     of a group). O^T keeps one query row per lane, so the rescale by
//     exp(m_old - m_new) is a per-lane multiply, done only when some row's
//     max moved.
//   * Q4_0 tiles are loaded as raw 18-byte blocks and decoded exactly
//     ((c-8)*d) while being written to the fp32 LDS tile.
//   * Stream-K schedule: the visited key tiles of every (kv head, query
//     block) segment form one list, and a grid of one work-group per CU takes
//     equal contiguous runs of it, so a long causal row is spread over several
//     CUs instead of setting the critical path. A segment cut by a run
//     boundary writes per-piece partials {m, l, acc} that a small combine
//     kernel merges ([FA] decode combine formula); a whole segment writes its
//     output directly.
//   * K/V tiles are double-buffered in LDS with one barrier per tile: fp32
//     rows go straight from global memory into the next buffer
//     (buffer_load_dwordx4 ... lds, one row per wave instruction, so no staging
//     registers), requested row by row between the current tile's QK MFMAs;
//     Q4_0 blocks are staged in registers and decoded into the next buffer
//     after the current tile's matrix work.
//   * Output rows leave through LDS (the tile buffers, free after the last
//     tile), so that every store instruction writes whole contiguous rows.
//   * Lazy rescale: a row's reference max only moves when a tile's max
//     exceeds it by more than kTau (log2 units). Probabilities are then
//     bounded by 2^kTau, and the O rescale (a pass over all accumulators)
//     runs a few times per row instead of on most tiles; the final acc / l
//     is unchanged up to rounding because acc and l share the reference.
//   * Tiles inside every row's key set skip the mask.
//   * Paged varlen batch ([VT] PagedAttention, fp32 rows): the same kernel
//     with the segments of every request in one stream-K list. Requests are
//     described on the device (query_start_loc, seq_lens, block table), so
//     the launch needs no device-to-host read: each work-group rebuilds the
//     request table in LDS, a segment is a (request, kv head, query block),
//     and each K/V row is DMA'd through its own descriptor at its page.
//   * Optional LSE output (ln of the softmax denominator) per row, from the
//     final {m, l}: the state [VT] MergeAttnStates merges.
//   * fp16-shadow keys of a Q4_0 cache ([FA] "fp16 sink + recent-window
//     exemption"): the same kernel in a third mode folds, per query block,
//     the union of its rows' shadow keys (sink rows, then the window ring
//     rows the block can reach: about 9 tiles of 32) on the MFMA path, fp16
//     rows converted into the fp32 LDS tiles, each key masked per row by the
//     shadow predicate. It leaves every row's unnormalised partial
//     {m, l, acc}, from which the main Q4_0 pass starts.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <int HD, int G, int FMT>
struct PrefillShape {
    static constexpr int W = kPrefillWaves;
    static constexpr int R = kPrefillRowsPerWave;
    static_assert(R == 16, "16-row waves (16x16x4 MFMA tiles)");
    static constexpr int NTHR = 64 * W;         // threads per work-group
    static constexpr int BK = kPrefillKeyTile;
    static constexpr int BQ = W * R / G;        // query positions per work-group
    static constexpr int PW = R / G;            // query positions per wave
    static constexpr int KS = HD + 4;           // LDS row stride (floats): conflict-free 16-B reads
    static constexpr int NBLK = HD / 16;        // 16-dim output blocks of O^T
    static constexpr int NBB = HD / 64;         // 16-byte V reads per lane per PV step
    static constexpr int QPL = HD / 4;          // q operand floats per lane
    static constexpr int NB = HD / kQ4Block;    // Q4 blocks per row
    static constexpr int RB = FMT == 0 ? HD * 4 : NB * kQ4BlockBytes;
    static constexpr int QITEMS = 2 * BK * NB;                         // Q4 (row, block) items, K and V
    static constexpr int IPT = (QITEMS + NTHR - 1) / NTHR;             // Q4 items per thread
    static constexpr int BUF = 2 * BK * KS;     // floats per buffer: K tile then V tile
    static constexpr size_t LDS_BYTES = (size_t)2 * BUF * sizeof(float);
};

// Reference-max slack of the lazy rescale (log2 units): p <= 2^kTau.
constexpr float kTau = 8.0f;

__device__ __forceinline__ void scale_acc(f32x4 &acc, float c) { acc *= c; }

// Wait for all of this wave's vector-memory operations (incl. LDS DMA).
__device__ __forceinline__ void wait_vmem() { wait_vmem_le<0>(); }

constexpr int kXcds = 8;   // XCDs of an MI355X; block b runs on XCD b % 8
// Segment s of the schedule is query block seg_qblock(s) of kv head
// s / n_qblocks. Within a head the causal segments alternate long and short
// (last block, first block, second to last, second, ...), so that a
// contiguous run of tiles spans few segments and no work-group collects a
// long string of short segments with their fixed per-segment costs.
__device__ __forceinline__ int seg_qblock(int s, int n_qblocks) {
    const int i = s % n_qblocks;
    return (i & 1) ? (i >> 1) : n_qblocks - 1 - (i >> 1);
}

// Block-wide exclusive scan of one int per thread (a prefill work-group of
// kPrefillWaves waves); also returns the total. `scratch` holds one int per wave.
__device__ __forceinline__ int block_excl_scan(int x, int tid, int *scratch, int *total) {
    const int lane = tid & 63, w = tid >> 6;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == 63) scratch[w] = incl;
    __syncthreads();
    int before = 0, sum = 0;
#pragma unroll
    for (int i = 0; i < kPrefillWaves; i++) {
        const int v = scratch[i];
        before += i < w ? v : 0;
        sum += v;
    }
    *total = sum;
    return before + incl - x;
}

// Kernel modes: plain (one sequence of a slot cache), paged (varlen batch
// over a paged fp32 cache), shadow (the fp16-shadow keys of a Q4_0 slot
// cache, fp32 tiles; writes partials).
constexpr int kModePlain = 0, kModePaged = 1, kModeShadow = 2;

template <int HD, int G, int FMT, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kPrefillWaves, 64 * kPrefillWaves),
                          amdgpu_waves_per_eu(kPrefillWaves / 4, kPrefillWaves / 4)))
void prefill_kernel(PrefillArgs a) {
    constexpr bool PG = MODE == kModePaged;
    constexpr bool SH = MODE == kModeShadow;
    static_assert(!(PG || SH) || FMT == 0, "paged and shadow modes stage fp32 tiles");
    using Sh = PrefillShape<HD, G, FMT>;
    constexpr int BK = Sh::BK, KS = Sh::KS;
    constexpr int NB = Sh::NB, RB = Sh::RB;
    constexpr int ROWS = Sh::W * Sh::R;
    constexpr int R = Sh::R, NTHR = Sh::NTHR;
    extern __shared__ __attribute__((aligned(16))) float lds[];   // 16-byte LDS accesses need 16-byte alignment
    __shared__ int scan_scratch[kPrefillWaves];
    __shared__ int run_info[8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index: uniform
    // lane = (query row n16 of the wave, lane group g4): the B column and
    // B row of a 16x16x4 MFMA
    const int n16 = lane & 15, g4 = lane >> 4;
    const bool row_lead = g4 == 0;    // one lane per row

    // ---- paged batch: the requests' geometry, in LDS behind the K/V
    // buffers. Segments are numbered request by request, then kv head, then
    // query block. Device metadata is clamped so that no access leaves the
    // query, output, block-table or cache buffers: query tokens to [0, n),
    // a request's context to its block-table row.
    int *rq_seg0 = (int *)(lds + 2 * Sh::BUF);   // [n_req + 1] first segment of each request
    int *rq_ctx = rq_seg0 + a.n_req + 1;          // position of its first query token
    int *rq_tok = rq_ctx + a.n_req;               // its first query token
    int *rq_len = rq_tok + a.n_req;               // its query tokens
    int nsegs = a.n_kv * a.n_qblocks;
    if constexpr (PG) {
        const int cap = a.bt_stride * a.block_size;
        int carry = 0;
        for (int base = 0; base < a.n_req; base += NTHR) {
            const int r = base + tid;
            int cnt = 0;
            if (r < a.n_req) {
                const int t0 = min(max(a.qsl[r], 0), a.n);
                const int len = min(min(max(a.qsl[r + 1], t0), a.n) - t0, cap);
                const int seq = min(max(a.seq_lens[r], len), cap);
                rq_ctx[r] = seq - len;
                rq_tok[r] = t0;
                rq_len[r] = len;
                cnt = a.n_kv * ((len + Sh::BQ - 1) / Sh::BQ);
            }
            int chunk;
            const int before = block_excl_scan(cnt, tid, scan_scratch, &chunk);
            if (r < a.n_req) rq_seg0[r] = carry + before;
            carry += chunk;
        }
        if (tid == 0) rq_seg0[a.n_req] = carry;
        __syncthreads();
        nsegs = carry;
    }

    // Segment s: query block [q0, q1] (positions) of kv head kvh; position
    // p is query token p + tok.
    struct Seg {
        int q0, q1, kvh, tok, req;
    };
    auto seg_of = [&](int s) -> Seg {
        Seg g;
        if constexpr (PG) {
            int lo = 0, hi = a.n_req - 1;      // the last request starting at or before s
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (rq_seg0[mid] <= s) lo = mid;
                else hi = mid - 1;
            }
            const int len = rq_len[lo], nqb = (len + Sh::BQ - 1) / Sh::BQ;
            const int loc = s - rq_seg0[lo];
            g.kvh = loc / nqb;
            g.q0 = rq_ctx[lo] + seg_qblock(loc % nqb, nqb) * Sh::BQ;
            g.q1 = min(g.q0 + Sh::BQ - 1, rq_ctx[lo] + len - 1);
            g.tok = rq_tok[lo] - rq_ctx[lo];
            g.req = lo;
        } else {
            g.kvh = s / a.n_qblocks;
            g.q0 = a.pos0 + seg_qblock(s, a.n_qblocks) * Sh::BQ;
            g.q1 = min(g.q0 + Sh::BQ - 1, a.pos0 + a.n - 1);
            g.tok = -a.pos0;
            g.req = 0;
        }
        return g;
    };

    // ---- schedule: total units, this work-group's run, the piece table.
    // A segment with c visited tiles is kSegUnits + c * kTileUnits units:
    // the leading units stand for the fixed cost a run pays to start a
    // segment (Q load, first-tile latency, output write), so runs that start
    // more segments get fewer tiles. Tile t of a segment whose tile units
    // start at T0 belongs to owner(T0 + t * kTileUnits). Every run spans at
    // least kTileUnits units (the host keeps work-groups <= tiles), so every
    // run between a segment's first and last owner owns one of its tiles.
    // Shadow mode: the keys of query block [q0, q1] that may come from the
    // fp16 shadow for some row, in list order: sink positions [0, n_sk),
    // then window positions [wlo, q1] (every position some row's ring window
    // reaches). List entry i is position i (i < n_sk) or wlo + i - n_sk.
    struct ShList {
        int n_sk, wlo, nk;
        __device__ int pos(int i) const { return i < n_sk ? i : wlo + i - n_sk; }
    };
    auto sh_list = [&](int q0, int q1) -> ShList {
        ShList l;
        l.n_sk = min(a.sh.sink, q1 + 1);
        l.wlo = max(a.sh.sink, q0 - a.sh.win + 1);
        l.nk = l.n_sk + (a.sh.win > 0 ? max(0, q1 - l.wlo + 1) : 0);
        return l;
    };
    auto seg_units = [&](int s, int *cnt) {
        if (s >= nsegs) {
            *cnt = 0;
            return 0;
        }
        const Seg g = seg_of(s);
        if constexpr (SH) *cnt = (sh_list(g.q0, g.q1).nk + BK - 1) / BK;
        else *cnt = seg_tiles(g.q0, g.q1, a.sink, a.win, BK).count;
        return *cnt > 0 ? *cnt * kTileUnits + kSegUnits : 0;
    };
    int total = 0;
    for (int base = 0; base < nsegs; base += NTHR) {
        const int s = base + tid;
        int cnt = 0;
        const int u = seg_units(s, &cnt);
        int chunk;
        block_excl_scan(u, tid, scan_scratch, &chunk);
        total += chunk;
    }
    // The host sizes the grid from the tile count; a paged launch cannot see
    // it, so its grid is the maximum and it keeps total / kTileUnits runs at
    // most (every run must span a whole tile), the other work-groups idle.
    int NWG = gridDim.x;
    if constexpr (PG) NWG = min(NWG, max(1, total / kTileUnits));
    // Work-groups are dealt to the 8 XCDs round-robin (block b on XCD b % 8);
    // give each XCD a contiguous stretch of runs so that its L2 holds the K/V
    // rows of few kv heads.
    const int b = blockIdx.x;
    const int wg = b >= NWG ? -1
                 : NWG % kXcds == 0 ? (b % kXcds) * (NWG / kXcds) + b / kXcds : b;
    const long long lo = wg < 0 ? 0 : (long long)wg * total / NWG;
    const long long hi = wg < 0 ? 0 : (long long)(wg + 1) * total / NWG;
    auto owner = [&](long long f) -> int { return (int)(((f + 1) * NWG - 1) / total); };
    if (tid == 0) {
        run_info[0] = -1;          // first segment of the run
        run_info[1] = -1;          // last segment of the run
    }
    {
        int f_carry = 0, p_carry = 0, c_carry = 0;
        for (int base = 0; base < nsegs; base += NTHR) {
            const int s = base + tid;
            int cnt = 0;
            const int u = seg_units(s, &cnt);
            int chunk, chunk_pc;
            const int F = f_carry + block_excl_scan(u, tid, scan_scratch, &chunk);
            const int T0 = F + kSegUnits;      // first tile unit
            const int np = cnt > 0 ? owner(T0 + (cnt - 1) * kTileUnits) - owner(T0) + 1 : 0;
            // pieces (< 2^16 in a launch) and cut segments, scanned together
            const int pc = np > 1 ? np | (1 << 16) : 0;
            const int PC = block_excl_scan(pc, tid, scan_scratch, &chunk_pc);
            const int P = p_carry + (PC & 0xffff);
            if (wg == 0 && np > 1) {
                const Seg g = seg_of(s);
                CutSeg &c = a.cuts->seg[c_carry + (PC >> 16)];
                c.piece0 = P;
                c.n_pieces = np;
                c.q0 = g.q0;
                c.q1 = g.q1;
                c.kvh = g.kvh;
                c.tok = g.tok;
            }
            if (u > 0 && F <= lo && lo < F + u) {
                run_info[0] = s;
                run_info[2] = F;
                run_info[3] = P;
            }
            if (u > 0 && F < hi && hi <= F + u) {
                run_info[1] = s;
                run_info[4] = F;
                run_info[5] = P;
            }
            f_carry += chunk;
            p_carry += chunk_pc & 0xffff;
            c_carry += chunk_pc >> 16;
        }
        if (wg == 0 && tid == 0) a.cuts->count = c_carry;
    }
    __syncthreads();
    const int s_first = run_info[0], s_last = run_info[1];

    unsigned visited = 0, skipped = 0;

    // ---- fold tiles [t_lo, t_hi) of one segment; whole segments write out,
    // cut ones write piece `piece` of the partial buffer
    auto run_segment = [&](int seg, int t_lo, int t_hi, bool whole, int piece, bool first_owner) {
    const Seg sg = seg_of(seg);
    const int kvh = sg.kvh, q0 = sg.q0, q1 = sg.q1;
    const SegTiles st = seg_tiles(q0, q1, a.sink, a.win, BK);
    if (!SH && first_owner) skipped += (unsigned)(st.walked - st.count);
    const ShList shl = sh_list(q0, q1);
    // first key (plain, paged) or list entry (shadow) of visited tile t
    auto tile_at = [&](int t) { return SH ? t * BK : st.tile(t) * BK; };

    const int row_wg = w * Sh::R + n16;
    const int p_row = q0 + row_wg / G;
    const int g = row_wg % G;
    const bool row_live = p_row <= q1;
    const int pw0 = q0 + w * Sh::PW;
    const int pw1 = min(pw0 + Sh::PW - 1, q1);

    const uint8_t *kbase = (const uint8_t *)a.k + (size_t)kvh * a.max_seq * RB;
    const uint8_t *vbase = (const uint8_t *)a.v + (size_t)kvh * a.max_seq * RB;

    // Q^T operand: this lane's row, pre-scaled, dims 16 j + 4 g4 + t as
    // qr[4 j + t]. Loaded after the first tile's request, so that the two
    // latencies overlap.
    float qr[Sh::QPL];
    auto load_q = [&]() {
        if (row_live) {
            const float *qrow = a.q + ((size_t)(p_row + sg.tok) * a.n_head + kvh * G + g) * HD;
#pragma unroll
            for (int i = 0; i < Sh::QPL / 4; i++) {
                const f32x4 v = *(const f32x4 *)(qrow + 16 * i + 4 * g4);
#pragma unroll
                for (int t = 0; t < 4; t++) qr[4 * i + t] = v[t] * a.qscale;
            }
        } else {
#pragma unroll
            for (int i = 0; i < Sh::QPL; i++) qr[i] = 0.0f;
        }
    };

    // O^T accumulators: NBLK 16x16 blocks; block b holds dims
    // 64 (b >> 2) + 4 m + (b & 3) (m its row index), so that a lane's PV
    // operands of a key are contiguous in the V row
    constexpr int NO = Sh::NBLK;
    f32x4 O[NO];
#pragma unroll
    for (int n = 0; n < NO; n++) O[n] = f32x4{};
    float m_run = -INFINITY, l_run = 0.0f;
    // fp16 shadow: one piece per segment (the first) starts from the row's
    // shadow-key partial, its acc read through the d permutation of the
    // output stores below
    // (only a Q4_0 cache has a shadow)
    const bool shadowed = FMT == 1 && !SH && (a.sh.sink > 0 || a.sh.win > 0);
    if (FMT == 1 && shadowed && first_owner && row_live) {
        const size_t rf = (size_t)(p_row + sg.tok) * a.n_head + kvh * G + g;
        const float *sp = a.out + rf * HD;
#pragma unroll
        for (int r = 0; r < 4; r++) {
#pragma unroll
            for (int bb = 0; bb < Sh::NBB; bb++) {
                const f32x4 v = *(const f32x4 *)(sp + 64 * bb + 16 * g4 + 4 * r);
#pragma unroll
                for (int e = 0; e < 4; e++) O[4 * bb + e][r] = v[e];
            }
        }
        m_run = a.sh_m[rf];
        l_run = row_lead ? a.sh_l[rf] : 0.0f;
    }

    // ---- staging registers of a Q4_0 tile (fp32 tiles need none)
    // A Q4_0 block (18 bytes) is staged as 5 dwords: from the block start
    // when it is 4-byte aligned (even blocks), else from 2 bytes before it.
    // Both stay inside the row, which holds an even number of blocks.
    uint32_t raw[FMT == 0 ? 1 : Sh::IPT][5];
    // shadow mode: fp16 rows staged as 16-byte chunks (8 values), item idx
    // -> chunk idx % CPR of row (idx / CPR) % BK of K (or V past BK rows)
    constexpr int CPR = HD / 8;
    constexpr int SIPT = SH ? 2 * BK * CPR / NTHR : 1;
    static_assert(!SH || (2 * BK * CPR) % NTHR == 0, "shadow staging chunks per thread");
    u32x4 sraw[SIPT];
    // Q4_0 item idx -> (row, block) of the K tile (idx < BK*NB) or V tile:
    // 8 consecutive items take 8 consecutive rows of one block, then the
    // next block. A wave thus reads 8 whole rows (contiguous in memory),
    // and its 16-byte LDS writes land on rows KS floats apart (16 bytes
    // apart modulo 128), one bank group per lane: no bank conflicts.
    auto q4_item = [](int idx, int &row, int &blk) {
        const int rem = idx % (BK * NB);
        const int g = rem / (8 * NB), w8 = rem % (8 * NB);
        blk = w8 >> 3;
        row = 8 * g + (w8 & 7);
    };

    // Starts loading the tile at key j0 into LDS buffer `buf` (fp32: DMA
    // into LDS; Q4_0: raw blocks into registers). Rows past q1 (only in a
    // block's diagonal tile) repeat row q1 (fp32) or are zero (Q4_0): their
    // scores are masked, and V must stay finite so that p = 0 contributes 0.
    // Paged: lane l (mod 32) holds the page and in-page row of tile row l
    // (rows past q1 repeat row q1), loaded a tile ahead of the DMA that uses
    // them so that the block-table read never stalls the wave.
    const int *bt_row = PG ? a.block_table + (size_t)sg.req * a.bt_stride : nullptr;
    int pf_page = 0, pf_row = 0;
    auto prefetch_pages = [&](int j0) {
        if constexpr (PG) {
            const int jr = j0 + min(lane & (BK - 1), q1 - j0);
            const int pi = jr / a.block_size;
            pf_row = jr - pi * a.block_size;
            pf_page = bt_row[pi];
        }
    };

    // fp32 tiles (plain and paged launches): a tile's DMA split by row, so
    // that the rows of the next tile can be requested between the MFMAs of
    // this tile's QK (scalar and memory instructions issue while an MFMA
    // runs), rather than in a burst with no MFMA to hide it. Lanes past
    // HD / 4 idle.
    //  * plain: descriptors over the rows of the tile that exist (j0 .. q1);
    //  * paged: one descriptor per row (pages need not be adjacent), from the
    //    byte offset of tile row r held by lane r (page ids outside the cache
    //    clamped into it). Row r's lane need not be a copying lane (HD = 64:
    //    16 of them for 32 rows), so the offsets are computed, and read out,
    //    with every lane active: a readlane may not sit inside the copying
    //    lanes' branch.
    constexpr bool SPLIT = FMT == 0 && !SH;
    constexpr int RPW = BK / Sh::W;               // rows per wave per tensor
    struct RowDma {
        __amdgpu_buffer_rsrc_t rk, rv;            // plain
        float *kd, *vd;
        int nrows;                                // plain
        int olo, ohi;                             // paged: this lane's tile row offset
    };
    auto row_dma = [&](int j0, int buf) -> RowDma {
        RowDma d{};
        d.kd = lds + buf * Sh::BUF;
        d.vd = d.kd + BK * KS;
        if constexpr (PG) {
            const long long pg = min(max(pf_page, 0), a.num_blocks - 1);
            const long long off =
                (pg * a.blk_stride + ((long long)pf_row * a.n_kv + kvh) * HD) * (long long)sizeof(float);
            d.olo = (int)(uint32_t)off;
            d.ohi = (int)(uint32_t)((unsigned long long)off >> 32);
        } else {
            d.nrows = min(q1 + 1 - j0, BK);
            const size_t tile0 = (size_t)j0 * RB;
            d.rk = raw_rsrc(kbase + tile0, (unsigned)(d.nrows * RB));
            d.rv = raw_rsrc(vbase + tile0, (unsigned)(d.nrows * RB));
        }
        return d;
    };
    auto issue_row = [&](const RowDma &d, int i) {
        const int row = w * RPW + i;
        if constexpr (PG) {
            const unsigned long long o =
                ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane(d.ohi, row) << 32) |
                (uint32_t)__builtin_amdgcn_readlane(d.olo, row);
            if (lane < HD / 4) {
                dma16(raw_rsrc((const uint8_t *)a.k + o, (unsigned)RB), 16 * lane, d.kd + row * KS);
                dma16(raw_rsrc((const uint8_t *)a.v + o, (unsigned)RB), 16 * lane, d.vd + row * KS);
            }
        } else {
            if (lane < HD / 4) {
                const unsigned voff = (unsigned)(min(row, d.nrows - 1) * RB + 16 * lane);
                dma16(d.rk, voff, d.kd + row * KS);
                dma16(d.rv, voff, d.vd + row * KS);
            }
        }
    };
    auto issue_tile = [&](int j0, int buf) {
        if constexpr (SH) {
            // entries past the list are zero rows (their keys are masked)
#pragma unroll
            for (int i = 0; i < SIPT; i++) {
                const int idx = tid + NTHR * i;
                const int c = idx % CPR, kk = (idx / CPR) % BK;
                const bool isv = idx >= BK * CPR;
                const int li = j0 + kk;
                if (li < shl.nk) {
                    const int ps = shl.pos(li);
                    const uint16_t *src =
                        ps < a.sh.sink
                            ? (isv ? a.sh.v_sink : a.sh.k_sink) +
                                  ((size_t)kvh * kShadowSinkMax + ps) * HD
                            : (isv ? a.sh.v_win : a.sh.k_win) +
                                  ((size_t)kvh * kShadowWinMax + ps % kShadowWinMax) * HD;
                    sraw[i] = *(const u32x4 *)(src + 8 * c);
                } else {
                    sraw[i] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        } else if constexpr (FMT == 0) {
            const RowDma d = row_dma(j0, buf);
#pragma unroll
            for (int i = 0; i < RPW; i++) issue_row(d, i);
        } else {
#pragma unroll
            for (int i = 0; i < Sh::IPT; i++) {
                const int idx = tid + NTHR * i;
                int row, blk;
                q4_item(idx, row, blk);
                const uint8_t *base = idx < BK * NB ? kbase : vbase;
                if (idx < Sh::QITEMS && j0 + row <= q1) {
                    const uint32_t *src = (const uint32_t *)(base + (size_t)(j0 + row) * RB +
                                                             blk * kQ4BlockBytes - 2 * (blk & 1));
#pragma unroll
                    for (int u = 0; u < 5; u++) raw[i][u] = src[u];
                } else {
#pragma unroll
                    for (int u = 0; u < 5; u++) raw[i][u] = 0;
                }
            }
        }
    };

    // Q4_0: decode the staged blocks into LDS buffer `buf`; shadow mode:
    // widen the staged fp16 rows.
    auto store_tile = [&](int buf) {
        if constexpr (SH) {
            float *kd = lds + buf * Sh::BUF;
            float *vd = kd + BK * KS;
#pragma unroll
            for (int i = 0; i < SIPT; i++) {
                const int idx = tid + NTHR * i;
                const int c = idx % CPR, kk = (idx / CPR) % BK;
                float *dst = (idx >= BK * CPR ? vd : kd) + kk * KS + 8 * c;
                const u32x4 r = sraw[i];
                *(f32x4 *)dst = f32x4{lo_h(r[0]), hi_h(r[0]), lo_h(r[1]), hi_h(r[1])};
                *(f32x4 *)(dst + 4) = f32x4{lo_h(r[2]), hi_h(r[2]), lo_h(r[3]), hi_h(r[3])};
            }
        } else if constexpr (FMT == 1) {
            float *kd = lds + buf * Sh::BUF;
            float *vd = kd + BK * KS;
            const NibConsts nk = nib_consts();
#pragma unroll
            for (int i = 0; i < Sh::IPT; i++) {
                const int idx = tid + NTHR * i;
                if (idx < Sh::QITEMS) {
                    int row, blk;
                    q4_item(idx, row, blk);
                    float *dst = (idx < BK * NB ? kd : vd) + row * KS + blk * kQ4Block;
                    const bool odd = (blk & 1) != 0;
                    const BlockScale sc =
                        block_scale(half_bits_to_float(odd ? raw[i][0] >> 16 : raw[i][0]));
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        // code bytes 4q..4q+3 of the block
                        const uint32_t cw = odd ? raw[i][q + 1]
                                                : __builtin_amdgcn_alignbyte(raw[i][q + 1], raw[i][q], 2);
                        float v[8];
                        dequant_word(cw, sc, nk, v);
                        *(f32x4 *)&dst[4 * q] = f32x4{v[0], v[1], v[2], v[3]};
                        *(f32x4 *)&dst[16 + 4 * q] = f32x4{v[4], v[5], v[6], v[7]};
                    }
                }
            }
        }
    };

    // Tile at key jc from LDS buffer `buf`. fp32 launches with `dma`: the
    // next tile's rows (`nd`) are requested into buffer buf ^ 1 during QK.
    auto compute_tile = [&](int jc, int buf, bool dma, const RowDma &nd) {
        const float *Ks = lds + buf * Sh::BUF;
        const float *Vs = Ks + BK * KS;
        constexpr int NBB = Sh::NBB;
        // S^T = K Q^T over the tile's two 16-key sets: in set ks the A row m
        // is key 16 ks + m; MFMA t of group j contracts dims 16 j + 4 k + t
        // (k = the B row, lane group g4), so a lane's K operand of a group is
        // one 16-byte read and its q operands are qr[4 j + t]. Register r of
        // set ks then holds key 16 ks + 4 g4 + r of row n16. LDS reads run one
        // group ahead of the MFMAs that consume them.
        f32x4 s0 = f32x4{}, s1 = f32x4{};
        const float *kr0 = Ks + n16 * KS + 4 * g4;
        const float *kr1 = kr0 + 16 * KS;
        // PV step st (0..7) contracts keys 16 (st >> 2) + 4 k + (st & 3): its
        // B operand is register st & 3 of set st >> 2. Its A operand for
        // output block b is V at dim 64 (b >> 2) + 4 m + (b & 3) of that key
        // (m = lane & 15), so a lane's operands of a step are NBB 16-byte
        // reads of its key's row, contiguous across the 16 lanes of a group.
        auto vread = [&](int st, f32x4 (&vv)[NBB]) {
            const float *vr = Vs + (16 * (st >> 2) + 4 * g4 + (st & 3)) * KS + 4 * n16;
#pragma unroll
            for (int bb = 0; bb < NBB; bb++) vv[bb] = *(const f32x4 *)(vr + 64 * bb);
        };
        constexpr int NJ = HD / 16;
        f32x4 kc0 = *(const f32x4 *)kr0, kc1 = *(const f32x4 *)kr1;
        f32x4 vc[NBB];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            f32x4 kn0 = kc0, kn1 = kc1;
            if (j + 1 < NJ) {
                kn0 = *(const f32x4 *)(kr0 + 16 * (j + 1));
                kn1 = *(const f32x4 *)(kr1 + 16 * (j + 1));
            } else {
                vread(0, vc);     // PV's first operands, read during the last MFMAs
            }
            if constexpr (SPLIT) {
                if (dma && j < RPW) issue_row(nd, j);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                s0 = mfma16(kc0[t], qr[4 * j + t], s0);
                s1 = mfma16(kc1[t], qr[4 * j + t], s1);
            }
            __builtin_amdgcn_sched_barrier(0);
            kc0 = kn0;
            kc1 = kn1;
        }
        const bool shadow_free =
            !shadowed || (jc >= a.sh.sink && (a.sh.win <= 0 || jc + BK - 1 <= pw0 - a.sh.win));
        const bool full = !SH && jc + BK - 1 <= pw0 && shadow_free &&
                          (a.win <= 0 || jc + BK - 1 < a.sink || jc >= pw1 - a.win + 1);
        if (SH) {
            const int lane_li = jc + (lane & 31);
            const int lane_ps = shl.pos(lane_li);
            const bool tag_ok = lane_li < shl.nk && lane_ps >= a.sh.sink &&
                                a.sh.win_pos[lane_ps % kShadowWinMax] == lane_ps;
            const unsigned tags = (unsigned)__ballot(tag_ok);
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int kl = 16 * ks + 4 * g4 + r;
                    const int li = jc + kl;
                    const int ps = shl.pos(li);
                    const bool from_shadow =
                        ps < a.sh.sink || (ps > p_row - a.sh.win && ((tags >> kl) & 1u) != 0);
                    const bool ok = row_live && li < shl.nk && from_shadow &&
                                    in_key_set(ps, p_row, a.sink, a.win);
                    f32x4 &sv = ks ? s1 : s0;
                    sv[r] = ok ? sv[r] : -INFINITY;
                }
            }
        } else if (!full) {
            const int hi_key = row_live ? p_row : -1;
            const int lo_win = a.win > 0 ? p_row - a.win + 1 : 0;
            const int sink_end = a.win > 0 ? min(a.sink, hi_key + 1) : 0;
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int key = jc + 16 * ks + 4 * g4 + r;
                    bool ok = (key <= hi_key) & ((key >= lo_win) | (key < sink_end));
                    if (FMT == 1 && !shadow_free)
                        ok = ok && !shadow_key(a.sh, a.sh.win_pos, key, p_row);
                    f32x4 &sv = ks ? s1 : s0;
                    sv[r] = ok ? sv[r] : -INFINITY;
                }
            }
        }
        float tmax = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                           fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        tmax = half_swap_max(row16_swap_max(tmax));   // over the row's four lane groups
        const bool rebase = tmax > m_run + kTau;
        if (__ballot(rebase)) {
            const float corr = rebase ? fast_exp2(m_run - tmax) : 1.0f;
            if (__ballot(rebase && m_run != -INFINITY)) {
#pragma unroll
                for (int n = 0; n < NO; n++) scale_acc(O[n], corr);
            }
            l_run *= corr;
            m_run = rebase ? tmax : m_run;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            s0[r] = fast_exp2(s0[r] - m_use);
            s1[r] = fast_exp2(s1[r] - m_use);
            psum += s0[r] + s1[r];
        }
        l_run += psum;

        // O^T += V^T P^T
#pragma unroll
        for (int st = 0; st < 8; st++) {
            f32x4 vn[NBB];
            if (st + 1 < 8) vread(st + 1, vn);
            __builtin_amdgcn_sched_barrier(0);
            const float p = (st >> 2) ? s1[st & 3] : s0[st & 3];
#pragma unroll
            for (int bb = 0; bb < NBB; bb++)
#pragma unroll
                for (int e = 0; e < 4; e++) O[4 * bb + e] = mfma16(vc[bb][e], p, O[4 * bb + e]);
            __builtin_amdgcn_sched_barrier(0);
            if (st + 1 < 8) {
#pragma unroll
                for (int bb = 0; bb < NBB; bb++) vc[bb] = vn[bb];
            }
        }
    };

    // Double-buffered walk, one barrier per tile: the barrier makes tile ti
    // (buffer buf) visible and guarantees every wave is done with buf ^ 1,
    // which then receives tile ti + 1 while tile ti is computed.
    lds_barrier();                // the previous segment no longer reads either buffer
    int buf = 0;
    int ti = t_lo;
    prefetch_pages(tile_at(ti));
    issue_tile(tile_at(ti), 0);
    if (PG && ti + 1 < t_hi) prefetch_pages(tile_at(ti + 1));
    store_tile(0);
    load_q();
    while (ti < t_hi) {
        wait_vmem();
        __syncthreads();
        const int jc = tile_at(ti);
        visited++;
        ti++;
        const bool more = ti < t_hi;
        RowDma nd{};
        if (more) {
            // fp32: the row offsets now (paged: from the pages read a tile
            // ahead), the requests during QK
            if constexpr (SPLIT) nd = row_dma(tile_at(ti), buf ^ 1);
            else issue_tile(tile_at(ti), buf ^ 1);
            if (PG && ti + 1 < t_hi) prefetch_pages(tile_at(ti + 1));
        }
        // Every wave computes every tile: for a wave whose rows need none of
        // its keys the tile is fully masked (p = 0, nothing changes). A branch
        // here would make the compiler carry O through VGPR copies.
        compute_tile(jc, buf, SPLIT && more, nd);
        if (more) store_tile(buf ^ 1);
        buf ^= 1;
    }

    // ---- finalise: out = acc / l (whole segment) or this piece's partial
    // a row's l is spread over its four lane groups
    float l_tot = l_run + __shfl_xor(l_run, 32);
    l_tot += __shfl_xor(l_tot, 16);
    float scale_out;
    if (whole && SH) {
        // the row's shadow partial: m, l to the workspace, acc (unnormalised) to out
        const size_t rf = (size_t)(p_row + sg.tok) * a.n_head + kvh * G + g;
        scale_out = 1.0f;
        if (row_live && row_lead) {
            const_cast<float *>(a.sh_m)[rf] = m_run;
            const_cast<float *>(a.sh_l)[rf] = l_tot;
        }
    } else if (whole) {
        const size_t t = (size_t)(p_row + sg.tok);
        scale_out = 1.0f / l_tot;
        // ln sum exp(scale q.k) = ln 2 * (m + log2 l): m is in base-2 units
        if (a.lse && row_live && row_lead)
            a.lse[(size_t)(kvh * G + g) * a.n + t] = (m_run + log2f(l_tot)) * kLn2;
    } else {
        const size_t prow = (size_t)piece * ROWS + row_wg;
        scale_out = 1.0f;
        if (row_lead) {
            a.ws_m[prow] = m_run;
            a.ws_l[prow] = l_tot;
        }
    }
    // O leaves through LDS. A lane's registers hold 16-byte pieces of its
    // own row (through the d permutation), so direct stores would touch 64
    // rows per instruction; staged as rows of stride KS, each store
    // instruction writes whole rows (HD contiguous floats). The staging area
    // is the tile buffers (W * R rows = 4 * BK rows), free once every wave
    // is past the last tile; the next segment's first barrier orders the
    // read-back below before the buffers are refilled. Both barriers order
    // LDS only; this segment's output stores stay in flight.
    lds_barrier();
    float *stg = lds + (size_t)w * Sh::R * KS;
    // block b, register r holds dim 64 (b >> 2) + 16 g4 + 4 r + (b & 3)
#pragma unroll
    for (int r = 0; r < 4; r++) {
#pragma unroll
        for (int bb = 0; bb < Sh::NBB; bb++) {
            float *dst = stg + n16 * KS + 64 * bb + 16 * g4 + 4 * r;
            *(f32x4 *)dst = f32x4{O[4 * bb + 0][r], O[4 * bb + 1][r], O[4 * bb + 2][r],
                                  O[4 * bb + 3][r]} * scale_out;
        }
    }
    wave_lds_sync();
    {
        constexpr int LPR = HD / 4;            // lanes per row (16 bytes each)
        constexpr int RPI = 64 / LPR;          // rows per store instruction
        const int rsub = lane / LPR, c4 = lane % LPR;
#pragma unroll
        for (int i = 0; i < Sh::R / RPI; i++) {
            const int rr = i * RPI + rsub;     // row within the wave
            const int rw = w * Sh::R + rr;     // row within the work-group
            const f32x4 v = *(const f32x4 *)(stg + rr * KS + 4 * c4);
            float *dst;
            bool live = true;
            if (whole) {
                const int pr = q0 + rw / G;
                live = pr <= q1;
                dst = a.out + (((size_t)(pr + sg.tok)) * a.n_head + kvh * G + rw % G) * HD;
            } else {
                dst = a.ws_acc + ((size_t)piece * ROWS + rw) * HD;
            }
            if (live) *(f32x4 *)(dst + 4 * c4) = v;
        }
    }
    };   // run_segment

    if (s_first >= 0 && lo < hi) {
        int F = run_info[2];
        for (int seg = s_first; seg <= s_last; seg++) {
            int cnt;
            const int u = seg_units(seg, &cnt);
            const int T0 = F + kSegUnits;
            // tiles whose first unit lies in [lo, hi)
            auto first_tile_at_or_after = [&](long long x) -> long long {
                return x <= T0 ? 0 : (x - T0 + kTileUnits - 1) / kTileUnits;
            };
            const int t_lo = (int)min(first_tile_at_or_after(lo), (long long)cnt);
            const int t_hi = (int)min(first_tile_at_or_after(hi), (long long)cnt);
            if (t_lo < t_hi) {     // this run owns tiles of the segment
                const int f_owner = owner(T0);
                const bool whole = owner(T0 + (cnt - 1) * kTileUnits) == f_owner;
                int piece = 0;
                if (!whole) {
                    // piece table offset of a cut segment: only the run's
                    // first and last segments can be cut
                    const int P = seg == s_first ? run_info[3] : run_info[5];
                    piece = P + (wg - f_owner);
                }
                run_segment(seg, t_lo, t_hi, whole, piece, f_owner == wg);
            }
            F += u;
        }
    }
    if (!SH && a.stats && tid == 0) {
        atomicAdd(&a.stats[0], (unsigned long long)visited);
        atomicAdd(&a.stats[1], (unsigned long long)skipped);
    }
}

// Merges the pieces of segments cut between work-groups:
// out = sum_p exp2(m_p - M) acc_p / sum_p exp2(m_p - M) l_p, ascending p.
// One work-group per (segment, chunk of kCombineRows rows); whole segments
// return at once. Each thread owns 4 consecutive output dims of one row.
constexpr int kCombineRows = 16;

template <int HD, int G, bool SH>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
    constexpr int ROWS = kPrefillWaves * kPrefillRowsPerWave;
    constexpr int TPR = HD / 4;                    // threads per row
    constexpr int RPP = 256 / TPR;                 // rows per pass
    if ((int)blockIdx.x >= a.cuts->count) return;
    const CutSeg c = a.cuts->seg[blockIdx.x];
    const int np = c.n_pieces, P = c.piece0;
    const int c4 = threadIdx.x % TPR;
#pragma unroll 1
    for (int rr = threadIdx.x / TPR; rr < kCombineRows; rr += RPP) {
        const int row = blockIdx.y * kCombineRows + rr;
        const int p = c.q0 + row / G;
        if (p > c.q1) continue;
        float M = -INFINITY;
        for (int k = 0; k < np; k++) M = fmaxf(M, a.ws_m[(size_t)(P + k) * ROWS + row]);
        f32x4 o = {};
        float L = 0.0f;
        for (int k = 0; k < np; k++) {
            const size_t pr = (size_t)(P + k) * ROWS + row;
            // a piece that saw no key (m = -inf; only shadow-mode rows, whose
            // shadow keys may all be masked) weighs nothing, also when every
            // piece is empty
            const float wgt = a.ws_m[pr] == -INFINITY ? 0.0f : fast_exp2(a.ws_m[pr] - M);
            L += a.ws_l[pr] * wgt;
            o += *(const f32x4 *)(a.ws_acc + pr * HD + 4 * c4) * wgt;
        }
        const int h = c.kvh * G + row % G;
        const size_t t = (size_t)(p + c.tok);
        if constexpr (SH) {
            // merged shadow partial, still unnormalised
            *(f32x4 *)(a.out + (t * a.n_head + h) * HD + 4 * c4) = o;
            if (c4 == 0) {
                const_cast<float *>(a.sh_m)[t * a.n_head + h] = M;
                const_cast<float *>(a.sh_l)[t * a.n_head + h] = L;
            }
        } else {
            *(f32x4 *)(a.out + (t * a.n_head + h) * HD + 4 * c4) = o * (1.0f / L);
            if (a.lse && c4 == 0) a.lse[(size_t)h * a.n + t] = (M + log2f(L)) * kLn2;
        }
    }
}

// Dynamic LDS of a launch: the two K/V buffers, plus the request table of
// a paged batch.
template <int HD, int G, int FMT, int MODE>
size_t lds_bytes(int n_req) {
    return PrefillShape<HD, G, FMT>::LDS_BYTES +
           (MODE == kModePaged ? (size_t)(4 * n_req + 1) * sizeof(int) : 0);
}

template <int HD, int G, int FMT, int MODE>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s) {
    static bool attr_set = false;   // per process; the attribute is per function
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)prefill_kernel<HD, G, FMT, MODE>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)lds_bytes<HD, G, FMT, MODE>(kPagedMaxReqs));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const size_t lds = lds_bytes<HD, G, FMT, MODE>(a.n_req);
    hipLaunchKernelGGL((prefill_kernel<HD, G, FMT, MODE>), dim3(a.n_wg), dim3(64 * kPrefillWaves),
                       lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // fewer cut segments than work-groups
    hipLaunchKernelGGL((prefill_combine_kernel<HD, G, MODE == kModeShadow>),
                       dim3(a.n_wg > 1 ? a.n_wg - 1 : 1,
                            kPrefillWaves * kPrefillRowsPerWave / kCombineRows),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int HD, int FMT, int MODE>
hipError_t by_group(int group, const PrefillArgs &a, hipStream_t s) {
    switch (group) {
    case 1: return launch_one<HD, 1, FMT, MODE>(a, s);
    case 2: return launch_one<HD, 2, FMT, MODE>(a, s);
    case 4: return launch_one<HD, 4, FMT, MODE>(a, s);
    case 8: return launch_one<HD, 8, FMT, MODE>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int FMT, int MODE>
hipError_t by_dim(int head_dim, int group, const PrefillArgs &a, hipStream_t s) {
    switch (head_dim) {
    case 64: return by_group<64, FMT, MODE>(group, a, s);
    case 128: return by_group<128, FMT, MODE>(group, a, s);
    case 256: return by_group<256, FMT, MODE>(group, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(int format, int head_dim, int group, const PrefillArgs &a,
                          hipStream_t s) {
    return format == 0 ? by_dim<0, kModePlain>(head_dim, group, a, s)
                       : by_dim<1, kModePlain>(head_dim, group, a, s);
}

hipError_t launch_paged_prefill(int head_dim, int group, const PrefillArgs &a, hipStream_t s) {
    return by_dim<0, kModePaged>(head_dim, group, a, s);
}

hipError_t launch_shadow_prefill(int head_dim, int group, const PrefillArgs &a, hipStream_t s) {
    return by_dim<0, kModeShadow>(head_dim, group, a, s);
}

}  // namespace fa
