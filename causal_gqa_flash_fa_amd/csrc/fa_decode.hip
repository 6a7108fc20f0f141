// Multi-slot split-KV decode on fp32 MFMA (gfx950): a partial pass that folds
// key tiles into partials {m, l, acc}, and a combine pass over (slot, head).
//
// Method ([FA] "Decode-mode flash attention", fc_attn_dec_plan and the
// "Multi-user decode attention" section): each slot's keys [0, pos] are cut
// into splits by a plan computed on the device from that slot's own
// position; a partial holds the running max m, running sum l and the
// unnormalised accumulator acc of the keys it folded; the combine rescales
// every partial of a (slot, head) by exp(m_s - M) and divides, in ascending
// order, with no atomics.
//
// MI355X schedule (stream-K over the splits): the splits of all (slot, kv
// head) segments, in order, form one list of work items; a fixed grid of
// single-wave work-groups takes equal contiguous runs of that list. A wave
// folds every split of one segment that falls in its run into one running
// state (consecutive splits are consecutive keys), so it writes one partial
// per segment it touches. Every wave gets the same amount of work whatever
// the context lengths, no work-group sits idle, and a wave streams many tiles
// between its prologue and its partial write. The list and the partial
// offsets are recomputed by every wave from the device positions; wave 0
// also writes the per-segment partial table that the combine reads.
//
// MFMA layout: one query row per slot leaves only G (<= 8) rows per kv head,
// too few for 32x32 or 16x16 tiles, so both contractions use
// v_mfma_f32_4x4x1f32 (16 blocks of 4x4x1, full fp32 rate on gfx950):
//   * QK: lane = key (64-key tiles). Every block gets the same 4 q-head
//     values (A, broadcast from LDS) and its 4 keys' K values (B, decoded in
//     registers): one instruction scores 64 keys x 4 heads for one
//     contraction element, and all G heads reuse each decoded K element.
//   * PV: lanes = output dims. Every block gets the same 4 heads'
//     probabilities of one key (A, from an LDS copy of P) and that key's V
//     values for its 4 dims (B).
// Scores are kept in base-2 units (q pre-scaled by scale*log2 e), so partial
// m values are log2-scaled and the combine uses exp2.
//
// Q4_0 tiles: each lane loads its own key's raw K row into registers (the
// next tile's rows fly during this tile's PV); the raw V tile goes into a
// per-wave LDS buffer by LDS DMA, in flight during QK and softmax. A code
// nibble c becomes (c - 8) * d with one v_fma_mix_f32: the nibble is placed
// in a binary16 whose value is 1024 + c (low nibble) or 1024 + 16 c (high
// nibble), and (1024 + c) * d - 1032 * d, (1024 + 16 c) * (d / 16) - 72 * d
// are exact. PV takes two keys per instruction (lanes 0-31 even keys, 32-63
// odd keys), each lane owning dims that share one block's code bytes, with
// its LDS operands read one step ahead; the two halves are summed at the end.
// fp32 tiles (bound by HBM, one wave per SIMD): QK splits the contraction
// four ways so that four lanes read one key's 64 contiguous bytes at a time,
// PV reads each V row as one vector load per lane, and both stream from
// memory through 16-deep register rings.
//
// The running max is recomputed across the wave only when some score exceeds
// it by more than 8 (base-2 units); any reference max gives the same
// softmax, and the bound keeps every exp2(s - m) <= 256.
#include "fa_device.hpp"
#include "fa_internal.hpp"
#include "fa_shadow.hpp"
#include "fa_decode_sched.hpp"

namespace fa {
namespace {

template <int HD, int G, int FMT>
struct DShape {
    static constexpr int BKD = kDecodeKeyTile;      // keys per tile, one per lane in QK
    static constexpr int NHG = (G + 3) / 4;         // groups of 4 q heads
    static constexpr int HP = NHG * 4;              // padded head count
    // padded LDS q rows: the Q4_0 broadcast reads (HD + 4) and the fp32
    // per-quarter reads (HD + 16: row r starts 64 r bytes into a bank period)
    // hit distinct banks
    static constexpr int QS = FMT == 0 ? HD + 16 : HD + 4;
    static constexpr int PS = BKD + 4;
    static constexpr int NB = HD / kQ4Block;
    static constexpr int RB = FMT == 0 ? HD * 4 : NB * kQ4BlockBytes;
    static constexpr int CB = FMT == 0 ? 16 : RB / 9;   // Q4: 9 chunks of 16 / 8 / 4 bytes per row
    static constexpr int TILE_BYTES = FMT == 0 ? 16 : BKD * RB;
    static constexpr int LPB = 32 / NB;             // Q4 PV: lanes per block per half-wave
    static constexpr int BPL = 16 / LPB;            // Q4 PV: code bytes per lane (4 / 2 / 1)
    static constexpr int OD = FMT == 0 ? HD / 64 : 2 * BPL;   // output dims per lane
};

template <int CB> struct Chunk;
template <> struct Chunk<16> { typedef u32x4 T; };
template <> struct Chunk<8> { typedef u32x2 T; };
template <> struct Chunk<4> { typedef uint32_t T; };

// Output dim of accumulator c in `lane`.
template <int HD, int FMT>
__device__ __forceinline__ int o_dim(int lane, int c) {
    if constexpr (FMT == 0) {
        return (HD / 64) * lane + c;      // consecutive dims per lane: one vector load per V row
    } else {
        using Sh = DShape<HD, 1, 1>;
        const int ll = lane & 31;
        const int bb = ll / Sh::LPB, jb = (ll % Sh::LPB) * Sh::BPL;
        return bb * kQ4Block + jb + (c < Sh::BPL ? c : 16 + c - Sh::BPL);
    }
}

__device__ __forceinline__ float byte_f(uint32_t w, int t) {
    return (float)((w >> (8 * t)) & 0xffu);   // v_cvt_f32_ubyte{t}
}

template <int HD, int G, int FMT, bool PG>
// Q4_0 tiles run two waves per SIMD (bound by issue, the waves hide each
// other's latencies); fp32 tiles one (bound by HBM: the whole register file
// goes to the load rings below, 16 K loads and 16 V rows in flight).
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64), amdgpu_waves_per_eu(FMT == 0 ? 1 : 2)))
void decode_partial_kernel(DecodeArgs a) {
    static_assert(!PG || FMT == 0, "paged caches hold fp32 rows");
    using Sh = DShape<HD, G, FMT>;
    constexpr int BKD = Sh::BKD, NHG = Sh::NHG, HP = Sh::HP, QS = Sh::QS, PS = Sh::PS;
    constexpr int NB = Sh::NB, RB = Sh::RB, CB = Sh::CB, BPL = Sh::BPL, OD = Sh::OD;
    constexpr float TAU = 8.0f;
    typedef typename Chunk<CB>::T chunk_t;

    __shared__ __attribute__((aligned(16))) float Qs[HP * QS];
    __shared__ __attribute__((aligned(16))) float Pw[HP * PS];
    __shared__ __attribute__((aligned(16))) uint8_t Rw[Sh::TILE_BYTES];

    const int lane = threadIdx.x;
    // fp16-shadow work items first (Q4_0 only), with this work-group's LDS:
    // they are short and finish while the stream-K waves below run
    if constexpr (FMT == 1) {
        if ((int)blockIdx.x < a.sh_waves) {
            shadow_pass_wave<HD, G>(a.shp, blockIdx.x, Qs, Pw, (int *)Rw);
            return;
        }
    }
    const int w = blockIdx.x - (FMT == 1 ? a.sh_waves : 0);
    const int NW = gridDim.x - (FMT == 1 ? a.sh_waves : 0);
    unsigned vis = 0, skp = 0;

    // ---- per-segment fold of items [it_lo, it_hi) into one partial
    auto run_segment = [&](int seg, int pos_seg, int it_lo, int it_hi, int pidx) {
        const int slot = seg / a.n_kv, kvh = seg % a.n_kv;
        const int pos = pos_seg;
        const bool shadowed = a.sh.sink > 0 || a.sh.win > 0;
        const int *wpos = a.sh.win_pos + (size_t)slot * kShadowWinMax;
        int split_len;
        slot_items(pos, a, &split_len);
        const int L = pos + 1;
        const int k_lo = it_lo * split_len;
        const int k_hi = min(L, it_hi * split_len);

        // q rows of the group (contiguous in memory) -> Qs, scaled; rows
        // past G are zero. All loads are issued before the first store.
        {
            constexpr int NQ = HP * HD / 256;   // float4 per lane
            const float *qg = a.q + ((size_t)slot * a.n_head + kvh * G) * HD;
            f32x4 qv[NQ];
#pragma unroll
            for (int i = 0; i < NQ; i++) {
                const int f = 4 * (lane + 64 * i);
                qv[i] = f / HD < G ? *(const f32x4 *)(qg + f) : f32x4{};
            }
            wave_lds_sync();      // previous segment done with Qs
#pragma unroll
            for (int i = 0; i < NQ; i++) {
                const int f = 4 * (lane + 64 * i);
                *(f32x4 *)&Qs[(f / HD) * QS + f % HD] = qv[i] * a.qscale;
            }
        }
        wave_lds_sync();

        float m[HP], l[HP];
        f32x4 O[OD][NHG];
#pragma unroll
        for (int h = 0; h < HP; h++) {
            m[h] = -INFINITY;
            l[h] = 0.0f;
        }
#pragma unroll
        for (int c = 0; c < OD; c++)
#pragma unroll
            for (int hg = 0; hg < NHG; hg++) O[c][hg] = f32x4{};

        const size_t head_rows = ((size_t)slot * a.n_kv + kvh) * a.max_seq;
        const uint8_t *kb = (const uint8_t *)a.k + head_rows * RB;
        const uint8_t *vb = (const uint8_t *)a.v + head_rows * RB;
        const int win_first = pos - a.win + 1;     // first key of the recent window

        // first visited tile at or after j ([FA] fc_attn_tile_in_window)
        auto next_visited = [&](int j) -> int {
            if (j < k_hi && a.win > 0 && j >= a.sink && min(j + BKD - 1, k_hi - 1) < win_first) {
                const int jn = (win_first / BKD) * BKD;    // tile holding the window's first key
                const int stop = min(jn, k_hi);
                skp += (unsigned)((stop - j + BKD - 1) / BKD);
                return jn >= k_hi ? k_hi : jn;
            }
            return j;
        };

        // softmax of one tile's scores; lane = key, register = head in group
        auto softmax_tile = [&](f32x4 (&sacc)[NHG], bool kval, int pslot) {
#pragma unroll
            for (int hg = 0; hg < NHG; hg++) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int h = 4 * hg + i;
                    const float s = kval ? sacc[hg][i] : -INFINITY;
                    if (__ballot(s > m[h] + TAU)) {
                        const float m_new = fmaxf(m[h], wave_max(s));
                        const float corr = fast_exp2(m[h] - m_new);
                        m[h] = m_new;
                        l[h] *= corr;
#pragma unroll
                        for (int c = 0; c < OD; c++) O[c][hg][i] *= corr;
                    }
                    // a masked key adds nothing, also while no key has been seen
                    // (m = -inf; fp16-shadow keys can mask whole tiles)
                    const float p = kval ? fast_exp2(s - m[h]) : 0.0f;
                    l[h] += p;
                    Pw[h * PS + pslot] = p;
                }
            }
        };

        const float *qlane = Qs + (lane & 3) * QS;

        if constexpr (FMT == 0) {
            // ---------------- fp32 tiles: direct row reads, software-pipelined
            // At 4 FLOP per byte the fp32 tile is bound by memory, so:
            //  * K rows are read 64 contiguous bytes at a time. The 16 blocks
            //    of each QK MFMA split the contraction in four instead of
            //    covering 64 keys: block 4 kg + u takes keys 4 kg + j
            //    (j = lane & 3) of a 16-key set and the dims of quarter u of
            //    every 16-dim chunk, so the 4 lanes of one key (u = 0..3)
            //    load its 64 bytes of a chunk together (a lane per key
            //    loading 16 bytes touched 64 rows per instruction, ~20%
            //    slower). Key set s of the tile accumulates in acc[s]; at the
            //    end the four quarter sums are added across lanes (xor 4, 8)
            //    and lane l keeps key set u(l): lane l holds key
            //    K(l) = 16 u + 4 kg + j, a fixed permutation of the tile.
            //  * Both operands stream through register rings: K KD loads
            //    ahead of the MFMAs (the next tile's first KD during this
            //    tile's PV), V (lanes = dims) VD rows ahead (the tile's first
            //    VD before QK). Rows past k_hi repeat row k_hi - 1 (their
            //    keys are masked, so V only has to be finite). A lane owns
            //    VPR consecutive output dims, so a V row is one vector load
            //    per lane. Scheduling
            //    fences keep every load where it is written (the scheduler
            //    would otherwise sink the ring loads next to their uses to
            //    save registers), and LDS operands are read one step ahead.
            constexpr int NCH = HD / 16;                // 16-dim chunks per row
            constexpr int NKL = 4 * NCH;                // K loads per tile (chunk, key set)
            // K loads in flight: 16 (deeper rings timed the same); with one
            // wave per SIMD there are registers for them beside the
            // accumulators of 8 heads (two waves per SIMD had left room for 8,
            // and streamed ~2% slower)
            constexpr int KD = NKL < 16 ? NKL : 16;
            constexpr int VD = 16;                      // V rows in flight
            constexpr int VPR = HD / 64;                // V floats per lane per row (= OD)
            const int qu = (lane >> 2) & 3;             // contraction quarter of this lane
            const int kl = 4 * (lane >> 4) + (lane & 3);   // key of this lane in a 16-key set
            const int kperm = 16 * qu + kl;             // the tile key this lane ends up with
            f32x4 kring[KD];
            float vring[VD][VPR];
            // Paged: byte offset (from the cache base) of kv head kvh's row
            // `row`; wave-uniform. A 16-key set starts at a multiple of 16
            // and block_size is one too, so the set's rows are consecutive
            // rows of one page: the set needs one lookup. Table indices and
            // page ids are clamped into range; rows past k_hi are masked
            // keys (K) or replaced by row k_hi - 1 (V).
            const int *btr = PG ? a.block_table + (size_t)slot * a.bt_stride : nullptr;
            const size_t rowb = (size_t)a.n_kv * HD * sizeof(float);   // bytes between page rows
            // The table is read through the constant address space: the
            // entry is a scalar load, counted apart from the vector loads in
            // flight, so reading it never drains the K and V rings.
            auto row_off = [&](int row) -> size_t {
                const int ru = __builtin_amdgcn_readfirstlane(row);
                const int pi = ru / a.block_size;
                const __attribute__((address_space(4))) int *bt4 =
                    (const __attribute__((address_space(4))) int *)(btr + min(pi, a.bt_stride - 1));
                const int pg = min(max(*bt4, 0), a.num_blocks - 1);
                return (size_t)pg * (size_t)a.blk_stride * sizeof(float) +
                       (size_t)(ru - pi * a.block_size) * rowb + (size_t)kvh * HD * sizeof(float);
            };
            size_t set_off[4] = {0, 0, 0, 0}, next_off[4] = {0, 0, 0, 0};
            const size_t last_off = PG ? row_off(k_hi - 1) : 0;
            // load c = 4 * chunk + key set
            // K and V rows are read once per call: non-temporal loads (the
            // 64-slot fp32 decode streamed 4.8 GB in 0.735 instead of 0.770 ms;
            // for Q4_0 rows, 144 bytes that share cache lines, the same hint
            // was slower)
            auto kload_at = [&](int j, int c, const size_t (&off)[4]) -> f32x4 {
                if constexpr (PG) {
                    return __builtin_nontemporal_load(
                        (const f32x4 *)((const uint8_t *)a.k + off[c & 3] + kl * rowb +
                                        64 * (c >> 2) + 16 * qu));
                } else {
                    const int row = min(j + 16 * (c & 3) + kl, k_hi - 1);
                    return __builtin_nontemporal_load(
                        (const f32x4 *)(kb + (size_t)row * RB + 64 * (c >> 2) + 16 * qu));
                }
            };
            auto kload = [&](int j, int c) -> f32x4 { return kload_at(j, c, set_off); };
            // lane holds dims VPR * lane .. VPR * lane + VPR - 1: a row is one
            // vector load per lane
            auto vload = [&](int j, int r, float (&dst)[VPR]) {
                const float *vr;
                if constexpr (PG) {
                    const size_t o = j + r < k_hi ? set_off[r >> 4] + (size_t)(r & 15) * rowb : last_off;
                    vr = (const float *)((const uint8_t *)a.v + o) + VPR * lane;
                } else {
                    vr = (const float *)(vb + (size_t)min(j + r, k_hi - 1) * RB) + VPR * lane;
                }
                if constexpr (VPR == 4) {
                    const f32x4 x = __builtin_nontemporal_load((const f32x4 *)vr);
                    dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
                } else if constexpr (VPR == 2) {
                    const f32x2 x = __builtin_nontemporal_load((const f32x2 *)vr);
                    dst[0] = x[0]; dst[1] = x[1];
                } else {
                    dst[0] = __builtin_nontemporal_load(vr);
                }
            };
            int j = next_visited(k_lo);
            if (j < k_hi) {
                if constexpr (PG) {
#pragma unroll
                    for (int ks = 0; ks < 4; ks++) set_off[ks] = row_off(j + 16 * ks);
                }
#pragma unroll
                for (int c = 0; c < KD; c++) kring[c] = kload(j, c);
            }
            while (j < k_hi) {
                vis++;
                const int jn = next_visited(j + BKD);
                if constexpr (PG) {
                    // the next tile's pages, read a tile ahead of its first K loads
                    if (jn < k_hi) {
#pragma unroll
                        for (int ks = 0; ks < 4; ks++) next_off[ks] = row_off(jn + 16 * ks);
                    }
                }
                const int key = j + kperm;
                const bool kval = key < k_hi && in_key_set(key, pos, a.sink, a.win);
#pragma unroll
                for (int r = 0; r < VD; r++) vload(j, r, vring[r]);
                f32x4 acc[4][NHG];
#pragma unroll
                for (int ks = 0; ks < 4; ks++)
#pragma unroll
                    for (int hg = 0; hg < NHG; hg++) acc[ks][hg] = f32x4{};
                // q operand of chunk b: heads 4 hg + (lane & 3), dims of quarter qu
                auto qread = [&](int b, f32x4 (&qv)[NHG]) {
#pragma unroll
                    for (int hg = 0; hg < NHG; hg++)
                        qv[hg] = *(const f32x4 *)(qlane + hg * 4 * QS + 16 * b + 4 * qu);
                };
                f32x4 qc[NHG];
                qread(0, qc);
#pragma unroll
                for (int b = 0; b < NCH; b++) {
                    f32x4 kv[4];
#pragma unroll
                    for (int ks = 0; ks < 4; ks++) {
                        const int c = 4 * b + ks;
                        kv[ks] = kring[c % KD];
                        if (c + KD < NKL) kring[c % KD] = kload(j, c + KD);
                    }
                    f32x4 qn[NHG];
                    if (b + 1 < NCH) qread(b + 1, qn);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < 4; t++)
#pragma unroll
                        for (int ks = 0; ks < 4; ks++)
#pragma unroll
                            for (int hg = 0; hg < NHG; hg++)
                                acc[ks][hg] = mfma4(qc[hg][t], kv[ks][t], acc[ks][hg]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (b + 1 < NCH) {
#pragma unroll
                        for (int hg = 0; hg < NHG; hg++) qc[hg] = qn[hg];
                    }
                }
                // quarter sums across the lanes of one key, then key set qu
                f32x4 sacc[NHG];
#pragma unroll
                for (int hg = 0; hg < NHG; hg++) {
#pragma unroll
                    for (int ks = 0; ks < 4; ks++) {
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            float x = acc[ks][hg][i];
                            x += __shfl_xor(x, 4);
                            x += __shfl_xor(x, 8);
                            acc[ks][hg][i] = x;
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        sacc[hg][i] = qu == 0 ? acc[0][hg][i]
                                    : qu == 1 ? acc[1][hg][i]
                                    : qu == 2 ? acc[2][hg][i] : acc[3][hg][i];
                }
                softmax_tile(sacc, kval, kperm);
                wave_lds_sync();
                const float *plane = Pw + (lane & 3) * PS;
                auto pread = [&](int t4, f32x4 (&pa)[NHG]) {
#pragma unroll
                    for (int hg = 0; hg < NHG; hg++)
                        pa[hg] = *(const f32x4 *)(plane + hg * 4 * PS + 4 * t4);
                };
                f32x4 pa[NHG];
                pread(0, pa);
#pragma unroll
                for (int r = 0; r < BKD; r++) {
                    const int t = r & 3;
                    float vv[VPR];
#pragma unroll
                    for (int c = 0; c < VPR; c++) vv[c] = vring[r % VD][c];
                    if (r + VD < BKD) vload(j, r + VD, vring[r % VD]);
                    // the next tile's first K chunks fly during the rest of PV
                    if (r == BKD - KD && jn < k_hi) {
#pragma unroll
                        for (int c = 0; c < KD; c++) kring[c] = kload_at(jn, c, next_off);
                    }
                    f32x4 pn[NHG];
                    if (t == 3 && r + 1 < BKD) pread((r + 1) / 4, pn);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int c = 0; c < VPR; c++)
#pragma unroll
                        for (int hg = 0; hg < NHG; hg++)
                            O[c][hg] = mfma4(pa[hg][t], vv[c], O[c][hg]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (t == 3 && r + 1 < BKD) {
#pragma unroll
                        for (int hg = 0; hg < NHG; hg++) pa[hg] = pn[hg];
                    }
                }
                wave_lds_sync();
                j = jn;
                if constexpr (PG) {
#pragma unroll
                    for (int ks = 0; ks < 4; ks++) set_off[ks] = next_off[ks];
                }
            }
        } else {
            // ---------------- Q4_0 tiles
            // K: lane = key; each lane loads its key's raw row into
            // registers, requested right after the previous tile's QK so it
            // flies during that tile's softmax and PV. V: the raw tile goes
            // straight into the wave's LDS buffer by DMA, requested at the
            // start of the tile (after the K rows have landed) so it flies
            // during QK and softmax. The descriptor covers exactly the rows
            // that exist: the buffer range check (per dword) returns zeros
            // past them, so rows past the end of a partial tile arrive as
            // all-zero blocks (scale 0) and masked keys (p = 0) add exact
            // zeros. The compiler does not count LDS DMA in its own
            // vmcnt bookkeeping, hence the explicit waits and this order: no
            // compiler-inserted wait for K ever sits behind a pending DMA.
            constexpr int NI = (Sh::TILE_BYTES + 1023) / 1024;   // V DMA instructions per tile
            chunk_t kr[9];
            auto fetch_k = [&](int j) {
                const chunk_t *src = (const chunk_t *)(kb + (size_t)min(j + lane, k_hi - 1) * RB);
#pragma unroll
                for (int i = 0; i < 9; i++) kr[i] = src[i];
            };
            auto dma_v = [&](int j) {
                const unsigned bytes = (unsigned)(min(BKD, k_hi - j) * RB);
                const __amdgpu_buffer_rsrc_t rs = raw_rsrc(vb + (size_t)j * RB, bytes);
#pragma unroll
                for (int c = 0; c < NI; c++) {
                    const unsigned o = (unsigned)(1024 * c + 16 * lane);
                    // only the last instruction can reach past the tile
                    if (c < NI - 1 || Sh::TILE_BYTES % 1024 == 0 || o < (unsigned)Sh::TILE_BYTES)
                        dma16(rs, o, Rw + 1024 * c);
                }
            };
            const NibConsts nk = nib_consts();
            int j = next_visited(k_lo);
            if (j < k_hi) fetch_k(j);
            while (j < k_hi) {
                const int tj = j;
                vis++;
                wait_vmem_le<0>();                    // this tile's K rows; nothing else in flight
                dma_v(tj);                            // Rw is free: the last PV ended with a sync
                uint32_t rw[RB / 4];
#pragma unroll
                for (int i = 0; i < 9; i++) {
                    if constexpr (CB == 16) {
                        rw[4 * i] = kr[i][0]; rw[4 * i + 1] = kr[i][1];
                        rw[4 * i + 2] = kr[i][2]; rw[4 * i + 3] = kr[i][3];
                    } else if constexpr (CB == 8) {
                        rw[2 * i] = kr[i][0]; rw[2 * i + 1] = kr[i][1];
                    } else {
                        rw[i] = kr[i];
                    }
                }

                // QK: 2 accumulator chains per head group, issued so that an
                // MFMA's accumulator was last written 2 * NHG instructions
                // earlier, not by the one just before; step st covers code
                // word q = st % 4 of block blk = st / 4. The q
                // operands of the next step are read before this step's MFMAs
                // (fenced so the scheduler keeps them there).
                const int key = tj + lane;
                // fp16-shadow keys are folded by the shadow pass, not here
                const bool kval = key < k_hi && in_key_set(key, pos, a.sink, a.win) &&
                                  !(shadowed && shadow_key(a.sh, wpos, key, pos));
                f32x4 sacc2[NHG][2];
#pragma unroll
                for (int hg = 0; hg < NHG; hg++) sacc2[hg][0] = sacc2[hg][1] = f32x4{};
                constexpr int NST = NB * 4;
                auto qread = [&](int st, f32x4 (&qa)[NHG], f32x4 (&qh)[NHG]) {
                    const int blk = st >> 2, q = st & 3;
#pragma unroll
                    for (int hg = 0; hg < NHG; hg++) {
                        const float *qb = qlane + hg * 4 * QS + blk * kQ4Block;
                        qa[hg] = *(const f32x4 *)(qb + 4 * q);
                        qh[hg] = *(const f32x4 *)(qb + 16 + 4 * q);
                    }
                };
                f32x4 qa[NHG], qh[NHG];
                qread(0, qa, qh);
                BlockScale sc{};
#pragma unroll
                for (int st = 0; st < NST; st++) {
                    const int blk = st >> 2, q = st & 3;
                    const int dw = blk * kQ4BlockBytes / 4;
                    const bool odd = (blk & 1) != 0;   // odd blocks start 2 bytes into a dword
                    if (q == 0)
                        sc = block_scale(half_bits_to_float(odd ? (rw[dw] >> 16) : (rw[dw] & 0xffffu)));
                    const uint32_t cw = odd ? rw[dw + 1 + q]
                                            : __builtin_amdgcn_alignbyte(rw[dw + q + 1], rw[dw + q], 2);
                    float kv[8];
                    dequant_word(cw, sc, nk, kv);      // elements blk*32 + 4q + t, blk*32 + 16 + 4q + t
                    f32x4 na[NHG], nh[NHG];
                    if (st + 1 < NST) qread(st + 1, na, nh);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int t = 0; t < 4; t++)
#pragma unroll
                        for (int hg = 0; hg < NHG; hg++)
                            sacc2[hg][t & 1] = mfma4(qa[hg][t], kv[t], sacc2[hg][t & 1]);
#pragma unroll
                    for (int t = 0; t < 4; t++)
#pragma unroll
                        for (int hg = 0; hg < NHG; hg++)
                            sacc2[hg][t & 1] = mfma4(qh[hg][t], kv[4 + t], sacc2[hg][t & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (st + 1 < NST) {
#pragma unroll
                        for (int hg = 0; hg < NHG; hg++) {
                            qa[hg] = na[hg];
                            qh[hg] = nh[hg];
                        }
                    }
                }
                j = next_visited(tj + BKD);
                const bool more = j < k_hi;
                f32x4 sacc[NHG];
#pragma unroll
                for (int hg = 0; hg < NHG; hg++)
                    sacc[hg] = sacc2[hg][0] + sacc2[hg][1];
                softmax_tile(sacc, kval, (lane & 1) * 32 + (lane >> 1));   // even keys, then odd

                wait_vmem_le<0>();                    // this tile's V bytes (nothing else in flight)
                wave_lds_sync();

                // PV: lanes 0-31 even keys, lanes 32-63 odd keys
                const int hk = lane >> 5;
                const int ll = lane & 31;
                const int bb = ll / Sh::LPB, jb = (ll % Sh::LPB) * BPL;
                const float *plane = Pw + (lane & 3) * PS + hk * 32;
                // Step i (t4 = i / 4, u = i % 4) takes key 2 i + hk. Its LDS
                // operands (block scale, code bytes; P values at each t4) are
                // read one step ahead, fenced so the scheduler keeps them
                // there, so LDS latency hides behind the previous step's
                // MFMAs. Fully unrolled: the compiler guards the first V read
                // with a wait for all outstanding memory operations (it
                // cannot tell the DMA is done), so the next tile's K rows are
                // requested only after the first t4 block, and fly during the
                // rest of PV.
                // raw LDS values only: any arithmetic on them here would make
                // the compiler wait for the reads just issued
                auto vread = [&](int i, uint32_t (&r)[3]) {
                    const uint8_t *vr = Rw + (2 * i + hk) * RB + bb * kQ4BlockBytes;
                    r[0] = *(const uint16_t *)vr;
                    if constexpr (BPL == 4) {
                        r[1] = *(const uint16_t *)(vr + 2 + jb);
                        r[2] = *(const uint16_t *)(vr + 4 + jb);
                    } else if constexpr (BPL == 2) {
                        r[1] = *(const uint16_t *)(vr + 2 + jb);
                    } else {
                        r[1] = vr[2 + jb];
                    }
                };
                auto pread = [&](int t4, f32x4 (&pa)[NHG]) {
#pragma unroll
                    for (int hg = 0; hg < NHG; hg++)
                        pa[hg] = *(const f32x4 *)(plane + hg * 4 * PS + 4 * t4);
                };
                uint32_t vr_c[3] = {0, 0, 0};
                f32x4 pa_c[NHG];
                vread(0, vr_c);
                pread(0, pa_c);
#pragma unroll
                for (int i = 0; i < 32; i++) {
                    const int t4 = i >> 2, u = i & 3;
                    if (i == 4 && more) fetch_k(j);
                    uint32_t vr_n[3] = {0, 0, 0};
                    f32x4 pa_n[NHG];
                    if (i + 1 < 32) vread(i + 1, vr_n);
                    if (u == 3 && t4 + 1 < 8) pread(t4 + 1, pa_n);
                    __builtin_amdgcn_sched_barrier(0);
                    const float d = half_bits_to_float(vr_c[0]);
                    const uint32_t cw_c = BPL == 4 ? vr_c[1] | (vr_c[2] << 16) : vr_c[1];
                    float vv[OD];
                    if constexpr (BPL == 4) {
                        dequant_word(cw_c, block_scale(d), nk, vv);   // elements jb + t, 16 + jb + t
                    } else {
                        const float m8d = -8.0f * d;
#pragma unroll
                        for (int b = 0; b < BPL; b++) {
                            vv[b] = fmaf(byte_f(cw_c & 0x0f0f0f0fu, b), d, m8d);
                            vv[BPL + b] = fmaf(byte_f((cw_c >> 4) & 0x0f0f0f0fu, b), d, m8d);
                        }
                    }
#pragma unroll
                    for (int c = 0; c < OD; c++)
#pragma unroll
                        for (int hg = 0; hg < NHG; hg++)
                            O[c][hg] = mfma4(pa_c[hg][u], vv[c], O[c][hg]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = 0; r < 3; r++) vr_c[r] = vr_n[r];
                    if (u == 3 && t4 + 1 < 8) {
#pragma unroll
                        for (int hg = 0; hg < NHG; hg++) pa_c[hg] = pa_n[hg];
                    }
                }
                wave_lds_sync();                      // Rw and Pw free again
            }
#pragma unroll
            for (int c = 0; c < OD; c++)
#pragma unroll
                for (int hg = 0; hg < NHG; hg++)
#pragma unroll
                    for (int i = 0; i < 4; i++) O[c][hg][i] += __shfl_xor(O[c][hg][i], 32);
        }

        // ---- this segment's partial: m, l and acc for the G heads
#pragma unroll
        for (int h = 0; h < HP; h++) l[h] = wave_sum(l[h]);
        const size_t pbase = (size_t)pidx * G;
        if (lane < G) {
            float mv = 0.0f, lv = 0.0f;
#pragma unroll
            for (int h = 0; h < HP; h++)
                if (h == lane) {
                    mv = m[h];
                    lv = l[h];
                }
            a.ws_m[pbase + lane] = mv;
            a.ws_l[pbase + lane] = lv;
        }
        if (FMT == 0 || lane < 32) {
#pragma unroll
            for (int c = 0; c < OD; c++)
#pragma unroll
                for (int hg = 0; hg < NHG; hg++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (4 * hg + i < G)
                            a.ws_acc[(pbase + 4 * hg + i) * HD + o_dim<HD, FMT>(lane, c)] = O[c][hg][i];
        }
    };

    decode_stream_k<PG, kDecodeWeightFirst, kDecodeWeightSecond>(a, w, NW, lane, run_segment);

    if (a.stats && lane == 0) {
        atomicAdd(&a.stats[0], (unsigned long long)vis);
        atomicAdd(&a.stats[1], (unsigned long long)skp);
    }
}

// out = sum_r exp2(m_r - M) acc_r / sum_r exp2(m_r - M) l_r over the
// segment's partials in ascending order, then its fp16-shadow partials.
// One wave per (slot, head); lane e owns the V = HD/64 consecutive output
// elements from V*e. The partials are taken in chunks of up to CH: lane u
// loads m and l of the chunk's partial u, every lane loads its V elements of
// each of the chunk's accumulators (one 4V-byte load per partial), and all of
// a chunk's loads are in flight at once. The chunk max and the sum of the
// weighted l are wave reductions; the weight exp2(m_u - M) of partial u is
// computed by lane u and read back with readlane. When a later chunk (or a
// shadow partial) raises M, the sums so far are rescaled by
// exp2(M_old - M_new); with at most CH partials this is exactly the two-pass
// form: one max, then the weighted sums.
template <int HD, int G>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
    constexpr int V = HD / 64;
    constexpr int CH = 32;
    typedef float vec __attribute__((ext_vector_type(V)));
    const int gh = blockIdx.x;              // slot * n_head + head
    const int slot = gh / a.n_head, h = gh % a.n_head;
    const int seg = slot * a.n_kv + h / G, g = h % G;
    const int P = a.seg_table[2 * seg], n = a.seg_table[2 * seg + 1];
    const int lane = threadIdx.x;
    float M = -INFINITY, L = 0.0f;
    vec o = 0.0f;
    // move the reference max up to m_new (uniform), rescaling the sums so far
    auto rebase = [&](float m_new) {
        if (m_new > M) {
            const float cs = M == -INFINITY ? 0.0f : fast_exp2(M - m_new);
            L *= cs;
            o *= cs;
            M = m_new;
        }
    };
    for (int r0 = 0; r0 < n; r0 += CH) {
        const int cnt = min(CH, n - r0);
        const size_t p0 = (size_t)(P + r0) * G + g;   // (partial r0, head g)
        float mu = -INFINITY, lu = 0.0f;
        if (lane < cnt) {
            mu = a.ws_m[p0 + (size_t)lane * G];
            lu = a.ws_l[p0 + (size_t)lane * G];
        }
        vec x[CH];
#pragma unroll
        for (int u = 0; u < CH; u++)
            x[u] = u < cnt ? *(const vec *)(a.ws_acc + (p0 + (size_t)u * G) * HD + lane * V)
                           : vec(0.0f);
        rebase(wave_max(mu));
        // an empty partial (m = -inf: a split whose keys all come from the
        // fp16 shadow) weighs 0, also while M is still -inf
        const float wu = mu == -INFINITY ? 0.0f : fast_exp2(mu - M);
        L += wave_sum(lu * wu);
#pragma unroll
        for (int u = 0; u < CH; u++) {
            if (u < cnt) {
                const float wgt = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wu), u));
                o += x[u] * wgt;
            }
        }
    }
    for (int c = 0; c < a.sh_groups; c++) {   // fp16-shadow partials of the segment
        const size_t pi = ((size_t)seg * a.sh_groups + c) * G + g;
        const float m = a.sh_m[pi];
        if (m == -INFINITY) continue;            // no shadow key: weight 0
        rebase(m);
        const float wgt = fast_exp2(m - M);
        L += a.sh_l[pi] * wgt;
        o += *(const vec *)(a.sh_acc + pi * HD + lane * V) * wgt;
    }
    const vec r = o / L;                        // no partial (bad position): 0/0 = NaN
    float *dst = a.out + (size_t)gh * HD + lane * V;
    if (((uintptr_t)a.out & (sizeof(vec) - 1)) == 0) {
        *(vec *)dst = r;
    } else {                                    // out is only 4-byte aligned
#pragma unroll
        for (int i = 0; i < V; i++) dst[i] = r[i];
    }
    // ln sum exp(scale q.k) = ln 2 * (M + log2 L): partial m are in base-2 units
    if (a.lse && lane == 0) a.lse[(size_t)h * a.n_slots + slot] = (M + log2f(L)) * kLn2;
}

template <int HD, int G, int FMT, bool PG>
hipError_t launch_one(const DecodeArgs &a, int waves, hipStream_t s) {
    hipLaunchKernelGGL((decode_partial_kernel<HD, G, FMT, PG>), dim3(waves + a.sh_waves), dim3(64),
                       0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<HD, G>), dim3(a.n_slots * a.n_head), dim3(64), 0, s,
                       a);
    return hipGetLastError();
}

template <int HD, int FMT, bool PG>
hipError_t by_group(int group, const DecodeArgs &a, int waves, hipStream_t s) {
    switch (group) {
    case 1: return launch_one<HD, 1, FMT, PG>(a, waves, s);
    case 2: return launch_one<HD, 2, FMT, PG>(a, waves, s);
    case 4: return launch_one<HD, 4, FMT, PG>(a, waves, s);
    case 8: return launch_one<HD, 8, FMT, PG>(a, waves, s);
    }
    return hipErrorInvalidValue;
}

template <int FMT, bool PG>
hipError_t by_dim(int head_dim, int group, const DecodeArgs &a, int waves, hipStream_t s) {
    switch (head_dim) {
    case 64: return by_group<64, FMT, PG>(group, a, waves, s);
    case 128: return by_group<128, FMT, PG>(group, a, waves, s);
    case 256: return by_group<256, FMT, PG>(group, a, waves, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(int format, int head_dim, int group, const DecodeArgs &a, int waves,
                         hipStream_t s) {
    return format == 0 ? by_dim<0, false>(head_dim, group, a, waves, s)
                       : by_dim<1, false>(head_dim, group, a, waves, s);
}

hipError_t launch_paged_decode(int head_dim, int group, const DecodeArgs &a, int waves,
                               hipStream_t s) {
    return by_dim<0, true>(head_dim, group, a, waves, s);
}

hipError_t launch_decode_combine(int head_dim, int group, const DecodeArgs &a, hipStream_t s) {
    const dim3 grid(a.n_slots * a.n_head);
#define FA_COMBINE(HD, G)                                                                      \
    if (head_dim == HD && group == G) {                                                        \
        hipLaunchKernelGGL((decode_combine_kernel<HD, G>), grid, dim3(64), 0, s, a);           \
        return hipGetLastError();                                                              \
    }
    FA_COMBINE(64, 1) FA_COMBINE(64, 2) FA_COMBINE(64, 4) FA_COMBINE(64, 8)
    FA_COMBINE(128, 1) FA_COMBINE(128, 2) FA_COMBINE(128, 4) FA_COMBINE(128, 8)
    FA_COMBINE(256, 1) FA_COMBINE(256, 2) FA_COMBINE(256, 4) FA_COMBINE(256, 8)
#undef FA_COMBINE
    return hipErrorInvalidValue;
}

}  // namespace fa
