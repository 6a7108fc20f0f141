// Stream-K schedule of the split-KV decode, shared by the decode kernels.
//
// [FA] "Decode-mode flash attention" and fc_attn_dec_plan: every slot's keys
// [0, pos] are cut into splits by the plan, computed on the device from that
// slot's own position. The splits of all (slot, kv head) segments, in order,
// form one list of work items, and a fixed grid of single-wave work-groups
// takes equal contiguous runs of it. A wave folds every split of one segment
// that falls in its run into one running state (consecutive splits are
// consecutive keys) and writes one partial per segment it touches. The list
// and the partial offsets are recomputed by every wave from the device
// positions with wave scans; wave 0 also writes the per-segment partial
// table {first partial, partial count} that the combine reads.
#pragma once

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

// Items (splits) of a slot whose query sits at `pos`; 0 for a position
// outside the cache.
__device__ __forceinline__ int slot_items(int pos, const DecodeArgs &a, int *split_len) {
    if (pos < 0 || pos >= a.max_seq) {
        *split_len = kDecodeKeyTile;
        return 0;
    }
    int n;
    return decode_plan(pos + 1, a.kps, a.cap, kDecodeKeyTile, &n, split_len);
}

// Query position of a slot (paged: the request's last position, its length
// clamped to its block-table row).
template <bool PG>
__device__ __forceinline__ int decode_query_pos(const DecodeArgs &a, int slot) {
    if constexpr (PG) return min(max(a.seq_lens[slot], 0), a.max_seq) - 1;
    else return a.pos[slot];
}

// Segments whose items, query position and item-list offset the scan keeps
// in registers (64 per register), for the partial table and for finding the
// wave's first segment without reading memory again (by then busy with other
// waves' tile loads).
constexpr int kSchedCached = 4;

// Runs wave w's share (of NW waves) of the item list: for every segment its
// run touches, calls run_segment(seg, pos, it_lo, it_hi, partial) with the
// segment's query position, the run's items [it_lo, it_hi) of that segment
// and the index of the partial it writes.
//
// Partial numbering: along the item list, the (wave, segment) pairs that
// touch advance monotonically in both, so the pair (w, s) gets number s + w.
// The numbers are distinct and below nsegs + NW, and the partials of segment
// s are the consecutive numbers s + owner(first item) .. s + owner(last item),
// which is what the partial table records (so no wave but wave 0, which
// writes the table, needs the owner division).
template <bool PG, int WA, int WB, class SegFn>
__device__ __forceinline__ void decode_stream_k(const DecodeArgs &a, int w, int NW, int lane,
                                                SegFn &&run_segment) {
    const int nsegs = a.n_slots * a.n_kv;
    // items and query position of segment s (this lane's of a 64-segment chunk)
    auto seg_info = [&](int s, int &pos) -> int {
        pos = s < nsegs ? decode_query_pos<PG>(a, s / a.n_kv) : -1;
        int sl;
        return s < nsegs ? slot_items(pos, a, &sl) : 0;
    };
    // ---- pass 1: items per segment, each segment's offset F in the item
    // list (an exclusive prefix sum), and the total
    int c_it[kSchedCached], c_pos[kSchedCached], c_F[kSchedCached];
    int total = 0;
#pragma unroll
    for (int c = 0; c < kSchedCached; c++) {
        c_it[c] = 0;
        c_pos[c] = -1;
        c_F[c] = 0;
        if (64 * c < nsegs) {
            c_it[c] = seg_info(64 * c + lane, c_pos[c]);
            const int incl = wave_incl_scan(c_it[c], lane);
            c_F[c] = total + incl - c_it[c];
            total += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
        }
    }
    const int cached_total = total;
    for (int base = 64 * kSchedCached; base < nsegs; base += 64) {
        int pos;
        total += __builtin_amdgcn_readfirstlane(wave_sum_i(seg_info(base + lane, pos)));
    }
    // Run boundaries. With two waves per SIMD (NW = 2 kDecodeSimds), the
    // waves of the first kDecodeSimds work-groups are dispatched first, one
    // per SIMD, and each shares its SIMD with one of the later ones. The
    // issue arbiter favours the older wave, so with equal runs the later
    // waves finished ~10% later and then ran alone with nothing to hide
    // their latencies. Runs are therefore weighted WA : WB in that case
    // (equal otherwise): wave w's run is [total cum(w) / Wt, total cum(w + 1) / Wt).
    const bool paired = NW == 2 * kDecodeSimds;
    const int wa = paired ? WA : 1, wb = paired ? WB : 1;
    const int H = paired ? kDecodeSimds : NW;
    const long long Wt = (long long)wa * H + (long long)wb * (NW - H);
    auto cum = [&](int v) -> long long {
        return v <= H ? (long long)wa * v : (long long)wa * H + (long long)wb * (v - H);
    };
    const long long lo = total * cum(w) / Wt;
    const long long hi = total * cum(w + 1) / Wt;
    // wave owning item f: the last wave whose run starts at or before f, i.e.
    // the largest v with cum(v) <= ((f + 1) Wt - 1) / total
    auto owner = [&](long long f) -> int {
        const long long c = ((f + 1) * Wt - 1) / total;
        const long long v = c < (long long)wa * H ? c / wa : H + (c - (long long)wa * H) / wb;
        return (int)min(v, (long long)NW - 1);
    };

    // ---- the partial table (wave 0): segment s's partials are the numbers
    // s + owner(F_s) .. s + owner(F_s + it_s - 1)
    if (w == 0) {
        auto table = [&](int base, int it, int F) {
            const int s = base + lane;
            if (s < nsegs) {
                const int w0 = it > 0 ? owner(F) : 0;
                a.seg_table[2 * s] = s + w0;
                a.seg_table[2 * s + 1] = it > 0 ? owner(F + it - 1) - w0 + 1 : 0;
            }
        };
#pragma unroll
        for (int c = 0; c < kSchedCached; c++)
            if (64 * c < nsegs) table(64 * c, c_it[c], c_F[c]);
        int f_carry = cached_total;
        for (int base = 64 * kSchedCached; base < nsegs; base += 64) {
            int pos;
            const int it = seg_info(base + lane, pos);
            const int incl = wave_incl_scan(it, lane);
            table(base, it, f_carry + incl - it);
            f_carry += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
        }
    }
    // ---- this wave's first segment: the first one with items past lo (its
    // offset is then <= lo). An empty run (lo = hi, when there are fewer
    // items than waves) lies strictly inside at most one segment, whose
    // partial range then still counts this wave: it writes an empty partial
    // there. From here on the wave's state is scalar.
    const bool empty = lo >= hi;
    int s = -1, Fs = 0, its = 0, poss = -1;
    auto find = [&](int base, int it, int pos, int F) {
        const unsigned long long m = __ballot(it > 0 && F + it > lo && (!empty || F < lo));
        if (m) {
            const int b = __builtin_ctzll(m);
            s = base + b;
            Fs = __builtin_amdgcn_readfirstlane(__shfl(F, b));
            its = __builtin_amdgcn_readfirstlane(__shfl(it, b));
            poss = __builtin_amdgcn_readfirstlane(__shfl(pos, b));
        }
    };
#pragma unroll
    for (int c = 0; c < kSchedCached; c++)
        if (s < 0 && 64 * c < nsegs) find(64 * c, c_it[c], c_pos[c], c_F[c]);
    if (s < 0) {
        int f_carry = cached_total;
        for (int base = 64 * kSchedCached; s < 0 && base < nsegs; base += 64) {
            int pos;
            const int it = seg_info(base + lane, pos);
            const int incl = wave_incl_scan(it, lane);
            find(base, it, pos, f_carry + incl - it);
            f_carry += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
        }
    }
    if (s < 0) return;                         // an empty run on a segment boundary
    if (empty) {
        run_segment(s, poss, (int)lo - Fs, (int)lo - Fs, s + w);
        return;
    }

    // ---- the run: consecutive segments from s while its items last
    for (;;) {
        const int it_lo = (int)max(lo, (long long)Fs) - Fs;
        const int it_hi = (int)min(hi, (long long)Fs + its) - Fs;
        run_segment(s, poss, it_lo, it_hi, s + w);
        Fs += its;
        if (Fs >= hi) break;
        // the next segment with items starts at item Fs
        its = 0;
        while (++s < nsegs) {
            poss = __builtin_amdgcn_readfirstlane(decode_query_pos<PG>(a, s / a.n_kv));
            int sl;
            its = slot_items(poss, a, &sl);
            if (its > 0) break;
        }
        if (its == 0) break;                   // (not reached: Fs < hi <= total)
    }
}

}  // namespace fa
