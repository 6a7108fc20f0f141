// Attention over the fp16 shadow keys of a Q4_0 cache, for decode.
//
// [FA] "fp16 sink + recent-window exemption" (fc_kvq4_is_fp16 and the fp16
// read paths of the Q4 decode): for a query at position p, key s is read from
// the fp16 shadow instead of the Q4_0 body iff s is a sink position or lies
// in the recent window of p and the window ring still holds it. That key set
// is small (at most FA_SHADOW_SINK_MAX + FA_SHADOW_WIN_MAX keys) and the same
// for all heads of a GQA group. A work item folds one query row's shadow keys
// (intersected with its key set) into a softmax partial {m, l, acc} in the
// decode kernel's conventions (scores in base-2 units, acc unnormalised); the
// decode partial kernel runs these items as its first work-groups and its
// combine merges them. One single-wave work-group per (query, kv head, chunk
// group): QK with one candidate key per lane (its fp16 row against the G q
// rows in LDS), online softmax across 64-key chunks, PV with output dims on
// lanes. (Prefill folds the shadow keys on its MFMA path instead, in the
// prefill kernel's shadow mode.)
#pragma once

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

__device__ __forceinline__ float shadow_wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float shadow_wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ float shadow_h2f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

// Work item `wi` (= (query * n_kv + kv head) * chunk_groups + chunk group).
// LDS scratch of the calling work-group: Qs >= G*HD floats (16-byte
// aligned), Ps >= G*64 floats, Rs >= 64 ints (the V row of each chunk key:
// sink row, kShadowSinkMax + ring row, or -1).
template <int HD, int G>
__device__ __forceinline__ void shadow_pass_wave(const ShadowPassArgs &a, int wi, float *Qs,
                                                 float *Ps, int *Rs) {
    constexpr int NDL = HD / 64;   // output dims per lane in PV
    const int lane = threadIdx.x;
    const int ncg = a.chunk_groups;
    const int item = wi / ncg, cg = wi % ncg;
    const int i = item / a.n_kv, kvh = item % a.n_kv;
    const int p = a.d_pos ? a.d_pos[i] : a.pos0 + i;
    const bool p_ok = p >= 0 && p < a.max_seq;
    const int slot = a.d_pos ? i : 0;
    const ShadowArgs &sh = a.sh;
    const size_t hkv = (size_t)slot * a.n_kv + kvh;
    const uint16_t *ksink = sh.k_sink + hkv * kShadowSinkMax * HD;
    const uint16_t *vsink = sh.v_sink + hkv * kShadowSinkMax * HD;
    const uint16_t *kwin = sh.k_win + hkv * kShadowWinMax * HD;
    const uint16_t *vwin = sh.v_win + hkv * kShadowWinMax * HD;
    const int *wpos = sh.win_pos + (size_t)slot * kShadowWinMax;

    // candidates: sink positions [0, nsink), then window positions [wlo, p]
    const int nsink = p_ok ? min(sh.sink, p + 1) : 0;
    const int wlo = max(max(p - sh.win + 1, sh.sink), 0);
    const int nwin = (p_ok && sh.win > 0) ? max(0, p - wlo + 1) : 0;
    const int ncand = nsink + nwin;
    const int nchunk = (ncand + 63) / 64;
    const int c_lo = cg * a.chunks_per_group;
    const int c_hi = min(nchunk, c_lo + a.chunks_per_group);

    // q rows of the group, pre-scaled to base-2 scores
    for (int e = lane; e < G * HD; e += 64)
        Qs[e] = a.q[((size_t)i * a.n_head + kvh * G) * HD + e] * a.qscale;
    __syncthreads();

    float m[G], l[G], acc[G][NDL];
#pragma unroll
    for (int g = 0; g < G; g++) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int d = 0; d < NDL; d++) acc[g][d] = 0.0f;
    }

    for (int c = c_lo; c < c_hi; c++) {
        const int cand = c * 64 + lane;
        const bool in_sink = cand < nsink;
        const int s = in_sink ? cand : wlo + (cand - nsink);
        bool ok = cand < ncand && in_key_set(s, p, a.sink, a.win);
        if (ok && !in_sink) ok = wpos[s % kShadowWinMax] == s;
        const int row = ok ? (in_sink ? s : kShadowSinkMax + s % kShadowWinMax) : -1;
        // a lane without a key reads row 0 of a buffer that exists (its
        // scores are discarded)
        const uint16_t *kr = row < 0 ? (sh.sink > 0 ? ksink : kwin)
                                     : (in_sink ? ksink + (size_t)s * HD
                                                : kwin + (size_t)(s % kShadowWinMax) * HD);

        // QK: this lane's key against the G q rows
        float sc[G];
#pragma unroll
        for (int g = 0; g < G; g++) sc[g] = 0.0f;
        // unrolled so that several 16-byte loads of the row are in flight
#pragma unroll 8
        for (int e8 = 0; e8 < HD / 8; e8++) {
            const u32x4 w = ((const u32x4 *)kr)[e8];
            float kv[8];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                kv[2 * t] = shadow_h2f(w[t]);
                kv[2 * t + 1] = shadow_h2f(w[t] >> 16);
            }
#pragma unroll
            for (int g = 0; g < G; g++) {
                const f32x4 q0 = *(const f32x4 *)&Qs[g * HD + 8 * e8];
                const f32x4 q1 = *(const f32x4 *)&Qs[g * HD + 8 * e8 + 4];
                sc[g] += q0[0] * kv[0] + q0[1] * kv[1] + q0[2] * kv[2] + q0[3] * kv[3] +
                         q1[0] * kv[4] + q1[1] * kv[5] + q1[2] * kv[6] + q1[3] * kv[7];
            }
        }

        // online softmax per head (the chunk max is wave-wide)
#pragma unroll
        for (int g = 0; g < G; g++) {
            const float s_g = ok ? sc[g] : -INFINITY;
            const float m_new = fmaxf(m[g], shadow_wave_max(s_g));
            const float corr = m_new == -INFINITY ? 1.0f : fast_exp2(m[g] - m_new);
            const float pg = m_new == -INFINITY ? 0.0f : fast_exp2(s_g - m_new);
            l[g] = l[g] * corr + pg;
#pragma unroll
            for (int d = 0; d < NDL; d++) acc[g][d] *= corr;
            m[g] = m_new;
            Ps[g * 64 + lane] = pg;
        }
        Rs[lane] = row;
        __syncthreads();

        // PV: output dims lane*NDL .. lane*NDL+NDL-1. Unrolled so that several
        // rows' loads are in flight; a key without a row reads row 0 of an
        // existing buffer and is zeroed after the load.
        const int jn = min(64, ncand - c * 64);
#pragma unroll 8
        for (int j = 0; j < jn; j++) {
            const int r = Rs[j];
            const uint16_t *vr = r < 0 ? (sh.sink > 0 ? vsink : vwin)
                                       : (r < kShadowSinkMax ? vsink + (size_t)r * HD
                                                             : vwin + (size_t)(r - kShadowSinkMax) * HD);
            float vv[NDL];
            if constexpr (NDL == 4) {
                const u32x2 w = *(const u32x2 *)(vr + 4 * lane);
                vv[0] = shadow_h2f(w[0]);
                vv[1] = shadow_h2f(w[0] >> 16);
                vv[2] = shadow_h2f(w[1]);
                vv[3] = shadow_h2f(w[1] >> 16);
            } else if constexpr (NDL == 2) {
                const uint32_t w = *(const uint32_t *)(vr + 2 * lane);
                vv[0] = shadow_h2f(w);
                vv[1] = shadow_h2f(w >> 16);
            } else {
                vv[0] = shadow_h2f(vr[lane]);
            }
            if (r < 0) {
#pragma unroll
                for (int d = 0; d < NDL; d++) vv[d] = 0.0f;
            }
#pragma unroll
            for (int g = 0; g < G; g++) {
                const float pg = Ps[g * 64 + j];
#pragma unroll
                for (int d = 0; d < NDL; d++) acc[g][d] = fmaf(pg, vv[d], acc[g][d]);
            }
        }
        __syncthreads();
    }

    // partial of each head: row (item * ncg + cg) * G + g
#pragma unroll
    for (int g = 0; g < G; g++) {
        const size_t r = ((size_t)item * ncg + cg) * G + g;
        const float lt = shadow_wave_sum(l[g]);
        if (lane == 0) {
            a.m_out[r] = m[g];
            a.l_out[r] = lt;
        }
#pragma unroll
        for (int d = 0; d < NDL; d++) a.acc_out[r * HD + lane * NDL + d] = acc[g][d];
    }
}


}  // namespace fa
