// Attention over the fp16 shadow keys of a Q4_0 cache.
//
// [FA] "fp16 sink + recent-window exemption" (fc_kvq4_is_fp16, the fp16
// sink / window read paths of fc_attn_flash_prefill_q4 and the Q4 decode):
// for a query at position p, key s is read from the fp16 shadow instead of
// the Q4_0 body iff s is a sink position or lies in the recent window of p
// and the window ring still holds it. That key subset is small (at most
// FA_SHADOW_SINK_MAX + FA_SHADOW_WIN_MAX keys per query) and the same for all
// heads of a GQA group, so it is handled here, off the main kernels' paths:
// this pass folds each query row's shadow keys (intersected with its key
// set) into a softmax partial {m, l, acc}, with the main kernels'
// conventions (scores in base-2 units, acc unnormalised). The main kernels
// skip exactly these keys and merge the partial: decode through its combine
// pass, prefill by starting each segment's running state from it.
//
// One single-wave work-group per (query, kv head[, chunk group]): QK with
// one candidate key per lane (its fp16 row against the G q rows in LDS),
// online softmax across 64-key chunks, PV with output dims on lanes.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ float h2f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

template <int HD, int G>
__global__ __launch_bounds__(64) void shadow_pass_kernel(ShadowPassArgs a) {
    constexpr int NDL = HD / 64;   // output dims per lane in PV
    __shared__ __attribute__((aligned(16))) float Qs[G][HD];
    __shared__ float Ps[G][64];
    __shared__ int Rs[64];         // V row of each chunk key: sink row, 8 + ring row, or -1
    const int lane = threadIdx.x;
    const int ncg = a.chunk_groups;
    const int item = blockIdx.x / ncg, cg = blockIdx.x % ncg;
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
        Qs[e / HD][e % HD] = a.q[((size_t)i * a.n_head + kvh * G) * HD + e] * a.qscale;
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
        for (int e8 = 0; e8 < HD / 8; e8++) {
            const u32x4 w = ((const u32x4 *)kr)[e8];
            float kv[8];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                kv[2 * t] = h2f(w[t]);
                kv[2 * t + 1] = h2f(w[t] >> 16);
            }
#pragma unroll
            for (int g = 0; g < G; g++) {
                const f32x4 q0 = *(const f32x4 *)&Qs[g][8 * e8];
                const f32x4 q1 = *(const f32x4 *)&Qs[g][8 * e8 + 4];
                sc[g] += q0[0] * kv[0] + q0[1] * kv[1] + q0[2] * kv[2] + q0[3] * kv[3] +
                         q1[0] * kv[4] + q1[1] * kv[5] + q1[2] * kv[6] + q1[3] * kv[7];
            }
        }

        // online softmax per head (the chunk max is wave-wide)
#pragma unroll
        for (int g = 0; g < G; g++) {
            const float s_g = ok ? sc[g] : -INFINITY;
            const float m_new = fmaxf(m[g], wave_max_f(s_g));
            const float corr = m_new == -INFINITY ? 1.0f : fast_exp2(m[g] - m_new);
            const float pg = m_new == -INFINITY ? 0.0f : fast_exp2(s_g - m_new);
            l[g] = l[g] * corr + pg;
#pragma unroll
            for (int d = 0; d < NDL; d++) acc[g][d] *= corr;
            m[g] = m_new;
            Ps[g][lane] = pg;
        }
        Rs[lane] = row;
        __syncthreads();

        // PV: output dims lane*NDL .. lane*NDL+NDL-1
        const int jn = min(64, ncand - c * 64);
        for (int j = 0; j < jn; j++) {
            const int r = Rs[j];
            if (r < 0) continue;   // the same for every lane
            const uint16_t *vr = r < kShadowSinkMax ? vsink + (size_t)r * HD
                                                    : vwin + (size_t)(r - kShadowSinkMax) * HD;
            float vv[NDL];
            if constexpr (NDL == 4) {
                const u32x2 w = *(const u32x2 *)(vr + 4 * lane);
                vv[0] = h2f(w[0]);
                vv[1] = h2f(w[0] >> 16);
                vv[2] = h2f(w[1]);
                vv[3] = h2f(w[1] >> 16);
            } else if constexpr (NDL == 2) {
                const uint32_t w = *(const uint32_t *)(vr + 2 * lane);
                vv[0] = h2f(w);
                vv[1] = h2f(w >> 16);
            } else {
                vv[0] = h2f(vr[lane]);
            }
#pragma unroll
            for (int g = 0; g < G; g++) {
                const float pg = Ps[g][j];
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
        const float lt = wave_sum_f(l[g]);
        if (lane == 0) {
            a.m_out[r] = m[g];
            a.l_out[r] = lt;
        }
#pragma unroll
        for (int d = 0; d < NDL; d++) a.acc_out[r * HD + lane * NDL + d] = acc[g][d];
    }
}

template <int HD>
hipError_t by_group(int group, const ShadowPassArgs &a, int items, hipStream_t s) {
    const dim3 grid((unsigned)(items * a.chunk_groups));
    switch (group) {
    case 1: hipLaunchKernelGGL((shadow_pass_kernel<HD, 1>), grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((shadow_pass_kernel<HD, 2>), grid, dim3(64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((shadow_pass_kernel<HD, 4>), grid, dim3(64), 0, s, a); break;
    case 8: hipLaunchKernelGGL((shadow_pass_kernel<HD, 8>), grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shadow_pass(int head_dim, int group, const ShadowPassArgs &a, int items,
                              hipStream_t s) {
    switch (head_dim) {
    case 64: return by_group<64>(group, a, items, s);
    case 128: return by_group<128>(group, a, items, s);
    case 256: return by_group<256>(group, a, items, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
