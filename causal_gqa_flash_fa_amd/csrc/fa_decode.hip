// Multi-slot split-KV decode on fp32 MFMA (gfx950): a partial pass over
// (split, kv head, slot) and a combine pass over (slot, head).
//
// Method ([FA] "Decode-mode flash attention", fc_attn_dec_plan and the
// "Multi-user decode attention" section): each slot's keys [0, pos] are cut
// into splits by a plan computed from that slot's own position; each split
// folds its tiles into a partial {running max m, running sum l, unnormalised
// accumulator acc}; splits past a slot's plan write empty partials
// (m = -inf, l = 0, acc = 0); the combine rescales every partial by
// exp(m_s - M) and divides, splits in ascending order.
//
// MI355X layout of the work: with one query row per slot the GQA group has
// only G (<= 8) rows, far too few for 32x32 or 16x16 MFMA tiles. This kernel
// uses v_mfma_f32_4x4x1f32 (16 blocks of 4x4x1, same 64 FLOP/clk/SIMD rate)
// with the keys spread across the 16 blocks:
//   * QK: lane = key (64 keys per wave tile). Every block receives the same
//     4 q-head values (A, from LDS, broadcast) and its 4 keys' K values (B,
//     decoded in registers), so one instruction scores 64 keys x 4 heads for
//     one contraction element and all G heads reuse each decoded K element.
//   * PV: lane = output dims. Every block receives the same 4 heads'
//     probabilities for one key (A, from a per-wave LDS copy of P) and 4 of
//     that key's V values (B), so one instruction adds one key's V row into
//     64 dims x 4 heads.
// Both contractions keep every MFMA row busy. The 4 waves of a work-group
// take interleaved 64-key tiles of the split, keep independent (m, l, acc)
// and merge them through LDS before writing the split's partial.
// Scores are kept in base-2 units (q pre-scaled by scale*log2 e), so the
// partial m is log2-scaled and the combine uses exp2.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <int HD, int G, int FMT>
struct DecodeShape {
    static constexpr int W = kDecodeWaves;
    static constexpr int BKD = kDecodeKeyTile;   // keys per wave tile (one per lane)
    static constexpr int NHG = (G + 3) / 4;      // groups of 4 q heads
    static constexpr int HP = NHG * 4;           // padded head count
    static constexpr int VPL = HD / 64;          // V values (output dims) per lane
    static constexpr int NB = HD / kQ4Block;
    static constexpr int RB = FMT == 0 ? HD * 4 : NB * kQ4BlockBytes;
};

// Output dim held by `lane` for its c-th PV accumulator. fp32 rows: plain
// stride 64. Q4_0 rows: the dims a lane owns share one or two code bytes of
// one block, so its V values come from a single 2-byte (or 1-byte) read.
template <int HD, int FMT>
__device__ __forceinline__ int pv_dim(int lane, int c) {
    if constexpr (FMT == 0) {
        return lane + 64 * c;
    } else if constexpr (HD == 256) {
        const int bb = lane >> 3, jj = 2 * (lane & 7);
        const int off[4] = {0, 1, 16, 17};
        return 32 * bb + jj + off[c];
    } else if constexpr (HD == 128) {
        return 32 * (lane >> 4) + (lane & 15) + 16 * c;
    } else {
        return lane;
    }
}

template <int HD, int G, int FMT>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
    using Sh = DecodeShape<HD, G, FMT>;
    constexpr int W = Sh::W, BKD = Sh::BKD, NHG = Sh::NHG, HP = Sh::HP, VPL = Sh::VPL;
    constexpr int NB = Sh::NB, RB = Sh::RB;
    __shared__ float Qs[HP * HD];
    __shared__ float Ps[W][HP * BKD];
    __shared__ float Om[W][HP * HD];
    __shared__ float Mm[W][HP], Lm[W][HP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int split0 = blockIdx.x;
    const int S = gridDim.x;
    const int kvh = blockIdx.y;
    const int slot = blockIdx.z;

    const int pos = a.pos[slot];
    const bool bad = pos < 0 || pos >= a.max_seq;
    const int L = pos + 1;

    for (int idx = tid; idx < HP * HD; idx += 256) {
        const int hr = idx / HD, e = idx % HD;
        Qs[idx] = hr < G ? a.q[((size_t)slot * a.n_head + kvh * G + hr) * HD + e] * a.qscale
                         : 0.0f;
    }
    __syncthreads();

    float m[HP], l[HP];
    f32x4 O[VPL][NHG];
#pragma unroll
    for (int h = 0; h < HP; h++) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < VPL; c++)
#pragma unroll
        for (int hg = 0; hg < NHG; hg++) O[c][hg] = f32x4{};

    unsigned vis = 0, skp = 0;
    const size_t head_rows = ((size_t)slot * a.n_kv + kvh) * a.max_seq;
    const uint8_t *kb = (const uint8_t *)a.k + head_rows * RB;
    const uint8_t *vb = (const uint8_t *)a.v + head_rows * RB;
    float *Pw = Ps[w];

    auto tile = [&](int j0, int k_hi) {
        const int key = j0 + lane;
        const bool kval = key < k_hi && in_key_set(key, pos, a.sink, a.win);
        const int krow = min(key, k_hi - 1);        // never read past the live rows
        f32x4 sacc[NHG];
#pragma unroll
        for (int hg = 0; hg < NHG; hg++) sacc[hg] = f32x4{};
        const float *qlane = Qs + (lane & 3) * HD;

        if constexpr (FMT == 0) {
            const f32x4 *kr = (const f32x4 *)(kb + (size_t)krow * RB);
#pragma unroll 8
            for (int c4 = 0; c4 < HD / 4; c4++) {
                const f32x4 kv = kr[c4];
#pragma unroll
                for (int hg = 0; hg < NHG; hg++) {
                    const f32x4 qv = *(const f32x4 *)(qlane + hg * 4 * HD + 4 * c4);
#pragma unroll
                    for (int t = 0; t < 4; t++) sacc[hg] = mfma4(qv[t], kv[t], sacc[hg]);
                }
            }
        } else {
            // this lane's whole Q4 row as dwords (row starts are 4-byte aligned)
            uint32_t rw[RB / 4];
            const uint8_t *kr = kb + (size_t)krow * RB;
            if constexpr (RB % 16 == 0) {
#pragma unroll
                for (int i = 0; i < RB / 16; i++) {
                    const u32x4 v = ((const u32x4 *)kr)[i];
                    rw[4 * i] = v[0]; rw[4 * i + 1] = v[1]; rw[4 * i + 2] = v[2]; rw[4 * i + 3] = v[3];
                }
            } else if constexpr (RB % 8 == 0) {
#pragma unroll
                for (int i = 0; i < RB / 8; i++) {
                    const u32x2 v = ((const u32x2 *)kr)[i];
                    rw[2 * i] = v[0]; rw[2 * i + 1] = v[1];
                }
            } else {
#pragma unroll
                for (int i = 0; i < RB / 4; i++) rw[i] = ((const uint32_t *)kr)[i];
            }
#pragma unroll
            for (int blk = 0; blk < NB; blk++) {
                const int o = blk * kQ4BlockBytes;     // compile-time after unrolling
                const int dw = o / 4;
                const bool odd = (blk & 1) != 0;       // odd blocks start 2 bytes into a dword
                const uint32_t sbits = odd ? (rw[dw] >> 16) : (rw[dw] & 0xffffu);
                const float d = half_bits_to_float(sbits);
                const float m8d = -8.0f * d;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const uint32_t cw = odd ? rw[dw + 1 + q]
                                            : ((rw[dw + q] >> 16) | (rw[dw + q + 1] << 16));
                    const float lo[4] = {fmaf(nib(cw, 0), d, m8d), fmaf(nib(cw, 8), d, m8d),
                                         fmaf(nib(cw, 16), d, m8d), fmaf(nib(cw, 24), d, m8d)};
                    const float hi[4] = {fmaf(nib(cw, 4), d, m8d), fmaf(nib(cw, 12), d, m8d),
                                         fmaf(nib(cw, 20), d, m8d), fmaf(nib(cw, 28), d, m8d)};
#pragma unroll
                    for (int hg = 0; hg < NHG; hg++) {
                        const float *qb = qlane + hg * 4 * HD + blk * kQ4Block;
                        const f32x4 qa = *(const f32x4 *)(qb + 4 * q);
                        const f32x4 qh = *(const f32x4 *)(qb + 16 + 4 * q);
#pragma unroll
                        for (int t = 0; t < 4; t++) {
                            sacc[hg] = mfma4(qa[t], lo[t], sacc[hg]);
                            sacc[hg] = mfma4(qh[t], hi[t], sacc[hg]);
                        }
                    }
                }
            }
        }

        // online softmax per head; lane = key, register = head within group
        float corr[HP];
        bool moved = false;
#pragma unroll
        for (int hg = 0; hg < NHG; hg++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int h = 4 * hg + i;
                const float s = kval ? sacc[hg][i] : -INFINITY;
                const float tmax = wave_max(s);
                const float m_new = fmaxf(m[h], tmax);
                const float m_use = m_new == -INFINITY ? 0.0f : m_new;
                corr[h] = fast_exp2(m[h] - m_use);
                moved |= m_new > m[h];
                m[h] = m_new;
                const float p = fast_exp2(s - m_use);
                l[h] = l[h] * corr[h] + p;
                Pw[h * BKD + lane] = p;
            }
        }
        if (moved) {
#pragma unroll
            for (int c = 0; c < VPL; c++)
#pragma unroll
                for (int hg = 0; hg < NHG; hg++)
#pragma unroll
                    for (int i = 0; i < 4; i++) O[c][hg][i] *= corr[4 * hg + i];
        }
        wave_lds_sync();

        // PV: one key per contraction step, lanes over output dims
        const float *plane = Pw + (lane & 3) * BKD;
#pragma unroll 2
        for (int k4 = 0; k4 < BKD / 4; k4++) {
            f32x4 pa[NHG];
#pragma unroll
            for (int hg = 0; hg < NHG; hg++) pa[hg] = *(const f32x4 *)(plane + hg * 4 * BKD + 4 * k4);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int vrow = min(j0 + 4 * k4 + t, k_hi - 1);
                float vv[VPL];
                if constexpr (FMT == 0) {
                    const float *vr = (const float *)(vb + (size_t)vrow * RB);
#pragma unroll
                    for (int c = 0; c < VPL; c++) vv[c] = vr[lane + 64 * c];
                } else {
                    const uint8_t *vr = vb + (size_t)vrow * RB;
                    if constexpr (HD == 256) {
                        const int bb = lane >> 3, jj = 2 * (lane & 7);
                        const float d = half_bits_to_float(*(const uint16_t *)(vr + bb * kQ4BlockBytes));
                        const uint32_t cw = *(const uint16_t *)(vr + bb * kQ4BlockBytes + 2 + jj);
                        const float m8d = -8.0f * d;
                        vv[0] = fmaf(nib(cw, 0), d, m8d);    // element jj
                        vv[1] = fmaf(nib(cw, 8), d, m8d);    // element jj+1
                        vv[2] = fmaf(nib(cw, 4), d, m8d);    // element jj+16
                        vv[3] = fmaf(nib(cw, 12), d, m8d);   // element jj+17
                    } else if constexpr (HD == 128) {
                        const int bb = lane >> 4, jj = lane & 15;
                        const float d = half_bits_to_float(*(const uint16_t *)(vr + bb * kQ4BlockBytes));
                        const uint32_t cb = vr[bb * kQ4BlockBytes + 2 + jj];
                        const float m8d = -8.0f * d;
                        vv[0] = fmaf(nib(cb, 0), d, m8d);
                        vv[1] = fmaf(nib(cb, 4), d, m8d);
                    } else {
                        const int bb = lane >> 5, e = lane & 31;
                        const float d = half_bits_to_float(*(const uint16_t *)(vr + bb * kQ4BlockBytes));
                        const uint32_t cb = vr[bb * kQ4BlockBytes + 2 + (e & 15)];
                        vv[0] = fmaf(nib(cb, e < 16 ? 0 : 4), d, -8.0f * d);
                    }
                }
#pragma unroll
                for (int c = 0; c < VPL; c++)
#pragma unroll
                    for (int hg = 0; hg < NHG; hg++) O[c][hg] = mfma4(pa[hg][t], vv[c], O[c][hg]);
            }
        }
        wave_lds_sync();          // P of this tile consumed before the next overwrites it
    };

    if (!bad) {
        int n_splits, split_len;
        const int live = decode_plan(L, a.kps, a.cap, BKD, &n_splits, &split_len);
        for (int sp = split0; sp < live; sp += S) {
            const int k_lo = sp * split_len;
            const int k_hi = min(L, k_lo + split_len);
            for (int j0 = k_lo + BKD * w; j0 < k_hi; j0 += BKD * W) {
                const int e = min(j0 + BKD - 1, k_hi - 1);
                if (a.win > 0 && j0 >= a.sink && e < pos - a.win + 1) {
                    skp++;
                    continue;
                }
                vis++;
                tile(j0, k_hi);
            }
        }
    }

    // ---- merge the 4 waves' states, then write this split's partial
#pragma unroll
    for (int h = 0; h < HP; h++) l[h] = wave_sum(l[h]);
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < HP; h++) {
            Mm[w][h] = m[h];
            Lm[w][h] = l[h];
        }
    }
#pragma unroll
    for (int c = 0; c < VPL; c++)
#pragma unroll
        for (int hg = 0; hg < NHG; hg++)
#pragma unroll
            for (int i = 0; i < 4; i++) Om[w][(4 * hg + i) * HD + pv_dim<HD, FMT>(lane, c)] = O[c][hg][i];
    __syncthreads();

    for (int idx = tid; idx < G * HD; idx += 256) {
        const int h = idx / HD, dd = idx % HD;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < W; ww++) M = fmaxf(M, Mm[ww][h]);
        float o = 0.0f, lsum = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < W; ww++) {
                const float sc = fast_exp2(Mm[ww][h] - M);
                o += Om[ww][h * HD + dd] * sc;
                lsum += Lm[ww][h] * sc;
            }
        }
        const size_t pidx = ((size_t)slot * a.n_head + kvh * G + h) * S + split0;
        a.ws_acc[pidx * HD + dd] = o;
        if (dd == 0) {
            a.ws_m[pidx] = M;
            a.ws_l[pidx] = lsum;
        }
    }
    if (a.stats && lane == 0) {
        atomicAdd(&a.stats[0], (unsigned long long)vis);
        atomicAdd(&a.stats[1], (unsigned long long)skp);
    }
}

// out = sum_s exp2(m_s - M) acc_s / sum_s exp2(m_s - M) l_s, ascending s.
template <int HD>
__global__ __launch_bounds__(HD) void decode_combine_kernel(DecodeArgs a, int S) {
    const size_t gh = blockIdx.x;           // slot * n_head + head
    const int dd = threadIdx.x;
    const float *mm = a.ws_m + gh * S;
    const float *ll = a.ws_l + gh * S;
    const float *acc = a.ws_acc + gh * S * HD;
    float M = -INFINITY;
    for (int s = 0; s < S; s++) M = fmaxf(M, mm[s]);
    float o = 0.0f, L = 0.0f;
    for (int s = 0; s < S; s++) {
        const float wgt = fast_exp2(mm[s] - M);
        L += ll[s] * wgt;
        o += acc[(size_t)s * HD + dd] * wgt;
    }
    a.out[gh * HD + dd] = o / L;
}

template <int HD, int G, int FMT>
hipError_t launch_one(const DecodeArgs &a, int n_slots, int splits, hipStream_t s) {
    hipLaunchKernelGGL((decode_partial_kernel<HD, G, FMT>), dim3(splits, a.n_kv, n_slots),
                       dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel<HD>, dim3(n_slots * a.n_head), dim3(HD), 0, s, a,
                       splits);
    return hipGetLastError();
}

template <int HD, int FMT>
hipError_t by_group(int group, const DecodeArgs &a, int n_slots, int splits, hipStream_t s) {
    switch (group) {
    case 1: return launch_one<HD, 1, FMT>(a, n_slots, splits, s);
    case 2: return launch_one<HD, 2, FMT>(a, n_slots, splits, s);
    case 4: return launch_one<HD, 4, FMT>(a, n_slots, splits, s);
    case 8: return launch_one<HD, 8, FMT>(a, n_slots, splits, s);
    }
    return hipErrorInvalidValue;
}

template <int FMT>
hipError_t by_dim(int head_dim, int group, const DecodeArgs &a, int n_slots, int splits,
                  hipStream_t s) {
    switch (head_dim) {
    case 64: return by_group<64, FMT>(group, a, n_slots, splits, s);
    case 128: return by_group<128, FMT>(group, a, n_slots, splits, s);
    case 256: return by_group<256, FMT>(group, a, n_slots, splits, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(int format, int head_dim, int group, const DecodeArgs &a, int n_slots,
                         int launch_splits, hipStream_t s) {
    return format == 0 ? by_dim<0>(head_dim, group, a, n_slots, launch_splits, s)
                       : by_dim<1>(head_dim, group, a, n_slots, launch_splits, s);
}

}  // namespace fa
