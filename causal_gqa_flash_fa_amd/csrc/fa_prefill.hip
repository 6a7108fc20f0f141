// Causal GQA flash-attention prefill on fp32 MFMA (gfx950).
//
// Method ([FA] file header and fc_attn_flash_prefill): key tiles are folded
// into a running max m, running sum l and an unnormalised accumulator, so the
// score matrix never exists; the K/V tile is loaded once and serves every q
// head of the GQA group; tiles outside the sink U recent-window key set are
// skipped before any load or barrier ([FA] fc_attn_tile_in_window).
//
// MI355X layout of the work:
//   * A work-group of 4 waves owns BQ = 128/G consecutive query positions of
//     one kv head; each wave owns 32 (position, head) rows, row R -> position
//     q0 + R/G, head kvh*G + R%G. One 32-key K tile and V tile (fp32, padded
//     rows) sit in LDS and are shared by all 128 rows of the group.
//   * S^T = K Q^T with v_mfma_f32_32x32x2_f32: K rows come from LDS, Q^T is
//     held in registers (pre-scaled by scale*log2 e). The accumulator puts
//     one query row per lane (lane&31) and 16 keys per lane, so the softmax
//     needs one cross-lane step (lane ^ 32) per tile.
//   * O^T = V^T P^T, also 32x32x2: P^T is exactly the S^T accumulator after
//     the exponentials (the key order of the contraction is chosen to match
//     the accumulator layout), V^T comes from LDS with 16-byte reads, and O^T
//     keeps one query row per lane, so the rescale by exp(m_old - m_new) is a
//     per-lane multiply, done only when some row's max moved.
//   * Q4_0 tiles are loaded as raw 18-byte blocks and decoded exactly
//     ((c-8)*d) while being written to the fp32 LDS tile.
//   * Heavy (late) query blocks are dispatched first. The next tile's global
//     loads are issued into registers before the current tile is computed.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

template <int HD, int G, int FMT>
struct PrefillShape {
    static constexpr int W = kPrefillWaves;
    static constexpr int R = kPrefillRowsPerWave;
    static constexpr int BK = kPrefillKeyTile;
    static constexpr int BQ = W * R / G;        // query positions per work-group
    static constexpr int PW = R / G;            // query positions per wave
    static constexpr int KS = HD + 4;           // LDS row stride (floats): conflict-free 16-B reads
    static constexpr int NT = HD / 32;          // 32-wide output tiles of O^T
    static constexpr int GS = NT < 4 ? NT : 4;  // output tiles fed by one V read
    static constexpr int HH = HD / 2;           // contraction elements per lane half
    static constexpr int NB = HD / kQ4Block;    // Q4 blocks per row
    static constexpr int RB = FMT == 0 ? HD * 4 : NB * kQ4BlockBytes;
    static constexpr int NC = BK * HD / 4 / 256;                       // fp32 float4 per thread per tensor
    static constexpr int QITEMS = 2 * BK * NB;                         // Q4 (row, block) items, K and V
    static constexpr int IPT = (QITEMS + 255) / 256;                   // Q4 items per thread
    static constexpr size_t LDS_BYTES = (size_t)2 * BK * KS * sizeof(float);
};

template <int HD, int G, int FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(PrefillArgs a) {
    using Sh = PrefillShape<HD, G, FMT>;
    constexpr int BK = Sh::BK, KS = Sh::KS, NT = Sh::NT, GS = Sh::GS, HH = Sh::HH;
    constexpr int NB = Sh::NB, RB = Sh::RB;
    extern __shared__ float lds[];
    float *Ks = lds;
    float *Vs = lds + BK * KS;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hlf = lane >> 5;        // which half of the contraction / key sub-block
    const int r32 = lane & 31;        // this lane's query row within the wave

    const int bid = blockIdx.x;
    const int qb = a.n_qblocks - 1 - bid / a.n_kv;   // heavy blocks first
    const int kvh = bid % a.n_kv;
    const int q0 = a.pos0 + qb * Sh::BQ;
    const int q1 = min(q0 + Sh::BQ - 1, a.pos0 + a.n - 1);

    const int row_wg = w * Sh::R + r32;
    const int p_row = q0 + row_wg / G;
    const int g = row_wg % G;
    const bool row_live = p_row <= q1;
    const int pw0 = q0 + w * Sh::PW;
    const int pw1 = min(pw0 + Sh::PW - 1, q1);
    const bool wave_live = pw0 <= q1;

    const uint8_t *kbase = (const uint8_t *)a.k + (size_t)kvh * a.max_seq * RB;
    const uint8_t *vbase = (const uint8_t *)a.v + (size_t)kvh * a.max_seq * RB;

    // Q^T operand: this lane's row, contraction half hlf, pre-scaled.
    float qr[HH];
    if (row_live) {
        const f32x4 *qp = (const f32x4 *)(a.q + ((size_t)(p_row - a.pos0) * a.n_head +
                                                 kvh * G + g) * HD + hlf * HH);
#pragma unroll
        for (int i = 0; i < HH / 4; i++) {
            const f32x4 v = qp[i];
#pragma unroll
            for (int t = 0; t < 4; t++) qr[4 * i + t] = v[t] * a.qscale;
        }
    } else {
#pragma unroll
        for (int i = 0; i < HH; i++) qr[i] = 0.0f;
    }

    f32x16 O[NT];
#pragma unroll
    for (int n = 0; n < NT; n++) O[n] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;

    // ---- tile walk ([FA] fc_attn_tile_in_window over the block's rows)
    unsigned visited = 0, skipped = 0;
    const int win_lo = q0 - a.win + 1;    // first key of the union of the rows' windows
    auto first_visited = [&](int j0) -> int {
        if (j0 <= q1 && a.win > 0 && j0 >= a.sink && j0 + BK - 1 < win_lo) {
            const int jn = (win_lo / BK) * BK;
            skipped += (unsigned)((jn - j0) / BK);
            return jn;
        }
        return j0;
    };

    // ---- staging registers for the next tile
    f32x4 pk[FMT == 0 ? Sh::NC : 1], pv[FMT == 0 ? Sh::NC : 1];
    uint32_t raw[FMT == 0 ? 1 : Sh::IPT][9];

    auto load_tile = [&](int j0) {
        if constexpr (FMT == 0) {
#pragma unroll
            for (int i = 0; i < Sh::NC; i++) {
                const int c = tid + 256 * i;
                const int row = c / (HD / 4), c4 = c % (HD / 4);
                if (j0 + row <= q1) {
                    const size_t off = (size_t)(j0 + row) * HD + 4 * c4;
                    pk[i] = *(const f32x4 *)((const float *)kbase + off);
                    pv[i] = *(const f32x4 *)((const float *)vbase + off);
                } else {
                    pk[i] = f32x4{};
                    pv[i] = f32x4{};
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < Sh::IPT; i++) {
                const int idx = tid + 256 * i;
                const int rem = idx % (BK * NB);
                const int row = rem / NB, blk = rem % NB;
                const uint8_t *base = idx < BK * NB ? kbase : vbase;
                if (idx < Sh::QITEMS && j0 + row <= q1) {
                    const uint16_t *src =
                        (const uint16_t *)(base + (size_t)(j0 + row) * RB + blk * kQ4BlockBytes);
#pragma unroll
                    for (int u = 0; u < 9; u++) raw[i][u] = src[u];
                } else {
#pragma unroll
                    for (int u = 0; u < 9; u++) raw[i][u] = 0;
                }
            }
        }
    };

    auto store_tile = [&]() {
        if constexpr (FMT == 0) {
#pragma unroll
            for (int i = 0; i < Sh::NC; i++) {
                const int c = tid + 256 * i;
                const int row = c / (HD / 4), c4 = c % (HD / 4);
                *(f32x4 *)&Ks[row * KS + 4 * c4] = pk[i];
                *(f32x4 *)&Vs[row * KS + 4 * c4] = pv[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < Sh::IPT; i++) {
                const int idx = tid + 256 * i;
                if (idx < Sh::QITEMS) {
                    const int rem = idx % (BK * NB);
                    const int row = rem / NB, blk = rem % NB;
                    float *dst = (idx < BK * NB ? Ks : Vs) + row * KS + blk * kQ4Block;
                    const float d = half_bits_to_float(raw[i][0]);
                    const float m8d = -8.0f * d;
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const uint32_t cw = raw[i][1 + 2 * q] | (raw[i][2 + 2 * q] << 16);
                        // (c - 8) * d == c*d - 8d exactly: c*d has <= 15 significant bits
                        const f32x4 lo = {fmaf(nib(cw, 0), d, m8d), fmaf(nib(cw, 8), d, m8d),
                                          fmaf(nib(cw, 16), d, m8d), fmaf(nib(cw, 24), d, m8d)};
                        const f32x4 hi = {fmaf(nib(cw, 4), d, m8d), fmaf(nib(cw, 12), d, m8d),
                                          fmaf(nib(cw, 20), d, m8d), fmaf(nib(cw, 28), d, m8d)};
                        *(f32x4 *)&dst[4 * q] = lo;
                        *(f32x4 *)&dst[16 + 4 * q] = hi;
                    }
                }
            }
        }
    };

    auto compute_tile = [&](int jc) {
        // S^T = K Q^T: lane holds row r32, keys 8*(r/4) + 4*hlf + r%4
        f32x16 s = f32x16{};
        const float *krow = Ks + r32 * KS + hlf * HH;
#pragma unroll
        for (int i = 0; i < HH / 4; i++) {
            const f32x4 kv = *(const f32x4 *)(krow + 4 * i);
#pragma unroll
            for (int t = 0; t < 4; t++) s = mfma32(kv[t], qr[4 * i + t], s);
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int key = jc + 8 * (r >> 2) + 4 * hlf + (r & 3);
            const bool ok = row_live && in_key_set(key, p_row, a.sink, a.win);
            s[r] = ok ? s[r] : -INFINITY;
            tmax = fmaxf(tmax, s[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;   // all-masked row: keep p = 0
        const float corr = fast_exp2(m_run - m_use);
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            s[r] = fast_exp2(s[r] - m_use);
            psum += s[r];
        }
        l_run = l_run * corr + psum;
        if (__ballot(m_new > m_run)) {
#pragma unroll
            for (int n = 0; n < NT; n++) O[n] *= corr;
        }
        m_run = m_new;

        // O^T += V^T P^T: contraction step kk covers keys 8*(kk/4) + 4*hlf + kk%4
#pragma unroll
        for (int kk = 0; kk < 16; kk++) {
            const int key = 8 * (kk >> 2) + 4 * hlf + (kk & 3);
            const float *vrow = Vs + key * KS + GS * r32;
#pragma unroll
            for (int ng = 0; ng < NT / GS; ng++) {
                if constexpr (GS == 4) {
                    const f32x4 vv = *(const f32x4 *)(vrow + ng * 32 * GS);
#pragma unroll
                    for (int u = 0; u < 4; u++) O[ng * 4 + u] = mfma32(vv[u], s[kk], O[ng * 4 + u]);
                } else {
                    const f32x2 vv = *(const f32x2 *)(vrow + ng * 32 * GS);
#pragma unroll
                    for (int u = 0; u < 2; u++) O[ng * 2 + u] = mfma32(vv[u], s[kk], O[ng * 2 + u]);
                }
            }
        }
    };

    int j0 = first_visited(0);
    if (j0 <= q1) load_tile(j0);
    while (j0 <= q1) {
        __syncthreads();          // previous tile fully consumed
        store_tile();
        __syncthreads();
        const int jc = j0;
        visited++;
        j0 = first_visited(jc + BK);
        if (j0 <= q1) load_tile(j0);
        const bool wave_do = wave_live && jc <= pw1 &&
                             (a.win <= 0 || jc < a.sink || jc + BK - 1 >= pw0 - a.win + 1);
        if (wave_do) compute_tile(jc);
    }

    // ---- finalise: out = acc / l, scattered back through the d permutation
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (row_live) {
        const float inv = 1.0f / l_tot;
        float *op = a.out + ((size_t)(p_row - a.pos0) * a.n_head + kvh * G + g) * HD;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int mi = 8 * (r >> 2) + 4 * hlf + (r & 3);
#pragma unroll
            for (int ng = 0; ng < NT / GS; ng++) {
                float *dst = op + ng * 32 * GS + GS * mi;
                if constexpr (GS == 4) {
                    *(f32x4 *)dst = f32x4{O[ng * 4 + 0][r], O[ng * 4 + 1][r], O[ng * 4 + 2][r],
                                          O[ng * 4 + 3][r]} * inv;
                } else {
                    *(f32x2 *)dst = f32x2{O[ng * 2 + 0][r], O[ng * 2 + 1][r]} * inv;
                }
            }
        }
    }
    if (a.stats && tid == 0) {
        atomicAdd(&a.stats[0], (unsigned long long)visited);
        atomicAdd(&a.stats[1], (unsigned long long)skipped);
    }
}

template <int HD, int G, int FMT>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s) {
    using Sh = PrefillShape<HD, G, FMT>;
    static bool attr_set = false;   // per process; the attribute is per function
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)prefill_kernel<HD, G, FMT>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)Sh::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const dim3 grid((unsigned)(a.n_qblocks * a.n_kv));
    hipLaunchKernelGGL((prefill_kernel<HD, G, FMT>), grid, dim3(256), Sh::LDS_BYTES, s, a);
    return hipGetLastError();
}

template <int HD, int FMT>
hipError_t by_group(int group, const PrefillArgs &a, hipStream_t s) {
    switch (group) {
    case 1: return launch_one<HD, 1, FMT>(a, s);
    case 2: return launch_one<HD, 2, FMT>(a, s);
    case 4: return launch_one<HD, 4, FMT>(a, s);
    case 8: return launch_one<HD, 8, FMT>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int FMT>
hipError_t by_dim(int head_dim, int group, const PrefillArgs &a, hipStream_t s) {
    switch (head_dim) {
    case 64: return by_group<64, FMT>(group, a, s);
    case 128: return by_group<128, FMT>(group, a, s);
    case 256: return by_group<256, FMT>(group, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(int format, int head_dim, int group, const PrefillArgs &a,
                          hipStream_t s) {
    return format == 0 ? by_dim<0>(head_dim, group, a, s) : by_dim<1>(head_dim, group, a, s);
}

}  // namespace fa
