// Multi-slot split-KV decode over a Q4_0 cache on fp16 matrix cores, with
// hi/lo-split fp16 operands that keep close to fp32 accuracy.
//
// Method: the same decode as fa_decode ([FA] "Decode-mode flash attention",
// fc_attn_dec_plan, "Multi-user decode attention (slots)"; the stream-K
// schedule of fa_decode_sched.hpp, the partials {m, l, acc} and the combine
// of fa_decode.hip). Only the two tile contractions change: on gfx950 fp32
// MFMA runs at 1/16 of the fp16 rate, and a Q4_0 decode at G = 8 needs more
// fp32 MFMA time than it takes to read its bytes, while the integer codes of
// a Q4_0 block are exact fp16 values. So the fp32 operands are split into an
// fp16 high part and an fp16 low part (the two-pass hi/lo lane of the
// logicaffeine qwen38_batched.rs page; the Foundry attention.cu page narrows
// staging to fp16 for the same reason) and the contractions run on
// v_mfma_f32_16x16x32_f16 with fp32 accumulation:
//
//   * Codes as operands. A code nibble c masked into the low bits of a
//     binary16 is the subnormal c * 2^-24 (low nibble) or 16 c * 2^-24 (high
//     nibble, bits 4-7): exact, one AND per two codes. The MFMA takes
//     subnormal inputs exactly (checked on the GPU).
//   * QK. S^T[key][row] for 16 keys, rows = (limb, head): limb 0 holds
//     hi(q'), limb 1 lo(q') = q' - hi(q'), where q' = q 2^E per head (a power
//     of two keeps |16 q'| < 2^15). One MFMA covers one 32-element Q4 block,
//     and the block scale d (one per key and block) is applied to its fp32
//     result by one fused multiply-add per output. The -8 of the codes is one
//     more MFMA per 16 keys: each row's per-block sums of q' (hi/lo limbs,
//     scaled by 2^-6) against the keys' block scales, entering the score
//     times -2^-15. The two limb rows of a head are summed once per tile.
//   * PV. O[row][dim] for 16 dims of one block, rows = (limb, head) of
//     p * d * 2^-F (d the block scale of each key, 2^-F a power of two that
//     keeps the product within fp16), contraction over 32 keys, codes as the
//     other operand (a byte-transposed read of the V tile in LDS). The -8 of
//     the codes is sum_j p_j d_j per (head, block): one more MFMA per tile,
//     the limbs of 128 p against the block scales, subtracted at the end.
//   * Every product is exact in fp32 (11-bit by 11-bit significands) and
//     sums are fp32, so the result matches the fp32-input lane to about the
//     same rounding; the low limbs carry the bits fp16 drops.
//
// K and V tiles (32 keys) are DMA'd raw into a two-deep LDS ring
// (buffer_load ... lds): the next tile is requested as a tile starts and
// flies during its QK, softmax and PV. One query row per slot, so the G heads
// of a GQA group (padded to 8) and the two limbs fill the MFMA's 16 rows.
#include "fa_device.hpp"
#include "fa_internal.hpp"
#include "fa_decode_sched.hpp"

namespace fa {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// v_mfma_f32_16x16x32_f16, fp32 accumulate. Lane layout (checked on the
// GPU): A[m][k] in lane 16 (k / 8) + m, element k % 8; B[k][n] in lane
// 16 (k / 8) + n, element k % 8; D[m][n] in lane 16 (m / 4) + n, register m % 4.
__device__ __forceinline__ f32x4 mfma16h(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a),
                                                  __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// two binary16 in one register, lo in bits 0-15 (a vector build lets the
// compiler convert straight into either half)
__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
    return __builtin_bit_cast(uint32_t, h2{lo, hi});
}

// Waits for this wave's outstanding LDS reads (a DMA into a buffer must not
// overtake reads of its previous contents).
__device__ __forceinline__ void wait_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), other counters at their maximum
}

template <int HD>
struct HShape {
    static constexpr int NB = HD / kQ4Block;          // Q4 blocks per row
    static constexpr int RB = NB * kQ4BlockBytes;     // row bytes
    static constexpr int TK = 32;                     // keys per tile
    static constexpr int TILE = TK * RB;              // raw tile bytes
    // LDS slot of a tile: TILE rounded up to 256 bytes
    static constexpr int TSTR = (TILE + 255) / 256 * 256;
    // DMA instructions per tile, every lane active: 1 KB ones (16 bytes a
    // lane), then 256-byte dword ones for the rest of the slot (an LDS DMA
    // of fewer than 4 bytes still takes 4 bytes of LDS per lane); bytes past
    // the tile arrive as zeros in the slot's padding
    static constexpr int REM = TILE % 1024;
    static constexpr int NI = TILE / 1024 + (REM + 255) / 256;
    // P table row stride (floats): padded where the P and D tables still fit
    // in one K tile
    static constexpr int PS = 8 * (TK + 4) * 4 + NB * TK * 2 <= TILE ? TK + 4 : TK;
};

// K/V tile buffers per wave: the tile NBUF - 1 ahead is requested when a
// tile starts, so each tile's loads have NBUF - 1 tiles of work to land.
constexpr int kHiloBuffers = 2;

constexpr float kTau = 8.0f;            // lazy-rescale slack (log2 units)

// Two waves per SIMD (256 registers each): one wave's LDS reads and waits
// hide behind the other's VALU work. O (16 rows x head_dim) and the q limbs
// stay in registers through the tile loop; what does not fit is values live
// only around it.
template <int HD, int G>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64), amdgpu_waves_per_eu(2, 2)))
void decode_hilo_kernel(DecodeArgs a) {
    using Sh = HShape<HD>;
    constexpr int NB = Sh::NB, RB = Sh::RB, TK = Sh::TK, TILE = Sh::TILE, NI = Sh::NI;
    constexpr int TSTR = Sh::TSTR;
    constexpr int PS = Sh::PS;
    static_assert(G >= 1 && G <= 8, "group of at most 8 heads");

    constexpr int NBUF = kHiloBuffers;
    // ring of NBUF (K tile, V tile) buffers
    __shared__ __attribute__((aligned(16))) uint8_t KV[NBUF * 2 * TSTR];
    static_assert(8 * PS * 4 + NB * TK * 2 <= TILE, "P and D tables fit in a K tile");

    const int lane = threadIdx.x;
    const int n16 = lane & 15;          // MFMA column / row index within a 16-lane group
    const int g4 = lane >> 4;           // lane group: k-slots 8 g4 .. 8 g4 + 7
    const int hd4 = 4 * (g4 & 1);       // first head of this lane's accumulator rows
    const int w = blockIdx.x, NW = gridDim.x;
    unsigned vis = 0, skp = 0;

    auto run_segment = [&](int seg, int pos_seg, int it_lo, int it_hi, int pidx) {
        const int slot = seg / a.n_kv, kvh = seg % a.n_kv;
        const int pos = pos_seg;
        int split_len;
        slot_items(pos, a, &split_len);
        const int L = pos + 1;
        const int k_lo = it_lo * split_len;
        const int k_hi = min(L, it_hi * split_len);
        const size_t head_rows = ((size_t)slot * a.n_kv + kvh) * a.max_seq;
        const uint8_t *kb = (const uint8_t *)a.k + head_rows * RB;
        const uint8_t *vb = (const uint8_t *)a.v + head_rows * RB;
        const int win_first = pos - a.win + 1;

        // first visited tile at or after j ([FA] fc_attn_tile_in_window), in
        // the plan's 64-key tiles
        auto next_visited = [&](int j) -> int {
            if (j < k_hi && a.win > 0 && j >= a.sink &&
                min(j + kDecodeKeyTile - 1, k_hi - 1) < win_first) {
                const int jn = (win_first / kDecodeKeyTile) * kDecodeKeyTile;
                const int stop = min(jn, k_hi);
                skp += (unsigned)((stop - j + kDecodeKeyTile - 1) / kDecodeKeyTile);
                return jn >= k_hi ? k_hi : jn;
            }
            return j;
        };
        // raw 32-key K and V tiles at t0 <= k_hi into buffer `buf`; rows past
        // k_hi arrive as zeros (t0 = k_hi: an all-zero tile). The LDS
        // destination stays in the LDS address space (a generic pointer would
        // have to be cast back).
        typedef __attribute__((address_space(3))) uint8_t lds_u8;
        auto dma_tile = [&](int buf, int t0) {
            const unsigned bytes = (unsigned)(max(0, min(TK, k_hi - t0)) * RB);
            const __amdgpu_buffer_rsrc_t rk = raw_rsrc(kb + (size_t)t0 * RB, bytes);
            const __amdgpu_buffer_rsrc_t rv = raw_rsrc(vb + (size_t)t0 * RB, bytes);
            lds_u8 *dk = (lds_u8 *)KV + 2 * TSTR * buf;
            // no lane-dependent DMA: a conditional one makes the compiler's
            // count of outstanding loads conservative, and its wait for the q
            // loads would then wait for DMAs as well
#pragma unroll
            for (int c = 0; c < TILE / 1024; c++) {
                const unsigned o = (unsigned)(1024 * c + 16 * lane);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dk + 1024 * c, 16, o, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dk + TSTR + 1024 * c, 16, o, 0, 0, 0);
            }
            constexpr int B0 = TILE - Sh::REM;
#pragma unroll
            for (int c = 0; c < (Sh::REM + 255) / 256; c++) {
                const unsigned o = (unsigned)(B0 + 256 * c + 4 * lane);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dk + B0 + 256 * c, 4, o, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dk + TSTR + B0 + 256 * c, 4, o, 0, 0,
                                                         0);
            }
        };
        // the 32-key tile after t0: its second half, or the next visited
        // 64-key tile (tiles of the plan start at multiples of 64)
        auto next_tile = [&](int t0) -> int {
            if ((t0 & (kDecodeKeyTile - 1)) == 0 && t0 + TK < k_hi) return t0 + TK;
            return next_visited((t0 & ~(kDecodeKeyTile - 1)) + kDecodeKeyTile);
        };
        // wait until at most `later` tiles' requests are outstanding
        auto wait_tiles = [](int later) {
            if (later <= 0) wait_vmem_le<0>();
            else if (later == 1) wait_vmem_le<2 * NI>();
            else if (later == 2) wait_vmem_le<4 * NI>();
            else wait_vmem_le<6 * NI>();
        };
        wait_vmem_le<0>();          // nothing of an earlier segment in flight

        // ---- q operand of QK: row m = 8 limb + head, this lane's 8 contraction
        // elements of every block, and the per-block sums that the -8
        // correction MFMA takes. Byte t of the lane's code word (4 code bytes of
        // the block) gives B elements (lo(byte0), lo(byte2), lo(byte1),
        // lo(byte3), hi(byte0), hi(byte2), hi(byte1), hi(byte3)) where lo(x)
        // is element x and hi(x) element 16 + x of the block. Odd blocks: the
        // code word g is bytes 4g..4g+3; even blocks (code bytes start 2 bytes
        // into a dword): g < 3 takes bytes 4g+2..4g+5, g = 3 bytes 0, 1, 14, 15.
        // Either way the 8 elements are the pairs at o1 and o2 and at o1 + 16,
        // o2 + 16, interleaved: four 8-byte loads per block.
        const int qh = n16 & 7, limb = n16 >> 3;
        // rows past G read head G - 1 and are zeroed
        const float *qrow = a.q + ((size_t)slot * a.n_head + kvh * G + min(qh, G - 1)) * HD;
        float qv[NB][8];
#pragma unroll
        for (int b = 0; b < NB; b++) {
            const int o1 = (b & 1) ? 4 * g4 : (g4 < 3 ? 4 * g4 + 2 : 0);
            const int o2 = (b & 1) ? 4 * g4 + 2 : (g4 < 3 ? 4 * g4 + 4 : 14);
            const float *qb = qrow + b * kQ4Block;
            const float2 l1 = *(const float2 *)(qb + o1), l2 = *(const float2 *)(qb + o2);
            const float2 h1 = *(const float2 *)(qb + 16 + o1), h2 = *(const float2 *)(qb + 16 + o2);
            const float e[8] = {l1.x, l2.x, l1.y, l2.y, h1.x, h2.x, h1.y, h2.y};
#pragma unroll
            for (int i = 0; i < 8; i++) qv[b][i] = qh < G ? e[i] : 0.0f;
        }
        // rq[0] is the current tile, rq[1..] the ones requested after it (a
        // start >= k_hi: none); buf0 is rq[0]'s buffer. The first NBUF - 1
        // requests go out unconditionally (an empty one is an all-zero tile),
        // so the compiler's wait for the q loads above does not cover them:
        // they fly while the q operand is built.
        int rq[NBUF];
        int t_next = next_visited(k_lo);
        int buf0 = 0;
#pragma unroll
        for (int d = 0; d < NBUF - 1; d++) {
            rq[d] = t_next;
            dma_tile(d, t_next);
            if (t_next < k_hi) t_next = next_tile(t_next);
        }
        rq[NBUF - 1] = k_hi;

        float qmax = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; b++)
#pragma unroll
            for (int i = 0; i < 8; i++) qmax = fmaxf(qmax, fabsf(qv[b][i]));
        qmax = fmaxf(qmax, __shfl_xor(qmax, 16));
        qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
        int ex = 0;
        if (qmax > 0.0f) frexpf(qmax, &ex);             // qmax < 2^ex
        const int E = 11 - ex;                          // |q 2^E| < 2^11, |16 q 2^E| < 2^15
        u32x4 qa[NB];
        // The -8 of the codes: per (row, block) the MFMA gives
        // sum_i A_i B_i with B = c w 2^-24 (w the code weight of the slot), so
        // the block's term needs -8 2^-24 sum_i A_i w_i = -8 2^-24 part_b,
        // times the key's block scale d_b. Summed over blocks this is itself a
        // contraction: part_b 2^-6 (hi / lo limbs, lane groups 0 / 1) against
        // the keys' scales, one more MFMA per 16 keys, whose result enters the
        // score as -2^-15 x it.
        float cpart[NB];
#pragma unroll
        for (int b = 0; b < NB; b++) {
            _Float16 hv[8];
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float x = ldexpf(qv[b][i], E + (i < 4 ? 4 : 0));   // low-nibble slots x16
                const _Float16 hi = (_Float16)x;
                const _Float16 lo = (_Float16)(x - (float)hi);
                hv[i] = limb ? lo : hi;
                part += (float)hv[i] * (i < 4 ? 1.0f : 16.0f);   // the code weight of slot i
            }
            qa[b] = u32x4{pack_h2(hv[0], hv[1]), pack_h2(hv[2], hv[3]), pack_h2(hv[4], hv[5]),
                          pack_h2(hv[6], hv[7])};
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);                  // row n16's sum over the block
            cpart[b] = ldexpf(part, -6);                   // |part| < 2^20: fits binary16
        }
        u32x4 qcorr;
        {
            _Float16 cv[8];
#pragma unroll
            for (int b = 0; b < 8; b++) {
                const float x = b < NB ? cpart[b] : 0.0f;
                const _Float16 hi = (_Float16)x;
                const _Float16 lo = (_Float16)(x - (float)hi);
                cv[b] = g4 == 0 ? hi : g4 == 1 ? lo : (_Float16)0.0f;
            }
            qcorr = u32x4{pack_h2(cv[0], cv[1]), pack_h2(cv[2], cv[3]), pack_h2(cv[4], cv[5]),
                          pack_h2(cv[6], cv[7])};
        }
        // score scale of this lane's heads hd4 + r: qscale * 2^(20 - E_head)
        // (16 * 2^-24 from the code encoding, 2^-E from q')
        float cs[4];
#pragma unroll
        for (int r = 0; r < 4; r++)
            cs[r] = ldexpf(a.qscale, 20 - __shfl(E, hd4 + r));

        float m[4], l[4];
        f32x4 Olo[NB], Ohi[NB], Kc = f32x4{};
#pragma unroll
        for (int r = 0; r < 4; r++) {
            m[r] = -INFINITY;
            l[r] = 0.0f;
        }
#pragma unroll
        for (int b = 0; b < NB; b++) Olo[b] = Ohi[b] = f32x4{};
        // O is kept in units of 2^-F (A = p d 2^-F < 2^15 needs |d| < 2^(F + 7)):
        // fthr is the binary16 biased exponent at which a scale breaks that
        int F = -64, fthr = 0;
        float pscale = 0.0f;

        while (rq[0] < k_hi) {
            {
                const int t0 = rq[0];
                // request the tile NBUF - 1 ahead into the previous tile's buffer
                const int bnew = buf0 == 0 ? NBUF - 1 : buf0 - 1;
                rq[NBUF - 1] = t_next;
                if (t_next < k_hi) {
                    wait_lds();
                    dma_tile(bnew, t_next);
                    t_next = next_tile(t_next);
                }
                int later = 0;
#pragma unroll
                for (int d = 1; d < NBUF; d++) later += rq[d] < k_hi ? 1 : 0;
                wait_tiles(later);                  // this tile's K and V are in LDS
                if ((t0 & (kDecodeKeyTile - 1)) == 0) vis++;
                const uint8_t *Kt = KV + 2 * TSTR * buf0;
                const uint8_t *Vt = Kt + TSTR;
                // p [head][key] and the V block scales [block][key] go to this
                // buffer's K tile once QK has read it (the buffer is refilled
                // only after every LDS read of this tile has completed). In
                // arrays of their own, the compiler's LDS-DMA tracking made the
                // first read of them wait for the next tile's DMA.
                float *Pt = (float *)(KV + 2 * TSTR * buf0);
                uint16_t *Dt = (uint16_t *)(KV + 2 * TSTR * buf0 + 8 * PS * 4);

                // ---- QK: two sets of 16 keys, one MFMA per (set, block) plus
                // one for the -8 of the codes
                auto qk_set = [&](int s) -> f32x4 {
                    f32x4 acc = f32x4{};
                    const uint8_t *row = Kt + (16 * s + n16) * RB;
                    uint32_t dh[NB];                   // this key's block scales (binary16 bits)
#pragma unroll
                    for (int b = 0; b < NB; b++) {
                        uint32_t cw, sdw;
                        if (b & 1) {
                            cw = *(const uint32_t *)(row + 18 * b + 2 + 4 * g4);
                            sdw = *(const uint32_t *)(row + 18 * b - 2) >> 16;
                        } else {
                            sdw = *(const uint32_t *)(row + 18 * b);
                            const uint32_t da =
                                *(const uint32_t *)(row + 18 * b + (g4 < 3 ? 4 + 4 * g4 : 0));
                            const uint32_t db = *(const uint32_t *)(row + 18 * b + 16);
                            // g < 3: the word itself; g = 3: bytes 2, 3 of the
                            // scale word then bytes 0, 1 of the word at 16
                            cw = __builtin_amdgcn_perm(db, da, g4 < 3 ? 0x03020100u : 0x05040302u);
                        }
                        dh[b] = sdw & 0xffffu;
                        const uint32_t c8 = cw >> 8;
                        const u32x4 bq = {cw & 0x000F000Fu, c8 & 0x000F000Fu, cw & 0x00F000F0u,
                                          c8 & 0x00F000F0u};
                        const f32x4 c = mfma16h(qa[b], bq, f32x4{});
                        const float d = lo_h(sdw);
#pragma unroll
                        for (int r = 0; r < 4; r++) acc[r] = fmaf(c[r], d, acc[r]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    // scales of this key for blocks 0..7 (k-slots of lane groups 0, 1)
                    u32x4 bd = {};
                    if (g4 < 2) {
#pragma unroll
                        for (int q2 = 0; q2 < 4; q2++) {
                            const uint32_t d0 = 2 * q2 < NB ? dh[2 * q2] : 0u;
                            const uint32_t d1 = 2 * q2 + 1 < NB ? dh[2 * q2 + 1] : 0u;
                            bd[q2] = d0 | (d1 << 16);
                        }
                    }
                    const f32x4 cc = mfma16h(qcorr, bd, f32x4{});
#pragma unroll
                    for (int r = 0; r < 4; r++) acc[r] = fmaf(cc[r], -3.0517578125e-05f, acc[r]);
                    return acc;
                };
                const f32x4 S0 = qk_set(0);
                const f32x4 S1 = qk_set(1);

                // ---- softmax. Sum the limb rows: lanes 0-31 get keys 0-15,
                // lanes 32-63 keys 16-31 (heads hd4 + r, key n16 of the set).
                const int kl = 16 * (lane >> 5) + n16;
                const int key = t0 + kl;
                const bool kval = key < k_hi && in_key_set(key, pos, a.sink, a.win);
                float sc[4];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    // (elements copied out first: __builtin_bit_cast of an indexed
                    // vector element reads element 0 with this compiler)
                    const float s0 = S0[r], s1 = S1[r];
                    const auto sw = __builtin_amdgcn_permlane32_swap(
                        __builtin_bit_cast(uint32_t, s0), __builtin_bit_cast(uint32_t, s1), false,
                        false);
                    const float t = __builtin_bit_cast(float, (uint32_t)sw[0]) +
                                    __builtin_bit_cast(float, (uint32_t)sw[1]);
                    sc[r] = kval ? t * cs[r] : -INFINITY;
                }
                bool up = false;
#pragma unroll
                for (int r = 0; r < 4; r++) up |= sc[r] > m[r] + kTau;
                if (__ballot(up)) {
                    // new reference max for every head: over this tile's 32 keys
                    // (16 lanes of a row, both halves)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        float x = sc[r];
                        x = fmaxf(x, __shfl_xor(x, 1));
                        x = fmaxf(x, __shfl_xor(x, 2));
                        x = fmaxf(x, __shfl_xor(x, 4));
                        x = fmaxf(x, __shfl_xor(x, 8));
                        x = fmaxf(x, __shfl_xor(x, 32));
                        const float m_new = fmaxf(m[r], x);
                        const float corr = m_new == -INFINITY ? 1.0f : fast_exp2(m[r] - m_new);
                        m[r] = m_new;
                        l[r] *= corr;
#pragma unroll
                        for (int b = 0; b < NB; b++) {
                            Olo[b][r] *= corr;
                            Ohi[b][r] *= corr;
                        }
                        Kc[r] *= corr;
                    }
                }
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    // a masked key adds nothing, also while no key has been seen
                    p[r] = kval ? fast_exp2(sc[r] - m[r]) : 0.0f;
                    l[r] += p[r];
                }

                wave_lds_sync();     // QK's reads of the K tile come first
#pragma unroll
                for (int r = 0; r < 4; r++) Pt[(hd4 + r) * PS + kl] = p[r];
                // V block scales, [block][key]; lane: key lane & 31, blocks of its half
                {
                    const int vk = lane & 31;
                    int emax = 0;
#pragma unroll
                    for (int i = 0; i < NB / 2; i++) {        // same trip count in every lane
                        const int b = 2 * i + (lane >> 5);
                        const uint16_t dbits = *(const uint16_t *)(Vt + vk * RB + 18 * b);
                        Dt[b * TK + vk] = dbits;
                        emax = max(emax, (int)((dbits >> 10) & 31));
                    }
                    // a scale with binary16 exponent >= fthr would put p d 2^-F
                    // past 2^15: raise F (rare) and rescale O, kept exact (powers of 2)
                    if (__ballot(emax >= fthr)) {
                        int e = emax;
#pragma unroll
                        for (int o = 32; o >= 1; o >>= 1) e = max(e, __shfl_xor(e, o));
                        // |d| < 2^(e - 14); keep |d| 2^-F < 2^7
                        const int F_new = e - 21;
                        if (F_new > F) {
                            const float sh = ldexpf(1.0f, F - F_new);
#pragma unroll
                            for (int b = 0; b < NB; b++)
#pragma unroll
                                for (int r = 0; r < 4; r++) {
                                    Olo[b][r] *= sh;
                                    Ohi[b][r] *= sh;
                                }
                            F = F_new;
                        }
                        fthr = F + 21 + 1;
                        pscale = ldexpf(1.0f, -F);
                    }
                }
                wave_lds_sync();

                // ---- PV: rows (limb, head); this lane's 8 keys 8 g4 .. 8 g4 + 7
                const f32x4 pa = *(const f32x4 *)(Pt + qh * PS + 8 * g4);
                const f32x4 pb = *(const f32x4 *)(Pt + qh * PS + 8 * g4 + 4);
                const float pk[8] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
                // limb selection: the high-limb rows take fp16(x), the low-limb
                // rows fp16(x - fp16(x)); z is fp16(x) on the low rows, 0 on
                // the high rows, and the operand is fp16(x - z)
                float pf[8], pz[8];
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    pf[k] = pk[k] * pscale;
                    pz[k] = limb ? pf[k] : 0.0f;
                }
                // the -8 of the codes: Kc[row][block] += sum_j limb(128 p_j) d_jb
                // (p <= 2^8 after the lazy rescale; the factor 2^7 keeps the low
                // limbs of small p out of the binary16 subnormals)
                {
                    uint32_t ap[4];
#pragma unroll
                    for (int k2 = 0; k2 < 4; k2++) {
                        const float x0 = pk[2 * k2] * 128.0f, x1 = pk[2 * k2 + 1] * 128.0f;
                        const _Float16 z0 = (_Float16)(limb ? x0 : 0.0f);
                        const _Float16 z1 = (_Float16)(limb ? x1 : 0.0f);
                        ap[k2] = pack_h2((_Float16)(x0 - (float)z0), (_Float16)(x1 - (float)z1));
                    }
                    const u32x4 bd = n16 < NB ? *(const u32x4 *)(Dt + n16 * TK + 8 * g4) : u32x4{};
                    Kc = mfma16h(u32x4{ap[0], ap[1], ap[2], ap[3]}, bd, Kc);
                }
#pragma unroll
                for (int b = 0; b < NB; b++) {
                    const u32x4 d8 = *(const u32x4 *)(Dt + b * TK + 8 * g4);
                    uint32_t av[4];
#pragma unroll
                    for (int k2 = 0; k2 < 4; k2++) {
                        const float d0 = lo_h(d8[k2]), d1 = hi_h(d8[k2]);
                        const _Float16 z0 = (_Float16)(pz[2 * k2] * d0);
                        const _Float16 z1 = (_Float16)(pz[2 * k2 + 1] * d1);
                        av[k2] = pack_h2((_Float16)fmaf(pf[2 * k2], d0, -(float)z0),
                                         (_Float16)fmaf(pf[2 * k2 + 1], d1, -(float)z1));
                    }
                    const u32x4 A = {av[0], av[1], av[2], av[3]};
                    // codes of byte n16 of block b for keys 8 g4 + k, paired
                    const uint8_t *vcol = Vt + (8 * g4) * RB + 18 * b + 2 + n16;
                    uint32_t pr[4];
#pragma unroll
                    for (int k2 = 0; k2 < 4; k2++)
                        pr[k2] = __builtin_bit_cast(
                            uint32_t, u16x2{vcol[(2 * k2) * RB], vcol[(2 * k2 + 1) * RB]});
                    const u32x4 blo = {pr[0] & 0x000F000Fu, pr[1] & 0x000F000Fu,
                                       pr[2] & 0x000F000Fu, pr[3] & 0x000F000Fu};
                    const u32x4 bhi = {pr[0] & 0x00F000F0u, pr[1] & 0x00F000F0u,
                                       pr[2] & 0x00F000F0u, pr[3] & 0x00F000F0u};
                    Olo[b] = mfma16h(A, blo, Olo[b]);
                    Ohi[b] = mfma16h(A, bhi, Ohi[b]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int d = 0; d < NBUF - 1; d++) rq[d] = rq[d + 1];
            buf0 = buf0 + 1 == NBUF ? 0 : buf0 + 1;
        }

        // ---- this segment's partial: m, l and acc for the G heads
#pragma unroll
        for (int r = 0; r < 4; r++) {
            float x = l[r];
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
            x += __shfl_xor(x, 32);
            l[r] = x;
        }
        // limb rows summed (lanes l and l ^ 32 hold the two limbs of a head)
        auto limb_sum = [](float x) -> float {
            const uint32_t u = __builtin_bit_cast(uint32_t, x);
            const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            return __builtin_bit_cast(float, (uint32_t)sw[0]) +
                   __builtin_bit_cast(float, (uint32_t)sw[1]);
        };
        const size_t pbase = (size_t)pidx * G;
        if (n16 == 0 && lane < 32) {
#pragma unroll
            for (int r = 0; r < 4; r++)
                if (hd4 + r < G) {
                    a.ws_m[pbase + hd4 + r] = m[r];
                    a.ws_l[pbase + hd4 + r] = l[r];
                }
        }
        // acc[h][dim] = O 2^(F + 24) / w_dim - 8 Kc[h][block] / 128; O units 2^-F,
        // codes weighted 1 (low nibble dims) or 16 (high nibble dims)
        float kcf[4];
#pragma unroll
        for (int r = 0; r < 4; r++) kcf[r] = limb_sum(Kc[r]);
        const float olo_s = ldexpf(1.0f, F + 24), ohi_s = ldexpf(1.0f, F + 20);
#pragma unroll
        for (int b = 0; b < NB; b++) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float kb8 = 0.0625f * __shfl(kcf[r], 16 * (g4 & 1) + b);   // 8 Kc / 128
                const float vlo = limb_sum(Olo[b][r]) * olo_s - kb8;
                const float vhi = limb_sum(Ohi[b][r]) * ohi_s - kb8;
                if (lane < 32 && hd4 + r < G) {
                    float *dst = a.ws_acc + (pbase + hd4 + r) * HD + b * kQ4Block;
                    dst[n16] = vlo;
                    dst[16 + n16] = vhi;
                }
            }
        }
    };

    decode_stream_k<false, kDecodeWeightFirstHilo, kDecodeWeightSecondHilo>(a, w, NW, lane,
                                                                            run_segment);
    // a segment with no tiles still issued its first (all-zero) tile DMA:
    // nothing may be in flight into this work-group's LDS when it ends
    wait_vmem_le<0>();

    if (a.stats && lane == 0) {
        atomicAdd(&a.stats[0], (unsigned long long)vis);
        atomicAdd(&a.stats[1], (unsigned long long)skp);
    }
}

template <int HD, int G>
hipError_t launch_one(const DecodeArgs &a, int waves, hipStream_t s) {
    hipLaunchKernelGGL((decode_hilo_kernel<HD, G>), dim3(waves), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_combine(HD, G, a, s);
}

template <int HD>
hipError_t by_group(int group, const DecodeArgs &a, int waves, hipStream_t s) {
    switch (group) {
    case 1: return launch_one<HD, 1>(a, waves, s);
    case 2: return launch_one<HD, 2>(a, waves, s);
    case 4: return launch_one<HD, 4>(a, waves, s);
    case 8: return launch_one<HD, 8>(a, waves, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_hilo(int head_dim, int group, const DecodeArgs &a, int waves,
                              hipStream_t s) {
    switch (head_dim) {
    case 64: return by_group<64>(group, a, waves, s);
    case 128: return by_group<128>(group, a, waves, s);
    case 256: return by_group<256>(group, a, waves, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
