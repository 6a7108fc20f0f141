// KV-cache append: fp32 copy and fp32 -> Q4_0 block quantisation.
//
// [FA] fc_attn_kv_append: rows [n][n_kv][hd] land at cache[kv][pos0+t][:].
// [FA] fc_attn_kv_append_slots ("Multi-user decode attention (slots)"
// section): row t of [n_slots][n_kv][hd] lands in slot t at the position held
// in device memory, so the enqueued work does not depend on the position.
// The Q4_0 block format is an interchange format, so its definition fixes
// both the bytes and the order of the steps that produce them ([FA] "4-bit KV
// cache (Q4_0 blocks)" section, fc_kvq4_quant_block): per 32-element block,
// amax is the max of |x| (from 0); the scale d = amax / -8 (negative); with
// id = 1/d (0 for d = 0) each element's code is rint(x id) + 8 held to
// [0, 15]; bytes 0-1 are binary16(d) little-endian and byte 2 + j packs
// code_j | code_{j+16} << 4. A value decodes as (code - 8) d. Every step is an
// IEEE fp32 operation (correctly rounded divide, v_rndne for rint,
// v_cvt_f16_f32 round-to-even), so the bytes equal those of any other exact
// implementation of the definition.
//
// One thread owns one 32-element block here (no cross-lane fold), so both
// launches are plain streaming kernels: each thread reads 128 B of input and
// writes 18 B (Q4) or 16 B (fp32) with consecutive threads on consecutive
// addresses.
#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int kAppendThreads = 256;

// Cache row (h, position) of input row t and the byte offset of its slot;
// false when a device position lies outside the cache (nothing is written).
__device__ __forceinline__ bool dest_row(const AppendArgs &a, int t, int h, int64_t *row,
                                         size_t *slot_off, int *pos_out) {
    int pos = a.pos0 + t;
    *slot_off = 0;
    if (a.d_pos) {
        pos = a.d_pos[t];
        if (pos < 0 || pos >= a.max_seq) return false;
        *slot_off = (size_t)t * a.slot_bytes;
    }
    *row = (int64_t)h * a.max_seq + pos;
    *pos_out = pos;
    return true;
}

// fp16 shadow of one 32-element block of row `pos` ([FA] fc_attn_kv_append_q4
// mirror): the sink copy while pos < sink, the ring copy at row pos % ring
// size. A range append writes the ring only for its last kShadowWinMax rows,
// so no two threads of one call write the same ring row; one thread per row
// records the position the ring row now holds.
__device__ __forceinline__ void mirror_block(const AppendArgs &a, int tensor, int t, int h,
                                             int blk, int pos, const float *x) {
    const ShadowArgs &sh = a.sh;
    const int slot = a.d_pos ? t : 0;   // a range append's shadow bases are its slot's
    const size_t hd = (size_t)a.head_dim;
    u32x4 w[kQ4Block / 8];
#pragma unroll
    for (int c = 0; c < kQ4Block / 8; c++) {
        uint32_t hw[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)x[8 * c + 2 * i]);
            const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)x[8 * c + 2 * i + 1]);
            hw[i] = lo | (hi << 16);
        }
        w[c] = u32x4{hw[0], hw[1], hw[2], hw[3]};
    }
    if (pos < sh.sink) {
        uint16_t *base = tensor ? sh.v_sink : sh.k_sink;
        u32x4 *d = (u32x4 *)(base + (((size_t)slot * a.n_kv + h) * kShadowSinkMax + pos) * hd +
                             blk * kQ4Block);
#pragma unroll
        for (int c = 0; c < kQ4Block / 8; c++) d[c] = w[c];
    }
    const bool ring = sh.win > 0 && (a.d_pos || pos > a.pos0 + a.n - 1 - kShadowWinMax);
    if (ring) {
        uint16_t *base = tensor ? sh.v_win : sh.k_win;
        const int r = pos % kShadowWinMax;
        u32x4 *d = (u32x4 *)(base + (((size_t)slot * a.n_kv + h) * kShadowWinMax + r) * hd +
                             blk * kQ4Block);
#pragma unroll
        for (int c = 0; c < kQ4Block / 8; c++) d[c] = w[c];
        if (tensor == 0 && h == 0 && blk == 0) sh.win_pos[(size_t)slot * kShadowWinMax + r] = pos;
    }
}

__global__ __launch_bounds__(kAppendThreads) void append_f32_kernel(AppendArgs a) {
    const int tensor = blockIdx.y;                    // 0: K, 1: V
    const float *src = tensor ? a.v_new : a.k_new;
    uint8_t *base = (uint8_t *)(tensor ? a.v : a.k);
    const int c4_per_row = a.head_dim / 4;
    const int64_t total = (int64_t)a.n * a.n_kv * c4_per_row;
    const int64_t i = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
    if (i >= total) return;
    const int c4 = (int)(i % c4_per_row);
    const int64_t th = i / c4_per_row;                // t * n_kv + h
    const int h = (int)(th % a.n_kv);
    const int t = (int)(th / a.n_kv);
    int64_t row;
    size_t slot_off;
    int pos;
    if (!dest_row(a, t, h, &row, &slot_off, &pos)) return;
    const f32x4 x = *(const f32x4 *)(src + 4 * i);
    float *dst = (float *)(base + slot_off);
    *(f32x4 *)(dst + row * a.head_dim + 4 * c4) = x;
}

// Code of one element: clamp(rint(x * id) + 8, 0, 15) ([FA] fc_kvq4_quant_block),
// with the clamp taken in float before the integer conversion so that every
// product has a defined code: a NaN product (a NaN element, or 0 * inf when
// 1/d overflows for a block whose amax is below 2^-125) gives code 8, and
// infinities clamp to codes 0 and 15. On finite in-range data this is the
// integer clamp exactly.
__device__ __forceinline__ int q4_code(float x, float id) {
    const float r = rintf(x * id);
    const float t = r != r ? 0.0f : fminf(fmaxf(r, -8.0f), 7.0f);
    return (int)t + 8;
}

__global__ __launch_bounds__(kAppendThreads) void append_q4_kernel(AppendArgs a) {
    const int tensor = blockIdx.y;
    const float *src = tensor ? a.v_new : a.k_new;
    uint8_t *base = (uint8_t *)(tensor ? a.v : a.k);
    const int nb = a.head_dim / kQ4Block;
    const int64_t total = (int64_t)a.n * a.n_kv * nb;
    const int64_t i = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
    if (i >= total) return;
    const int blk = (int)(i % nb);
    const int64_t th = i / nb;
    const int h = (int)(th % a.n_kv);
    const int t = (int)(th / a.n_kv);
    int64_t row;
    size_t slot_off;
    int pos;
    if (!dest_row(a, t, h, &row, &slot_off, &pos)) return;

    float x[kQ4Block];
    const f32x4 *xs = (const f32x4 *)(src + i * kQ4Block);
#pragma unroll
    for (int c = 0; c < kQ4Block / 4; c++) {
        const f32x4 v = xs[c];
        x[4 * c + 0] = v[0];
        x[4 * c + 1] = v[1];
        x[4 * c + 2] = v[2];
        x[4 * c + 3] = v[3];
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kQ4Block; j++)
        amax = fmaxf(amax, fabsf(x[j]));
    const float d = amax / -8.0f;
    const float id = (d != 0.0f) ? 1.0f / d : 0.0f;

    const int rb = q4_row_bytes(a.head_dim);
    uint16_t *out = (uint16_t *)(base + slot_off + row * rb + blk * kQ4BlockBytes);
    // A zero scale is stored as binary16 -0.0 (0x8000), the sign of amax/-8.
    // Spelled out because the compiler folds the divide-by-(-8) and the fp16
    // conversion into one fused multiply-add whose +0 addend would turn -0
    // into +0.
    out[0] = d == 0.0f ? (uint16_t)0x8000u : __builtin_bit_cast(uint16_t, (_Float16)d);
#pragma unroll
    for (int j = 0; j < kQ4Block / 2; j += 2) {
        const int c0 = q4_code(x[j], id);
        const int c1 = q4_code(x[j + 1], id);
        const int c16 = q4_code(x[j + 16], id);
        const int c17 = q4_code(x[j + 17], id);
        const uint32_t b0 = (uint32_t)(c0 | (c16 << 4));
        const uint32_t b1 = (uint32_t)(c1 | (c17 << 4));
        out[1 + j / 2] = (uint16_t)(b0 | (b1 << 8));   // bytes 2+j, 3+j (little-endian)
    }
    if (a.sh.sink > 0 || a.sh.win > 0) mirror_block(a, tensor, t, h, blk, pos, x);
}

}  // namespace

hipError_t launch_append(int format, const AppendArgs &a, hipStream_t s) {
    const int per_row = format == 0 ? a.head_dim / 4 : a.head_dim / kQ4Block;
    const int64_t total = (int64_t)a.n * a.n_kv * per_row;
    const dim3 grid((unsigned)((total + kAppendThreads - 1) / kAppendThreads), 2);
    if (format == 0)
        hipLaunchKernelGGL(append_f32_kernel, grid, dim3(kAppendThreads), 0, s, a);
    else
        hipLaunchKernelGGL(append_q4_kernel, grid, dim3(kAppendThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace fa
