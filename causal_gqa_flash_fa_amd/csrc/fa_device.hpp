// Device-side helpers shared by the libfa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Q4_0 block geometry ([FA] "4-bit KV cache (Q4_0 blocks)"): 32 elements in
// 18 bytes, a binary16 scale then 16 code bytes (element j low nibble,
// element j+16 high nibble of byte 2+j).
constexpr int kQ4Block = 32;
constexpr int kQ4BlockBytes = 18;

__host__ __device__ constexpr int q4_row_bytes(int head_dim) {
    return head_dim / kQ4Block * kQ4BlockBytes;
}

// log2(e): scores are kept in base-2 units (s * log2 e) so the softmax
// exponentials are single v_exp_f32 instructions.
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

// Raw buffer descriptor over `bytes` bytes at `base` (dword 3: 32-bit data
// format, as for plain dword loads). Loads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// 16-byte buffer -> LDS copy (buffer_load_dwordx4 ... lds): lane i writes
// lds[16i .. 16i+15] from byte offset voff of the buffer; the LDS base is
// wave-uniform and inactive lanes write nothing. Completion is counted by
// vmcnt. The buffer form (rather than the global one) matters for the
// compiler: its wait-count model treats a pending global (flat-encoded) LDS
// load as touching both memory paths and then waits for every outstanding
// LDS read before each use.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, unsigned voff, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)lds,
                                             16, voff, 0, 0, 0);
}

// Wait until at most `n` of this wave's vector-memory operations (loads,
// LDS DMA, stores) are outstanding; they complete in issue order.
template <int n>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ float fast_exp2(float x) {
    return __builtin_amdgcn_exp2f(x);   // v_exp_f32; exp2(-inf) = 0
}

__device__ __forceinline__ float lo_h(uint32_t r) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(r & 0xffffu));
}
__device__ __forceinline__ float hi_h(uint32_t r) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(r >> 16));
}

// The 8 elements held by one code word w (bytes b0..b3): element e = low
// nibble of byte e, element 16 + e = high nibble of byte e (e = 0..3, relative
// to the word). A nibble masked into a binary16 with exponent bits 0x6400
// gives 1024 + c (low nibble, bits 0-3) or 1024 + 16 c (high nibble, bits
// 4-7, still inside the 10-bit mantissa), so one and-or per two elements
// builds fma_mix operands: (1024 + c) d - 1032 d and (1024 + 16 c) (d / 16)
// - 72 d are both exactly (c - 8) d. `k` holds the masks and exponent bits in
// registers so the and-or is a single three-operand instruction.
struct NibConsts {
    uint32_t lo, hi, ex;
};
__device__ __forceinline__ NibConsts nib_consts() {
    NibConsts k;
    // opaque to the compiler: kept in VGPRs instead of being folded as literals
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(k.lo));
    asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(k.hi));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.ex));
    return k;
}
// The per-block constants of dequant_word.
struct BlockScale {
    float d, d16, blo, bhi;
};
__device__ __forceinline__ BlockScale block_scale(float d) {
    return BlockScale{d, d * 0.0625f, -1032.0f * d, -72.0f * d};
}
// out[0..3] = elements e = 0..3 (low nibbles), out[4..7] = elements 16 + e.
__device__ __forceinline__ void dequant_word(uint32_t w, const BlockScale &sc, const NibConsts &k,
                                             float *out) {
    const float d = sc.d, d16 = sc.d16, blo = sc.blo, bhi = sc.bhi;
    const uint32_t w8 = w >> 8;
    const uint32_t a = (w & k.lo) | k.ex;     // bytes 0, 2 low nibbles
    const uint32_t b = (w8 & k.lo) | k.ex;    // bytes 1, 3 low nibbles
    const uint32_t c = (w & k.hi) | k.ex;     // bytes 0, 2 high nibbles (x16)
    const uint32_t e = (w8 & k.hi) | k.ex;    // bytes 1, 3 high nibbles (x16)
    out[0] = fmaf(lo_h(a), d, blo);
    out[1] = fmaf(lo_h(b), d, blo);
    out[2] = fmaf(hi_h(a), d, blo);
    out[3] = fmaf(hi_h(b), d, blo);
    out[4] = fmaf(lo_h(c), d16, bhi);
    out[5] = fmaf(lo_h(e), d16, bhi);
    out[6] = fmaf(hi_h(c), d16, bhi);
    out[7] = fmaf(hi_h(e), d16, bhi);
}

// MFMA wrappers (fp32 inputs, fp32 accumulate).
//   16x16x4: A[m][k] from lane (m = lane&15, k = lane>>4), B[k][n] from lane
//   (k = lane>>4, n = lane&15); D[m][n] in lane (n = lane&15), register r
//   holding m = 4*(lane>>4) + r.
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
//   4x4x1, 16 blocks: lane 4*blk+i gives A_blk[i], lane 4*blk+j gives
//   B_blk[j]; D_blk[i][j] lands in lane 4*blk+j, register i.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

// max(x[l], x[l ^ 32]) for every lane l. v_permlane32_swap exchanges the
// two 32-lane halves of a register: each lane receives its own value and its
// partner's, in an order that depends on the half (lanes below 32 get their
// own first), which a symmetric max does not see. One VALU instruction, where
// a shuffle through ds_bpermute is an LDS round trip.
__device__ __forceinline__ float half_swap_max(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// max(x[l], x[l ^ 16]) for every lane l: ds_swizzle in bitmask mode (within
// each 32-lane half, lane j reads lane j ^ 16), no LDS access.
__device__ __forceinline__ float row16_swap_max(float x) {
    const int y = __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), (0x10 << 10) | 0x1f);
    return fmaxf(x, __builtin_bit_cast(float, y));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data (a wave's LDS operations execute in order; this stops the compiler
// from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Work-group barrier that orders LDS accesses only: the wave's LDS
// operations complete before it arrives, while global loads and stores stay
// in flight across it (a full __syncthreads waits for those too).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Key-set membership ([FA] file header): causal, plus sink U recent window
// when attn_win > 0.
__device__ __forceinline__ bool in_key_set(int j, int p, int sink, int win) {
    return j <= p && (win <= 0 || j < sink || j >= p - win + 1);
}

}  // namespace fa
