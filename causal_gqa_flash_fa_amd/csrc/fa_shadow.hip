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
#include "fa_shadow.hpp"

namespace fa {
namespace {

template <int HD, int G>
__global__ __launch_bounds__(64) void shadow_pass_kernel(ShadowPassArgs a) {
    __shared__ __attribute__((aligned(16))) float Qs[G * HD];
    __shared__ float Ps[G * 64];
    __shared__ int Rs[64];
    shadow_pass_wave<HD, G>(a, blockIdx.x, Qs, Ps, Rs);
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
