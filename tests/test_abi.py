"""Host-side checks of libfa that need no GPU: the library loads, exports every
entry point include/fa.h declares, validates arguments before touching the
device, and its plan / geometry helpers agree with the oracle.
"""
import ctypes
import os
import re

import pytest

import causal_gqa_flash_fa_amd as fa
import oracle
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fa.h")
FAKE = 0x10000   # never dereferenced: every call below is refused before any launch


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(fa.lib, name), name          # ctypes lookup of the exported symbol
    assert sorted(fa.EXPORTS) == names


def test_one_hip_runtime_in_the_process():
    # torch and libfa must share one HIP runtime: streams and errors are
    # per-runtime objects
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(os.path.realpath(line.split()[-1]))
    assert len(paths) == 1, paths


def test_strerror_names_every_code():
    for code in range(0, -8, -1):
        assert fa.fa_strerror(code) != "unknown error code"
    assert fa.fa_strerror(-99) == "unknown error code"


def cache(fmt=fa.FA_KV_F32, n_slots=2, n_kv=2, hd=128, max_seq=100, k=FAKE, v=FAKE):
    return fa.fa_cache(fmt, n_slots, n_kv, hd, max_seq, k, v)


def rc_append(c, slot=0, pos0=0, n=1, kn=FAKE, vn=FAKE):
    return fa.lib.fa_kv_append(ctypes.byref(c) if c is not None else None, slot, pos0, n, kn, vn,
                               None)


def rc_append_slots(c, pos=FAKE, n_slots=1, kn=FAKE, vn=FAKE):
    return fa.lib.fa_kv_append_slots(ctypes.byref(c) if c is not None else None, pos, n_slots,
                                     kn, vn, None)


def rc_prefill(c, slot=0, q=FAKE, pos0=0, n=1, n_head=4, sink=0, win=0, scale=0.1, out=FAKE,
               ws=FAKE, ws_bytes=1 << 30):
    return fa.lib.fa_prefill(ctypes.byref(c) if c is not None else None, slot, q, pos0, n,
                             n_head, sink, win, scale, out, ws, ws_bytes, None, None)


def rc_decode(c, q=FAKE, pos=FAKE, n_slots=1, hint=10, n_head=4, scale=0.1, out=FAKE, ws=FAKE,
              ws_bytes=1 << 30):
    return fa.lib.fa_decode(ctypes.byref(c) if c is not None else None, q, pos, n_slots, hint,
                            n_head, 0, 0, scale, out, ws, ws_bytes, None, None)


def test_row_and_cache_bytes():
    assert fa.fa_cache_row_bytes(fa.FA_KV_F32, 256) == 1024
    assert fa.fa_cache_row_bytes(fa.FA_KV_Q4_0, 256) == 144
    assert fa.fa_cache_row_bytes(fa.FA_KV_Q4_0, 64) == 36
    assert fa.fa_cache_row_bytes(fa.FA_KV_Q4_0, 96) == 0
    assert fa.fa_cache_row_bytes(7, 128) == 0
    assert fa.fa_cache_bytes(cache(fa.FA_KV_Q4_0, 3, 2, 256, 32768)) == 3 * 2 * 32768 * 144
    assert fa.fa_cache_bytes(cache(n_slots=0)) == 0


def test_append_validation():
    assert rc_append(None) == fa.FA_ENULL
    assert rc_append(cache(hd=96)) == fa.FA_EUNSUPPORTED
    assert rc_append(cache(fmt=5)) == fa.FA_EUNSUPPORTED
    assert rc_append(cache(k=0)) == fa.FA_ENULL
    assert rc_append(cache(max_seq=0)) == fa.FA_EINVAL
    assert rc_append(cache(), slot=2) == fa.FA_EINVAL
    assert rc_append(cache(), slot=-1) == fa.FA_EINVAL
    assert rc_append(cache(), pos0=-1) == fa.FA_EINVAL
    assert rc_append(cache(), n=-1) == fa.FA_EINVAL
    assert rc_append(cache(), pos0=90, n=11) == fa.FA_ERANGE      # would wrap: refused
    assert rc_append(cache(), pos0=0, n=0) == fa.FA_OK            # empty: nothing enqueued
    assert rc_append(cache(), pos0=100, n=0) == fa.FA_OK
    assert rc_append(cache(), kn=0) == fa.FA_ENULL


def test_append_slots_validation():
    assert rc_append_slots(None) == fa.FA_ENULL
    assert rc_append_slots(cache(hd=96)) == fa.FA_EUNSUPPORTED
    assert rc_append_slots(cache(fmt=5)) == fa.FA_EUNSUPPORTED
    assert rc_append_slots(cache(v=0)) == fa.FA_ENULL
    assert rc_append_slots(cache(), n_slots=3) == fa.FA_EINVAL      # more slots than the cache
    assert rc_append_slots(cache(), n_slots=-1) == fa.FA_EINVAL
    assert rc_append_slots(cache(), n_slots=0) == fa.FA_OK          # empty: nothing enqueued
    assert rc_append_slots(cache(), pos=0) == fa.FA_ENULL
    assert rc_append_slots(cache(), kn=0) == fa.FA_ENULL
    assert rc_append_slots(cache(), vn=0) == fa.FA_ENULL


def test_prefill_validation():
    c = cache()
    assert rc_prefill(None) == fa.FA_ENULL
    assert rc_prefill(c, n_head=3) == fa.FA_EINVAL                 # not a multiple of n_kv
    assert rc_prefill(c, n_head=32) == fa.FA_EUNSUPPORTED          # group 16
    assert rc_prefill(c, n_head=6) == fa.FA_EUNSUPPORTED           # group 3
    assert rc_prefill(c, scale=0.0) == fa.FA_EINVAL
    assert rc_prefill(c, scale=-1.0) == fa.FA_EINVAL
    assert rc_prefill(c, scale=float("nan")) == fa.FA_EINVAL
    assert rc_prefill(c, scale=float("inf")) == fa.FA_EINVAL
    assert rc_prefill(c, slot=5) == fa.FA_EINVAL
    assert rc_prefill(c, pos0=50, n=51) == fa.FA_ERANGE
    assert rc_prefill(c, n=0) == fa.FA_OK
    assert rc_prefill(c, q=0) == fa.FA_ENULL
    assert rc_prefill(c, out=0) == fa.FA_ENULL
    assert rc_prefill(c, ws=0) == fa.FA_ENULL
    need = fa.fa_prefill_workspace_bytes(40, 4, 2, 128)
    assert need > 0
    assert rc_prefill(c, n=40, ws_bytes=need - 1) == fa.FA_EWORKSPACE
    assert fa.fa_prefill_workspace_bytes(40, 6, 2, 128) == 0      # group 3
    assert fa.fa_prefill_workspace_bytes(40, 4, 2, 96) == 0
    # the cut list and the pieces do not grow with n, the shadow rows do
    assert fa.fa_prefill_workspace_bytes(40000, 4, 2, 128) >= need


def test_decode_validation():
    c = cache(n_slots=4, max_seq=100)
    need = fa.fa_decode_workspace_bytes(c, 4, 4, 100)
    # at least one partial {m, l, acc[hd]} per (slot, head) plus the segment table
    assert need >= 4 * 4 * (128 + 2) * 4 + 4 * 2 * 2 * 4
    assert fa.fa_decode_workspace_bytes(c, 2, 4, 100) <= need
    assert fa.fa_decode_workspace_bytes(c, 4, 4, 50) <= need
    assert fa.fa_decode_workspace_bytes(c, 4, 3, 100) == 0      # heads not a multiple of n_kv
    assert rc_decode(None) == fa.FA_ENULL
    assert rc_decode(c, n_slots=5) == fa.FA_EINVAL
    assert rc_decode(c, hint=0) == fa.FA_EINVAL
    assert rc_decode(c, hint=101) == fa.FA_EINVAL
    assert rc_decode(c, n_head=8, scale=0.0) == fa.FA_EINVAL
    assert rc_decode(c, n_slots=4, hint=100, ws_bytes=need - 1) == fa.FA_EWORKSPACE
    assert rc_decode(c, n_slots=0) == fa.FA_OK
    assert rc_decode(c, ws=0) == fa.FA_ENULL
    assert rc_decode(c, ws=FAKE + 4) == fa.FA_EINVAL             # not 16-byte aligned
    assert rc_decode(c, pos=0) == fa.FA_ENULL


def paged(nb=10, bs=16, n_kv=2, hd=128, stride=0, k=FAKE, v=FAKE):
    return fa.fa_paged_cache(nb, bs, n_kv, hd, stride, k, v)


def rc_paged_append(c, k=FAKE, v=FAKE, sm=FAKE, n=3):
    return fa.lib.fa_paged_append(ctypes.byref(c) if c is not None else None, k, v, sm, n, None)


def rc_paged(c, q=FAKE, T=5, H=4, qsl=FAKE, sl=FAKE, R=2, bt=FAKE, mb=4, wl=-1, wr=0,
             scale=0.1, out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30):
    return fa.lib.fa_paged_attention(ctypes.byref(c) if c is not None else None, q, T, H, qsl,
                                     sl, R, bt, mb, wl, wr, scale, out, lse, ws, ws_bytes, None)


def test_paged_append_validation():
    assert rc_paged_append(None) == fa.FA_ENULL
    assert rc_paged_append(paged(hd=96)) == fa.FA_EUNSUPPORTED
    assert rc_paged_append(paged(nb=0)) == fa.FA_EINVAL
    assert rc_paged_append(paged(bs=0)) == fa.FA_EINVAL
    assert rc_paged_append(paged(k=0)) == fa.FA_ENULL
    assert rc_paged_append(paged(k=FAKE + 4)) == fa.FA_EINVAL          # not 16-byte aligned
    assert rc_paged_append(paged(stride=16 * 2 * 128 - 4)) == fa.FA_EINVAL   # pages overlap
    assert rc_paged_append(paged(stride=2 * 16 * 2 * 128 + 2)) == fa.FA_EINVAL  # page misaligned
    assert rc_paged_append(paged(), n=-1) == fa.FA_EINVAL
    assert rc_paged_append(paged(), n=0) == fa.FA_OK
    assert rc_paged_append(paged(), sm=0) == fa.FA_ENULL
    assert rc_paged_append(paged(), v=0) == fa.FA_ENULL
    assert rc_paged_append(paged(), k=FAKE + 8) == fa.FA_EINVAL


def test_paged_attention_validation():
    c = paged()
    assert rc_paged(None) == fa.FA_ENULL
    assert rc_paged(c, H=3) == fa.FA_EINVAL
    assert rc_paged(c, H=32) == fa.FA_EUNSUPPORTED
    assert rc_paged(c, scale=0.0) == fa.FA_EINVAL
    assert rc_paged(c, R=1025) == fa.FA_EINVAL               # request table capacity
    assert rc_paged(c, R=-1) == fa.FA_EINVAL
    assert rc_paged(c, mb=0) == fa.FA_EINVAL
    assert rc_paged(c, mb=1 << 28) == fa.FA_EINVAL           # positions past int32
    assert rc_paged(c, wl=3, wr=-1) == fa.FA_EINVAL
    assert rc_paged(c, T=0) == fa.FA_OK
    assert rc_paged(c, R=0) == fa.FA_OK
    for name in ("q", "qsl", "sl", "bt", "out", "ws"):
        assert rc_paged(c, **{name: 0}) == fa.FA_ENULL, name
    assert rc_paged(c, q=FAKE + 4) == fa.FA_EINVAL
    need = fa.fa_paged_workspace_bytes(128)
    assert need > 0 and fa.fa_paged_workspace_bytes(96) == 0
    assert fa.fa_paged_workspace_bytes(256) > need
    assert rc_paged(c, ws_bytes=need - 1) == fa.FA_EWORKSPACE


def test_paged_decode_validation():
    def rc(c=None, q=FAKE, R=3, H=4, sl=FAKE, bt=FAKE, mb=4, hint=50, wl=-1, wr=0, scale=0.1,
           out=FAKE, ws=FAKE, ws_bytes=1 << 30):
        c = paged() if c is None else c
        return fa.lib.fa_paged_decode(ctypes.byref(c), q, R, H, sl, bt, mb, hint, wl, wr, scale,
                                      out, None, ws, ws_bytes, None)
    assert fa.lib.fa_paged_decode(None, FAKE, 1, 4, FAKE, FAKE, 4, 10, -1, 0, 0.1, FAKE, None,
                                  FAKE, 1 << 30, None) == fa.FA_ENULL
    assert rc(c=paged(bs=24)) == fa.FA_EUNSUPPORTED        # block size not a multiple of 16
    assert rc(c=paged(hd=96)) == fa.FA_EUNSUPPORTED
    assert rc(H=3) == fa.FA_EINVAL
    assert rc(H=32) == fa.FA_EUNSUPPORTED
    assert rc(scale=-1.0) == fa.FA_EINVAL
    assert rc(R=-1) == fa.FA_EINVAL
    assert rc(mb=0) == fa.FA_EINVAL
    assert rc(hint=0) == fa.FA_EINVAL
    assert rc(hint=65) == fa.FA_EINVAL                      # past max_blocks * block_size
    assert rc(wl=5, wr=-1) == fa.FA_EINVAL
    assert rc(R=0) == fa.FA_OK
    for name in ("q", "sl", "bt", "out", "ws"):
        assert rc(**{name: 0}) == fa.FA_ENULL, name
    assert rc(ws=FAKE + 8) == fa.FA_EINVAL                      # not 16-byte aligned
    need = fa.fa_paged_decode_workspace_bytes(3, 4, 2, 128, 50)
    assert need > 0 and rc(ws_bytes=need - 1) == fa.FA_EWORKSPACE
    assert fa.fa_paged_decode_workspace_bytes(3, 4, 2, 128, 0) == 0
    assert fa.fa_paged_decode_workspace_bytes(3, 6, 2, 128, 50) == 0
    assert fa.fa_paged_decode_workspace_bytes(3, 4, 2, 128, 5000) >= need


def test_merge_validation():
    def rc(T=4, H=2, D=128, out=FAKE, po=FAKE, pl=FAKE, so=FAKE, sl=FAKE):
        return fa.lib.fa_merge_attn_states(out, None, po, pl, so, sl, T, H, D, -1, None)
    assert rc(D=6) == fa.FA_EINVAL
    assert rc(D=0) == fa.FA_EINVAL
    assert rc(H=0) == fa.FA_EINVAL
    assert rc(T=-1) == fa.FA_EINVAL
    assert rc(T=0) == fa.FA_OK
    for name in ("out", "po", "pl", "so", "sl"):
        assert rc(**{name: 0}) == fa.FA_ENULL, name
    assert rc(so=FAKE + 4) == fa.FA_EINVAL


def test_plan_matches_oracle_with_library_constants():
    kps, cap, tile = fa.fa_decode_plan_params()
    assert tile == 64 and kps >= tile and cap >= 1
    for L in list(range(1, 200)) + [4096, 4097, 20000, 32767, 32768, 65536]:
        assert fa.fa_decode_plan(L) == oracle.decode_plan(L, kps, cap, tile)
    assert fa.lib.fa_decode_plan(0, None, None) == fa.FA_EINVAL


def test_prefill_tile_shape():
    assert fa.fa_prefill_tile_shape(16, 2, 256) == (16, 32)
    assert fa.fa_prefill_tile_shape(4, 1, 64) == (32, 32)
    assert fa.fa_prefill_tile_shape(8, 8, 128) == (128, 32)
    with pytest.raises(fa.FaError):
        fa.fa_prefill_tile_shape(16, 2, 96)


def gpu_count():
    import torch
    return torch.cuda.device_count()


@pytest.mark.skipif(gpu_count() > 0, reason="only meaningful where no GPU is present")
def test_valid_call_without_a_gpu_fails_loudly():
    rc = rc_prefill(cache())
    assert rc in (fa.FA_EHIP, fa.FA_EDEVICE)
    with pytest.raises(fa.FaError):
        fa.fa_init()


def causal_units(n, n_kv, bq, bk):
    """Stream-K units of a full-causal prefill from position 0: 4 per visited
    key tile (block [q0, q1] walks q1 // bk + 1 tiles) and 5 per query block,
    for every kv head (closed form of the causal tile walk)."""
    import numpy as np
    q1 = np.minimum(np.arange(0, n, bq, dtype=np.int64) + bq - 1, n - 1)
    return n_kv * int((4 * (q1 // bk + 1) + 5).sum())


def test_prefill_schedule_beyond_32_bits_is_refused():
    # The prefill kernel counts its stream-K schedule units in 32-bit
    # integers; a call whose total does not fit is refused before launch.
    n_kv, hd = 8, 64
    bq, bk = fa.fa_prefill_tile_shape(n_kv, n_kv, hd)
    limit = (1 << 31) - 1
    lo, hi = 1 << 18, 1 << 20
    assert causal_units(lo, n_kv, bq, bk) <= limit < causal_units(hi, n_kv, bq, bk)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if causal_units(mid, n_kv, bq, bk) <= limit else (lo, mid)
    # the closed form against the oracle's tile walk at the boundary
    for n in (lo, hi):
        vis, _ = oracle.prefill_tile_counts(n, 0, 1, 0, 0, bq, bk)
        assert causal_units(n, n_kv, bq, bk) == n_kv * (4 * vis + 5 * (-(-n // bq)))
    c = cache(n_slots=1, n_kv=n_kv, hd=hd, max_seq=hi)
    # accepted (then refused only for the missing workspace) up to the limit
    assert rc_prefill(c, n=lo, n_head=n_kv, ws_bytes=0) == fa.FA_EWORKSPACE
    assert rc_prefill(c, n=hi, n_head=n_kv, ws_bytes=0) == fa.FA_EUNSUPPORTED
    # a window keeps the schedule small at the same length
    assert rc_prefill(c, n=hi, n_head=n_kv, win=1024, ws_bytes=0) == fa.FA_EWORKSPACE


def test_paged_schedule_bound_is_refused():
    # the batch lives on the device, so the host bounds the schedule from
    # num_tokens, num_reqs and the block-table width
    c = paged(nb=1 << 16, bs=16, n_kv=8, hd=64)
    assert rc_paged(c, T=1 << 20, H=8, R=1, mb=1 << 16, ws_bytes=0) == fa.FA_EUNSUPPORTED
    assert rc_paged(c, T=8192, H=8, R=50, mb=1 << 13, ws_bytes=0) == fa.FA_EWORKSPACE


def test_decode_item_count_beyond_32_bits_is_refused():
    # decode work items (at most the plan's split cap per slot and kv head)
    # are counted in 32-bit integers
    _, cap, _ = fa.fa_decode_plan_params()
    big = ((1 << 31) - 1) // cap
    c = cache(n_slots=big + 1, n_kv=1)
    assert rc_decode(c, n_slots=big + 1, ws_bytes=0) == fa.FA_EUNSUPPORTED
    assert rc_decode(c, n_slots=big, ws_bytes=0) == fa.FA_EWORKSPACE


def test_decode_noalloc_validation():
    c = cache(n_slots=4, max_seq=100)

    def rc(c=c, q=FAKE, pos=FAKE, n_slots=1, hint=10, n_head=4, scale=0.1, out=FAKE):
        return fa.lib.fa_decode_noalloc(ctypes.byref(c) if c is not None else None, q, pos,
                                        n_slots, hint, n_head, 0, 0, scale, out, None, None)
    assert rc(c=None) == fa.FA_ENULL
    assert rc(n_slots=5) == fa.FA_EINVAL
    assert rc(hint=0) == fa.FA_EINVAL
    assert rc(scale=0.0) == fa.FA_EINVAL
    assert rc(n_head=3) == fa.FA_EINVAL
    assert rc(n_slots=0) == fa.FA_OK
    assert rc(q=0) == fa.FA_ENULL
    assert rc(pos=0) == fa.FA_ENULL
    assert rc(out=0) == fa.FA_ENULL
    # a call that needs more than the library's fixed scratch is refused
    big = cache(fmt=fa.FA_KV_Q4_0, n_slots=4096, n_kv=2, hd=256, max_seq=4)
    assert fa.fa_decode_workspace_bytes(big, 4096, 16, 4) > fa.DECODE_SCRATCH_BYTES
    assert rc(c=big, n_slots=4096, hint=4, n_head=16) == fa.FA_EWORKSPACE


def test_decode_q4_hilo_validation():
    def rc(c, n_slots=1, hint=10, n_head=4, ws_bytes=1 << 30):
        return fa.lib.fa_decode_q4_hilo(ctypes.byref(c), FAKE, FAKE, n_slots, hint, n_head, 0, 0,
                                        0.1, FAKE, FAKE, ws_bytes, None, None)
    # Q4_0 caches only, and none with an fp16 shadow
    assert rc(cache(fmt=fa.FA_KV_F32, n_slots=4)) == fa.FA_EUNSUPPORTED
    shadowed = cache(fmt=fa.FA_KV_Q4_0, n_slots=4)
    shadowed.shadow_sink, shadowed.k_sink, shadowed.v_sink = 4, FAKE, FAKE
    assert rc(shadowed) == fa.FA_EUNSUPPORTED
    c = cache(fmt=fa.FA_KV_Q4_0, n_slots=4)
    assert rc(c, n_slots=5) == fa.FA_EINVAL
    assert rc(c, n_head=3) == fa.FA_EINVAL
    assert rc(c, n_slots=0) == fa.FA_OK
    need = fa.fa_decode_workspace_bytes(c, 4, 4, 100)
    assert rc(c, n_slots=4, hint=100, ws_bytes=need - 1) == fa.FA_EWORKSPACE
