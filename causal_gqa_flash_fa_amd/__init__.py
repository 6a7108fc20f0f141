"""Python binding of libfa: causal GQA flash attention for MI355X (gfx950).

Argument marshalling only. Every function here forwards to the C-ABI entry
point of the same name in libfa.so (declared in include/fa.h); all the
attention work runs in the HIP kernels behind it. PyTorch supplies device
memory and streams: tensors are passed by data pointer, streams by handle.

There is no fallback: if libfa.so is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK = 0
FA_EINVAL = -1
FA_ENULL = -2
FA_EUNSUPPORTED = -3
FA_EWORKSPACE = -4
FA_EHIP = -5
FA_ERANGE = -6
FA_EDEVICE = -7

FA_KV_F32 = 0
FA_KV_Q4_0 = 1

EXPORTS = [
    "fa_cache_row_bytes", "fa_cache_bytes", "fa_init", "fa_kv_append", "fa_kv_append_slots",
    "fa_prefill",
    "fa_prefill_tile_shape", "fa_prefill_workspace_bytes", "fa_decode_plan", "fa_decode_plan_params",
    "fa_decode_workspace_bytes", "fa_decode", "fa_decode_q4_hilo", "fa_decode_noalloc",
    "fa_strerror",
    "fa_last_hip_error",
    "fa_paged_append", "fa_paged_workspace_bytes", "fa_paged_attention", "fa_merge_attn_states",
    "fa_paged_decode", "fa_paged_decode_workspace_bytes",
]


SHADOW_SINK_MAX = 8
SHADOW_WIN_MAX = 256


class fa_cache(ctypes.Structure):
    """Mirror of `struct fa_cache` in include/fa.h."""
    _fields_ = [("format", ctypes.c_int), ("n_slots", ctypes.c_int),
                ("n_kv_head", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("max_seq", ctypes.c_int), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("shadow_sink", ctypes.c_int), ("shadow_win", ctypes.c_int),
                ("k_sink", ctypes.c_void_p), ("v_sink", ctypes.c_void_p),
                ("k_win", ctypes.c_void_p), ("v_win", ctypes.c_void_p),
                ("win_pos", ctypes.c_void_p)]


class fa_paged_cache(ctypes.Structure):
    """Mirror of `struct fa_paged_cache` in include/fa.h."""
    _fields_ = [("num_blocks", ctypes.c_int), ("block_size", ctypes.c_int),
                ("n_kv_head", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("block_stride", ctypes.c_longlong),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class FaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = f"{where}: {fa_strerror(code)} (code {code})"
        if code == FA_EHIP:
            msg += f" [{lib.fa_last_hip_error().decode()}]"
        super().__init__(msg)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python causal_gqa_flash_fa_amd/build.py` "
            "(there is no CPU fallback)")
    # torch first: its HIP runtime (soname libamdhip64.so.7) is then the one
    # libfa.so binds to. Loaded the other way round, torch pulls in a second
    # copy of the runtime, and its stream handles mean nothing to libfa's.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    PI = ctypes.POINTER(ctypes.c_int)
    C = ctypes.POINTER(fa_cache)
    L.fa_cache_row_bytes.argtypes = [I, I]
    L.fa_cache_row_bytes.restype = Z
    L.fa_cache_bytes.argtypes = [C]
    L.fa_cache_bytes.restype = Z
    L.fa_init.argtypes = []
    L.fa_init.restype = I
    L.fa_kv_append.argtypes = [C, I, I, I, P, P, P]
    L.fa_kv_append.restype = I
    L.fa_kv_append_slots.argtypes = [C, P, I, P, P, P]
    L.fa_kv_append_slots.restype = I
    L.fa_last_hip_error.argtypes = []
    L.fa_last_hip_error.restype = ctypes.c_char_p
    L.fa_prefill.argtypes = [C, I, P, I, I, I, I, I, F, P, P, Z, P, P]
    L.fa_prefill.restype = I
    L.fa_prefill_workspace_bytes.argtypes = [I, I, I, I]
    L.fa_prefill_workspace_bytes.restype = Z
    L.fa_prefill_tile_shape.argtypes = [I, I, I, PI, PI]
    L.fa_prefill_tile_shape.restype = I
    L.fa_decode_plan.argtypes = [I, PI, PI]
    L.fa_decode_plan.restype = I
    L.fa_decode_plan_params.argtypes = [PI, PI, PI]
    L.fa_decode_plan_params.restype = None
    L.fa_decode_workspace_bytes.argtypes = [C, I, I, I]
    L.fa_decode_workspace_bytes.restype = Z
    L.fa_decode.argtypes = [C, P, P, I, I, I, I, I, F, P, P, Z, P, P]
    L.fa_decode.restype = I
    L.fa_decode_q4_hilo.argtypes = [C, P, P, I, I, I, I, I, F, P, P, Z, P, P]
    L.fa_decode_q4_hilo.restype = I
    L.fa_decode_noalloc.argtypes = [C, P, P, I, I, I, I, I, F, P, P, P]
    L.fa_decode_noalloc.restype = I
    PC = ctypes.POINTER(fa_paged_cache)
    L.fa_paged_append.argtypes = [PC, P, P, P, I, P]
    L.fa_paged_append.restype = I
    L.fa_paged_workspace_bytes.argtypes = [I]
    L.fa_paged_workspace_bytes.restype = Z
    L.fa_paged_attention.argtypes = [PC, P, I, I, P, P, I, P, I, I, I, F, P, P, P, Z, P]
    L.fa_paged_attention.restype = I
    L.fa_paged_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    L.fa_paged_decode_workspace_bytes.restype = Z
    L.fa_paged_decode.argtypes = [PC, P, I, I, P, P, I, I, I, I, F, P, P, P, Z, P]
    L.fa_paged_decode.restype = I
    L.fa_merge_attn_states.argtypes = [P, P, P, P, P, P, I, I, I, I, P]
    L.fa_merge_attn_states.restype = I
    L.fa_strerror.argtypes = [I]
    L.fa_strerror.restype = ctypes.c_char_p
    return L


lib = _load()


def _ptr(x) -> int | None:
    """Device pointer of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    """hipStream_t handle: a torch stream, an int handle, or torch's current stream."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise FaError(rc, where)
    return rc


def fa_strerror(code: int) -> str:
    return lib.fa_strerror(code).decode()


def fa_cache_row_bytes(fmt: int, head_dim: int) -> int:
    return lib.fa_cache_row_bytes(fmt, head_dim)


def fa_cache_bytes(cache: fa_cache) -> int:
    return lib.fa_cache_bytes(ctypes.byref(cache))


def fa_init() -> None:
    _check(lib.fa_init(), "fa_init")


def fa_kv_append(cache: fa_cache, slot: int, pos0: int, n: int, k_new, v_new,
                 stream=None) -> None:
    _check(lib.fa_kv_append(ctypes.byref(cache), slot, pos0, n, _ptr(k_new), _ptr(v_new),
                            _stream(stream)), "fa_kv_append")


def fa_kv_append_slots(cache: fa_cache, d_pos, n_slots: int, k_new, v_new,
                       stream=None) -> None:
    _check(lib.fa_kv_append_slots(ctypes.byref(cache), _ptr(d_pos), n_slots, _ptr(k_new),
                                  _ptr(v_new), _stream(stream)), "fa_kv_append_slots")


def fa_prefill(cache: fa_cache, slot: int, q, pos0: int, n: int, n_head: int,
               attn_sink: int, attn_win: int, scale: float, out, ws, ws_bytes: int,
               tile_stats=None, stream=None) -> None:
    _check(lib.fa_prefill(ctypes.byref(cache), slot, _ptr(q), pos0, n, n_head, attn_sink,
                          attn_win, scale, _ptr(out), _ptr(ws), ws_bytes, _ptr(tile_stats),
                          _stream(stream)), "fa_prefill")


def fa_prefill_workspace_bytes(n: int, n_head: int, n_kv_head: int, head_dim: int) -> int:
    return lib.fa_prefill_workspace_bytes(n, n_head, n_kv_head, head_dim)


def fa_prefill_tile_shape(n_head: int, n_kv_head: int, head_dim: int) -> tuple[int, int]:
    bq, bk = ctypes.c_int(), ctypes.c_int()
    _check(lib.fa_prefill_tile_shape(n_head, n_kv_head, head_dim, ctypes.byref(bq),
                                     ctypes.byref(bk)), "fa_prefill_tile_shape")
    return bq.value, bk.value


def fa_decode_plan(seq_len: int) -> tuple[int, int, int]:
    """(live, n_splits, split_len)."""
    n, sl = ctypes.c_int(), ctypes.c_int()
    live = _check(lib.fa_decode_plan(seq_len, ctypes.byref(n), ctypes.byref(sl)),
                  "fa_decode_plan")
    return live, n.value, sl.value


def fa_decode_plan_params() -> tuple[int, int, int]:
    """(kps, cap, key_tile)."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib.fa_decode_plan_params(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def fa_decode_workspace_bytes(cache: fa_cache, n_slots: int, n_head: int, max_ctx: int) -> int:
    return lib.fa_decode_workspace_bytes(ctypes.byref(cache), n_slots, n_head, max_ctx)


def fa_decode(cache: fa_cache, q, d_pos, n_slots: int, max_ctx_hint: int, n_head: int,
              attn_sink: int, attn_win: int, scale: float, out, ws, ws_bytes: int,
              tile_stats=None, stream=None) -> None:
    _check(lib.fa_decode(ctypes.byref(cache), _ptr(q), _ptr(d_pos), n_slots, max_ctx_hint,
                         n_head, attn_sink, attn_win, scale, _ptr(out), _ptr(ws), ws_bytes,
                         _ptr(tile_stats), _stream(stream)), "fa_decode")


def fa_decode_q4_hilo(cache: fa_cache, q, d_pos, n_slots: int, max_ctx_hint: int, n_head: int,
                      attn_sink: int, attn_win: int, scale: float, out, ws, ws_bytes: int,
                      tile_stats=None, stream=None) -> None:
    _check(lib.fa_decode_q4_hilo(ctypes.byref(cache), _ptr(q), _ptr(d_pos), n_slots,
                                 max_ctx_hint, n_head, attn_sink, attn_win, scale, _ptr(out),
                                 _ptr(ws), ws_bytes, _ptr(tile_stats), _stream(stream)),
           "fa_decode_q4_hilo")


# Bytes of the library's per-GPU decode scratch (fa_decode_noalloc).
DECODE_SCRATCH_BYTES = 32 << 20


def fa_decode_noalloc(cache: fa_cache, q, d_pos, n_slots: int, max_ctx_hint: int, n_head: int,
                      attn_sink: int, attn_win: int, scale: float, out, tile_stats=None,
                      stream=None) -> None:
    _check(lib.fa_decode_noalloc(ctypes.byref(cache), _ptr(q), _ptr(d_pos), n_slots,
                                 max_ctx_hint, n_head, attn_sink, attn_win, scale, _ptr(out),
                                 _ptr(tile_stats), _stream(stream)), "fa_decode_noalloc")


def make_cache(fmt: int, n_slots: int, n_kv_head: int, head_dim: int, max_seq: int,
               device="cuda"):
    """Allocate K and V cache tensors with torch and describe them.

    Returns (fa_cache, k_tensor, v_tensor); keep the tensors alive as long as
    the struct is used. Memory comes from torch's allocator: libfa never
    allocates.
    """
    import torch
    probe = fa_cache(fmt, n_slots, n_kv_head, head_dim, max_seq, None, None)
    nbytes = lib.fa_cache_bytes(ctypes.byref(probe))
    if nbytes == 0:
        raise FaError(FA_EINVAL, "make_cache")
    k = torch.empty(nbytes, dtype=torch.uint8, device=device)
    v = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return fa_cache(fmt, n_slots, n_kv_head, head_dim, max_seq, k.data_ptr(), v.data_ptr()), k, v


def add_shadow(cache: fa_cache, sink: int, win: int, device="cuda"):
    """Allocate the fp16 sink / recent-window shadow of a Q4_0 cache with torch
    and record it in `cache` (win_pos filled with -1: no ring row holds a
    position yet). Returns the tensors (k_sink, v_sink, k_win, v_win, win_pos);
    keep them alive as long as the struct is used."""
    import torch
    n, h, d = cache.n_slots, cache.n_kv_head, cache.head_dim
    ks = torch.zeros((n, h, SHADOW_SINK_MAX, d), dtype=torch.float16, device=device)
    vs = torch.zeros_like(ks)
    kw = torch.zeros((n, h, SHADOW_WIN_MAX, d), dtype=torch.float16, device=device)
    vw = torch.zeros_like(kw)
    wp = torch.full((n, SHADOW_WIN_MAX), -1, dtype=torch.int32, device=device)
    cache.shadow_sink, cache.shadow_win = sink, win
    cache.k_sink, cache.v_sink = ks.data_ptr(), vs.data_ptr()
    cache.k_win, cache.v_win = kw.data_ptr(), vw.data_ptr()
    cache.win_pos = wp.data_ptr()
    return ks, vs, kw, vw, wp


def fa_paged_append(cache: fa_paged_cache, k, v, slot_mapping, num_slots: int,
                    stream=None) -> None:
    _check(lib.fa_paged_append(ctypes.byref(cache), _ptr(k), _ptr(v), _ptr(slot_mapping),
                               num_slots, _stream(stream)), "fa_paged_append")


def fa_paged_workspace_bytes(head_dim: int) -> int:
    return lib.fa_paged_workspace_bytes(head_dim)


def fa_paged_attention(cache: fa_paged_cache, q, num_tokens: int, n_head: int,
                       query_start_loc, seq_lens, num_reqs: int, block_table,
                       max_blocks_per_seq: int, window_left: int, window_right: int,
                       scale: float, out, lse, ws, ws_bytes: int, stream=None) -> None:
    _check(lib.fa_paged_attention(ctypes.byref(cache), _ptr(q), num_tokens, n_head,
                                  _ptr(query_start_loc), _ptr(seq_lens), num_reqs,
                                  _ptr(block_table), max_blocks_per_seq, window_left,
                                  window_right, scale, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                  _stream(stream)), "fa_paged_attention")


def fa_paged_decode_workspace_bytes(num_reqs: int, n_head: int, n_kv_head: int, head_dim: int,
                                    max_seq_len_hint: int) -> int:
    return lib.fa_paged_decode_workspace_bytes(num_reqs, n_head, n_kv_head, head_dim,
                                               max_seq_len_hint)


def fa_paged_decode(cache: fa_paged_cache, q, num_reqs: int, n_head: int, seq_lens, block_table,
                    max_blocks_per_seq: int, max_seq_len_hint: int, window_left: int,
                    window_right: int, scale: float, out, lse, ws, ws_bytes: int,
                    stream=None) -> None:
    _check(lib.fa_paged_decode(ctypes.byref(cache), _ptr(q), num_reqs, n_head, _ptr(seq_lens),
                               _ptr(block_table), max_blocks_per_seq, max_seq_len_hint,
                               window_left, window_right, scale, _ptr(out), _ptr(lse), _ptr(ws),
                               ws_bytes, _stream(stream)), "fa_paged_decode")


def fa_merge_attn_states(out, out_lse, prefix_out, prefix_lse, suffix_out, suffix_lse,
                         num_tokens: int, n_head: int, head_dim: int,
                         prefill_tokens_with_context: int = -1, stream=None) -> None:
    _check(lib.fa_merge_attn_states(_ptr(out), _ptr(out_lse), _ptr(prefix_out),
                                    _ptr(prefix_lse), _ptr(suffix_out), _ptr(suffix_lse),
                                    num_tokens, n_head, head_dim, prefill_tokens_with_context,
                                    _stream(stream)), "fa_merge_attn_states")


def make_paged_cache(num_blocks: int, block_size: int, n_kv_head: int, head_dim: int,
                     device="cuda", interleaved: bool = False):
    """Allocate a paged fp32 cache with torch and describe it.

    interleaved=False: separate k and v tensors [num_blocks][block_size][n_kv][hd].
    interleaved=True: one [num_blocks][2][block_size][n_kv][hd] tensor whose two
    halves are k and v (block stride 2 * block_size * n_kv * hd).
    Returns (fa_paged_cache, k_view, v_view), the views shaped
    [num_blocks][block_size][n_kv][hd]; keep them alive as long as the struct is used.
    """
    import torch
    shape = (num_blocks, block_size, n_kv_head, head_dim)
    if interleaved:
        kv = torch.empty((num_blocks, 2) + shape[1:], dtype=torch.float32, device=device)
        k, v = kv[:, 0], kv[:, 1]
        stride = 2 * block_size * n_kv_head * head_dim
    else:
        k = torch.empty(shape, dtype=torch.float32, device=device)
        v = torch.empty(shape, dtype=torch.float32, device=device)
        stride = 0
    return fa_paged_cache(num_blocks, block_size, n_kv_head, head_dim, stride, k.data_ptr(),
                          v.data_ptr()), k, v
