"""Python view of the CPU oracle (``oracle/oracle.c``) through ctypes.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``. The HIP library never imports it,
and it imports nothing from the HIP library. Argument conventions and the
passages each function follows are documented in ``oracle/oracle.h``.
"""
from __future__ import annotations

import concurrent.futures
import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "liboracle.so")
SRC_PATH = os.path.join(_DIR, "oracle.c")

# No fast-math and no FP contraction: the fp32 quantiser must round each step.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(quiet: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc; returns the library path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC_PATH, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=quiet)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, u16, dbl, flt = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint16,
                                   ctypes.c_double, ctypes.c_float)
        L.oracle_f32_to_f16.argtypes = [flt]
        L.oracle_f32_to_f16.restype = u16
        L.oracle_f16_to_f32.argtypes = [u16]
        L.oracle_f16_to_f32.restype = flt
        L.oracle_q4_quantize_rows.argtypes = [P, i64, i32, P]
        L.oracle_q4_dequantize_rows.argtypes = [P, i64, i32, P]
        L.oracle_key_in_set.argtypes = [i32, i32, i32, i32]
        L.oracle_key_in_set.restype = i32
        L.oracle_gqa_rows.argtypes = [P, P, i32, P, P, i32, i32, i32, i32, i32, i32,
                                      dbl, P, i64, P]
        L.oracle_gqa_rows.restype = i32
        L.oracle_key_is_fp16.argtypes = [i32, i32, i32, i32, i32]
        L.oracle_key_is_fp16.restype = i32
        L.oracle_gqa_rows_shadow.argtypes = [P, P, i32, P, P, P, P, i32, i32, i32, i32, i32,
                                             i32, dbl, i32, i32, i32, P, i64, P]
        L.oracle_gqa_rows_shadow.restype = i32
        L.oracle_gqa_lse.argtypes = [P, P, i32, P, i32, i32, i32, i32, i32, i32, dbl, P, i64, P]
        L.oracle_gqa_lse.restype = i32
        L.oracle_decode_plan.argtypes = [i32, i32, i32, i32, P, P]
        L.oracle_decode_plan.restype = i32
        L.oracle_tile_walk.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P]
        L.oracle_prefill_tile_counts.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P]
        L.oracle_decode_tile_counts.argtypes = [P, i32, i32, i32, i32, i32, i32, i32, P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def f32_to_f16_bits(x: float) -> int:
    return int(lib().oracle_f32_to_f16(float(x)))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().oracle_f16_to_f32(int(h)))


def q4_row_bytes(head_dim: int) -> int:
    return head_dim // 32 * 18


def q4_quantize(x: np.ndarray) -> np.ndarray:
    """float32 [..., head_dim] -> uint8 [..., head_dim/32*18] Q4_0 rows."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    hd = x.shape[-1]
    if hd % 32:
        raise ValueError("head_dim must be a multiple of 32")
    n_rows = x.size // hd
    out = np.empty(x.shape[:-1] + (q4_row_bytes(hd),), dtype=np.uint8)
    lib().oracle_q4_quantize_rows(_ptr(x), n_rows, hd, _ptr(out))
    return out


def q4_dequantize(rows: np.ndarray, head_dim: int) -> np.ndarray:
    """uint8 [..., head_dim/32*18] -> float32 [..., head_dim]."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    rb = q4_row_bytes(head_dim)
    if rows.shape[-1] != rb:
        raise ValueError("row bytes do not match head_dim")
    n_rows = rows.size // rb
    out = np.empty(rows.shape[:-1] + (head_dim,), dtype=np.float32)
    lib().oracle_q4_dequantize_rows(_ptr(rows), n_rows, head_dim, _ptr(out))
    return out


def key_in_set(j: int, p: int, attn_sink: int, attn_win: int) -> bool:
    return bool(lib().oracle_key_in_set(j, p, attn_sink, attn_win))


def gqa_rows(q: np.ndarray, q_pos, k: np.ndarray, v: np.ndarray, attn_sink: int,
             attn_win: int, scale: float, sel=None, threads: int = 1) -> np.ndarray:
    """Attention rows in float64.

    q [n_q][n_head][hd] f32; q_pos [n_q]; k, v [n_kv][kv_rows][hd] f32.
    sel: None (all n_q*n_head rows) or flat indices qi*n_head + h.
    threads > 1 splits the selected rows over worker threads (each call into
    the library is single-threaded and releases the GIL).
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n_q, n_head, hd = q.shape
    n_kv, kv_rows, hd2 = k.shape
    if hd2 != hd or v.shape != k.shape or q_pos.shape != (n_q,):
        raise ValueError("shape mismatch")
    if sel is None:
        sel = np.arange(n_q * n_head, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    out = np.empty((sel.size, hd), dtype=np.float64)

    def run(lo: int, hi: int) -> None:
        if hi <= lo:
            return
        part = sel[lo:hi]
        rc = lib().oracle_gqa_rows(_ptr(q), _ptr(q_pos), n_q, _ptr(k), _ptr(v), kv_rows,
                                   n_head, n_kv, hd, attn_sink, attn_win, float(scale),
                                   _ptr(part), part.size, out[lo:hi].ctypes.data)
        if rc != 0:
            raise ValueError("oracle_gqa_rows rejected its arguments")

    if threads <= 1 or sel.size < 2:
        run(0, sel.size)
    else:
        bounds = np.linspace(0, sel.size, threads + 1).astype(int)
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda i: run(bounds[i], bounds[i + 1]), range(threads)))
    return out


def key_is_fp16(s: int, p: int, shadow_sink: int, shadow_win: int, live_lo: int) -> bool:
    return bool(lib().oracle_key_is_fp16(s, p, shadow_sink, shadow_win, live_lo))


def f16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to binary16 (round-to-nearest-even), as float32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def gqa_rows_shadow(q: np.ndarray, q_pos, k: np.ndarray, v: np.ndarray, k16: np.ndarray,
                    v16: np.ndarray, attn_sink: int, attn_win: int, scale: float,
                    shadow_sink: int, shadow_win: int, live_lo: int, sel=None,
                    threads: int = 1) -> np.ndarray:
    """gqa_rows where key s of a query at p comes from k16/v16 (the fp16
    shadow, as float32) when key_is_fp16(s, p, ...) and from k/v (the
    dequantised Q4_0 body) otherwise. All four are [n_kv][kv_rows][hd]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k, v, k16, v16 = (np.ascontiguousarray(a, dtype=np.float32) for a in (k, v, k16, v16))
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n_q, n_head, hd = q.shape
    n_kv, kv_rows, hd2 = k.shape
    if hd2 != hd or q_pos.shape != (n_q,) or any(a.shape != k.shape for a in (v, k16, v16)):
        raise ValueError("shape mismatch")
    if sel is None:
        sel = np.arange(n_q * n_head, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    out = np.empty((sel.size, hd), dtype=np.float64)

    def run(lo: int, hi: int) -> None:
        if hi <= lo:
            return
        part = sel[lo:hi]
        rc = lib().oracle_gqa_rows_shadow(_ptr(q), _ptr(q_pos), n_q, _ptr(k), _ptr(v), _ptr(k16),
                                          _ptr(v16), kv_rows, n_head, n_kv, hd, attn_sink,
                                          attn_win, float(scale), shadow_sink, shadow_win,
                                          live_lo, _ptr(part), part.size,
                                          out[lo:hi].ctypes.data)
        if rc != 0:
            raise ValueError("oracle_gqa_rows_shadow rejected its arguments")

    if threads <= 1 or sel.size < 2:
        run(0, sel.size)
    else:
        bounds = np.linspace(0, sel.size, threads + 1).astype(int)
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda i: run(bounds[i], bounds[i + 1]), range(threads)))
    return out


def gqa_lse(q: np.ndarray, q_pos, k: np.ndarray, attn_sink: int, attn_win: int, scale: float,
            sel=None) -> np.ndarray:
    """Natural-log log-sum-exp of each row's scaled scores over its key set,
    float64 [len(sel)] (all n_q * n_head rows by default, flat index qi*H + h)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n_q, n_head, hd = q.shape
    n_kv, kv_rows, _ = k.shape
    if sel is None:
        sel = np.arange(n_q * n_head, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    out = np.empty(sel.size, dtype=np.float64)
    rc = lib().oracle_gqa_lse(_ptr(q), _ptr(q_pos), n_q, _ptr(k), kv_rows, n_head, n_kv, hd,
                              attn_sink, attn_win, float(scale), _ptr(sel), sel.size,
                              out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_gqa_lse rejected its arguments")
    return out


def paged_rows(cache: np.ndarray, block_row, seq_len: int) -> np.ndarray:
    """Contiguous [n_kv][seq_len][hd] rows of one request from a paged cache
    [num_blocks][block_size][n_kv][hd] ([VT] PagedAttention): key position j
    lives in block block_row[j // block_size] at offset j % block_size."""
    bs = cache.shape[1]
    j = np.arange(seq_len)
    blocks = np.asarray(block_row)[j // bs]
    return np.ascontiguousarray(cache[blocks, j % bs].transpose(1, 0, 2))


def merge_attn_states(prefix_out, prefix_lse, suffix_out, suffix_lse,
                      prefill_tokens_with_context: int = -1):
    """[VT] MergeAttnStates on float64 arrays: outputs [T][H][D], lse [H][T].
    Two results over disjoint key sets combine by their log-sum-exps; +inf LSE
    counts as -inf; if both are -inf the prefix output and -inf are kept;
    tokens at index >= prefill_tokens_with_context (when >= 0) take the suffix
    verbatim."""
    po, so = np.asarray(prefix_out, np.float64), np.asarray(suffix_out, np.float64)
    pl = np.where(np.isposinf(prefix_lse), -np.inf, np.asarray(prefix_lse, np.float64))
    sl = np.where(np.isposinf(suffix_lse), -np.inf, np.asarray(suffix_lse, np.float64))
    T, H, D = po.shape
    out, lse = np.empty_like(po), np.empty((H, T))
    for t in range(T):
        for h in range(H):
            if 0 <= prefill_tokens_with_context <= t:
                out[t, h], lse[h, t] = so[t, h], sl[h, t]
                continue
            a, b = pl[h, t], sl[h, t]
            if a == -np.inf and b == -np.inf:
                out[t, h], lse[h, t] = po[t, h], -np.inf
                continue
            m = max(a, b)
            pa, pb = np.exp(a - m), np.exp(b - m)
            out[t, h] = po[t, h] * (pa / (pa + pb)) + so[t, h] * (pb / (pa + pb))
            lse[h, t] = np.log(pa + pb) + m
    return out, lse


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos0: int,
            attn_sink: int, attn_win: int, scale: float, sel=None,
            threads: int = 1) -> np.ndarray:
    """Prefill rows t = 0..n-1 at positions pos0 + t.

    k_cache, v_cache [n_kv][max_seq][hd] f32 holding rows [0, pos0 + n).
    Returns [n][n_head][hd] float64 (or [len(sel)][hd] when sel is given).
    """
    n, n_head, hd = q.shape
    out = gqa_rows(q, np.arange(pos0, pos0 + n, dtype=np.int32), k_cache, v_cache,
                   attn_sink, attn_win, scale, sel=sel, threads=threads)
    return out if sel is not None else out.reshape(n, n_head, hd)


def decode_plan(seq_len: int, kps: int, cap: int, tile: int):
    """(live, n_splits, split_len) of the decode split plan."""
    n = ctypes.c_int()
    sl = ctypes.c_int()
    live = lib().oracle_decode_plan(seq_len, kps, cap, tile, ctypes.byref(n), ctypes.byref(sl))
    if live < 0:
        raise ValueError("bad plan arguments")
    return live, n.value, sl.value


def tile_walk(q0, q1, lo, hi, attn_sink, attn_win, bk):
    vis = ctypes.c_uint64(0)
    skp = ctypes.c_uint64(0)
    lib().oracle_tile_walk(q0, q1, lo, hi, attn_sink, attn_win, bk,
                           ctypes.byref(vis), ctypes.byref(skp))
    return vis.value, skp.value


def prefill_tile_counts(n, pos0, n_kv_head, attn_sink, attn_win, bq, bk):
    vis = ctypes.c_uint64(0)
    skp = ctypes.c_uint64(0)
    lib().oracle_prefill_tile_counts(n, pos0, n_kv_head, attn_sink, attn_win, bq, bk,
                                     ctypes.byref(vis), ctypes.byref(skp))
    return vis.value, skp.value


def decode_tile_counts(pos, n_kv_head, kps, cap, attn_sink, attn_win, bk):
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    vis = ctypes.c_uint64(0)
    skp = ctypes.c_uint64(0)
    lib().oracle_decode_tile_counts(_ptr(pos), pos.size, n_kv_head, kps, cap, attn_sink,
                                    attn_win, bk, ctypes.byref(vis), ctypes.byref(skp))
    return vis.value, skp.value
