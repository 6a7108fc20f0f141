"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module only draws random numbers and describes shapes. It holds none of
the attention arithmetic, so both the CPU oracle (``oracle/``) and the HIP
library (``causal_gqa_flash_fa_amd``) can be fed from it without sharing code.

Recipe: numpy ``Generator(PCG64(seed))`` standard normal, float32, with
seed = 20261202 + 100 * config_index + tensor_id, where tensor_id is
0 for q, 1 for k, 2 for v, 3 for decode context lengths (paged: the request
draw) and 4 for the paged page order; decode K/V of slot s (paged: request s)
add 1000 * s so slots can be generated one at a time.

The shapes follow the workloads the Foundry attention.cu page describes
(file header: 8k-token batched prefill of a G=8, head_dim=256 model; the
StreamingLLM sink + recent-window key set; the multi-user slots decode
section). q and k stand in for post-QK-norm+RoPE rows, v for raw value rows.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEED_BASE = 20261202

KV_F32 = 0
KV_Q4_0 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int            # position in the list below; part of every seed
    name: str
    kind: str             # "prefill" or "decode"
    n_head: int
    n_kv_head: int
    head_dim: int
    kv_format: int        # KV_F32 or KV_Q4_0
    n: int = 0            # prefill: query rows in the call
    pos0: int = 0         # prefill: absolute position of row 0
    attn_sink: int = 0
    attn_win: int = 0
    max_seq: int = 0
    n_slots: int = 1      # decode: sequence slots
    ctx_lo: int = 0       # decode: context length range, inclusive
    ctx_hi: int = 0
    shadow_sink: int = 0  # Q4_0: fp16 shadow of the first positions ...
    shadow_win: int = 0   # ... and of the recent window (0, 0: no shadow)
    block_size: int = 0   # paged: rows per page (n = query-token budget of the batch)

    @property
    def group(self) -> int:
        return self.n_head // self.n_kv_head

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = [
    Workload(0, "tiny-prefill-128", "prefill", 4, 1, 64, KV_F32, n=128, max_seq=128),
    Workload(1, "prefill-f32kv-2k", "prefill", 16, 2, 256, KV_F32, n=2048, max_seq=2048),
    Workload(2, "prefill-q4kv-8k", "prefill", 16, 2, 256, KV_Q4_0, n=8192, max_seq=8192),
    Workload(3, "window-prefill-32k", "prefill", 16, 2, 256, KV_F32, n=32768,
             attn_sink=4, attn_win=1024, max_seq=32768),
    Workload(4, "decode-64slots-q4kv", "decode", 16, 2, 256, KV_Q4_0, n_slots=64,
             ctx_lo=4096, ctx_hi=32768, max_seq=32768),
]
# The Q4_0 workloads again with the fp16 sink + recent-window shadow (the
# Foundry page's 4-position sink and its 256-row window ring), on the same
# seeded inputs (same index).
SHADOW_WORKLOADS = [
    dataclasses.replace(WORKLOADS[2], name="prefill-q4kv-8k-shadow", shadow_sink=4,
                        shadow_win=256),
    dataclasses.replace(WORKLOADS[4], name="decode-64slots-q4kv-shadow", shadow_sink=4,
                        shadow_win=256),
]
# The 64-slot decode again over an fp32 cache (same seeded inputs): at
# 4 FLOP/B it is bound by HBM, not by fp32 MFMA, so it measures the decode
# kernel's memory path against the bandwidth roofline.
F32_DECODE_WORKLOADS = [
    dataclasses.replace(WORKLOADS[4], name="decode-64slots-f32kv", kv_format=KV_F32),
]
# A varlen batch over a paged fp32 cache (the vLLM-style PagedAttention of the
# vllm-cpp-sys ops page): requests are drawn until 8192 query tokens are
# used, each either a decode step (one token, probability 1/2) or a prefill
# chunk of 64..1024 tokens, after a context of 0..8192 rows; pages of 16 rows
# are scattered over the cache in a seeded order.
PAGED_WORKLOADS = [
    Workload(5, "paged-varlen-8k", "paged", 16, 2, 256, KV_F32, n=8192, ctx_hi=8192,
             block_size=16),
]
# The 64-slot decode again (same seeded inputs) over a paged fp32 cache of
# 16-row pages in a seeded random order: one decode token per request.
PAGED_WORKLOADS.append(
    dataclasses.replace(WORKLOADS[4], name="paged-decode-64req-f32kv", kind="paged_decode",
                        kv_format=KV_F32, block_size=16))
BY_NAME = {w.name: w for w in
           WORKLOADS + SHADOW_WORKLOADS + F32_DECODE_WORKLOADS + PAGED_WORKLOADS}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(seed: int, shape) -> np.ndarray:
    """float32 standard normal of the given shape from PCG64(seed)."""
    return _rng(seed).standard_normal(size=shape, dtype=np.float32)


def seed_of(w: Workload, tensor_id: int, slot: int = 0) -> int:
    return SEED_BASE + 100 * w.index + tensor_id + 1000 * slot


def prefill_q(w: Workload, n: int | None = None) -> np.ndarray:
    """q [n][n_head][head_dim]; the first n rows of the workload's q."""
    n = w.n if n is None else n
    full = normal(seed_of(w, 0), (w.n, w.n_head, w.head_dim))
    return np.ascontiguousarray(full[:n])


def prefill_kv(w: Workload, n: int | None = None):
    """k_new, v_new [n][n_kv_head][head_dim] for the rows appended before the call."""
    rows = w.pos0 + w.n
    n = rows if n is None else n
    k = normal(seed_of(w, 1), (rows, w.n_kv_head, w.head_dim))[:n]
    v = normal(seed_of(w, 2), (rows, w.n_kv_head, w.head_dim))[:n]
    return np.ascontiguousarray(k), np.ascontiguousarray(v)


def decode_ctx(w: Workload) -> np.ndarray:
    """Per-slot context lengths, uniform integers in [ctx_lo, ctx_hi]."""
    return _rng(seed_of(w, 3)).integers(w.ctx_lo, w.ctx_hi, size=w.n_slots,
                                        endpoint=True).astype(np.int32)


def decode_q(w: Workload) -> np.ndarray:
    """q [n_slots][n_head][head_dim], one query row per slot."""
    return normal(seed_of(w, 0), (w.n_slots, w.n_head, w.head_dim))


def decode_kv(w: Workload, slot: int, ctx: int):
    """k, v [ctx][n_kv_head][head_dim] rows of one slot (positions 0..ctx-1)."""
    k = normal(seed_of(w, 1, slot), (ctx, w.n_kv_head, w.head_dim))
    v = normal(seed_of(w, 2, slot), (ctx, w.n_kv_head, w.head_dim))
    return k, v


def custom_prefill(seed: int, n: int, pos0: int, n_head: int, n_kv_head: int,
                   head_dim: int):
    """Ad-hoc prefill case for sweeps: q [n][H][hd], k/v [pos0+n][Hkv][hd]."""
    q = normal(seed, (n, n_head, head_dim))
    k = normal(seed + 1, (pos0 + n, n_kv_head, head_dim))
    v = normal(seed + 2, (pos0 + n, n_kv_head, head_dim))
    return q, k, v


def paged_requests(w: Workload) -> list[tuple[int, int]]:
    """(context rows before the chunk, query tokens) per request."""
    rng = _rng(seed_of(w, 3))
    reqs, budget = [], w.n
    while budget > 0:
        qlen = 1 if rng.random() < 0.5 else int(rng.integers(64, 1024, endpoint=True))
        qlen = min(qlen, budget)
        ctx = int(rng.integers(0, w.ctx_hi, endpoint=True))
        reqs.append((ctx, qlen))
        budget -= qlen
    return reqs


def paged_layout(w: Workload):
    """Block table and cache size of the batch: request r's pages, in a seeded
    random order over the cache. Returns (table int32 [R][max_blocks],
    num_blocks, seq_lens int32 [R], query_start_loc int32 [R+1])."""
    reqs = paged_requests(w)
    bs = w.block_size
    seq = np.array([c + n for c, n in reqs], np.int32)
    pages = (seq + bs - 1) // bs
    num_blocks = int(pages.sum())
    perm = _rng(seed_of(w, 4)).permutation(num_blocks).astype(np.int32)
    table = np.zeros((len(reqs), int(pages.max())), np.int32)
    at = 0
    for r, n in enumerate(pages):
        table[r, :n] = perm[at:at + n]
        at += n
    qsl = np.zeros(len(reqs) + 1, np.int32)
    qsl[1:] = np.cumsum([n for _, n in reqs])
    return table, num_blocks, seq, qsl


def paged_slots(table: np.ndarray, r: int, rows: np.ndarray, block_size: int) -> np.ndarray:
    """Cache slot (page * block_size + row in page) of key rows `rows` of request r."""
    return (table[r, rows // block_size].astype(np.int64) * block_size + rows % block_size)


def paged_q(w: Workload) -> np.ndarray:
    """q [tokens][n_head][head_dim] of the whole batch."""
    return normal(seed_of(w, 0), (w.n, w.n_head, w.head_dim))


def paged_kv(w: Workload, r: int, seq: int):
    """k, v [seq][n_kv_head][head_dim] rows of request r (positions 0..seq-1)."""
    k = normal(seed_of(w, 1, r), (seq, w.n_kv_head, w.head_dim))
    v = normal(seed_of(w, 2, r), (seq, w.n_kv_head, w.head_dim))
    return k, v


def decode_page_table(w: Workload, ctx: np.ndarray):
    """Pages of a decode batch whose request s holds ctx[s] rows: request by
    request, consecutive page slots of a seeded permutation of the cache.
    Returns (table int32 [R][max_blocks], num_blocks)."""
    bs = w.block_size
    pages = (ctx.astype(np.int64) + bs - 1) // bs
    num_blocks = int(pages.sum())
    perm = _rng(seed_of(w, 4)).permutation(num_blocks).astype(np.int32)
    table = np.zeros((len(ctx), int(pages.max())), np.int32)
    at = 0
    for r, n in enumerate(pages):
        table[r, :n] = perm[at:at + n]
        at += int(n)
    return table, num_blocks
