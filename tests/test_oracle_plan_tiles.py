"""Pins for the oracle's decode split plan and tile accounting.

Plan: Foundry cuda_kernels/attention.cu, fc_attn_dec_plan comment (about kps
keys per split, capped at cap splits, split length rounded up to the tile
width, live splits = ceil(L / split_len)). Tile predicate: the same page's
fc_attn_tile_in_window comment and the file header (tiles meeting neither
the sink nor the recent window are skipped before any staging; tiles past
the causal bound are never walked).

The plan is pinned by hand-worked examples and by a search-based
characterisation of what it computes (fewest kps-key pieces up to cap,
shortest tile-multiple split length that covers L with them, non-empty
splits); the tile counts by brute force
over every (query, key) pair on small shapes, and by the window workload's
closed-form pair count.
"""
import itertools

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("L,kps,cap,tile,want", [
    # worked by hand from the formula (live, n_splits, split_len)
    (100, 16, 64, 16, (7, 7, 16)),      # n=ceil(100/16)=7, len=ceil(100/7)=15->16, live=7
    (33, 4, 64, 16, (3, 9, 16)),        # n=9, len=4->16, live=3 < n
    (1, 16, 64, 16, (1, 1, 16)),        # a single key still gets one split
    (10000, 16, 64, 16, (63, 64, 160)),  # cap binds: len=ceil(10000/64)=157->160, live=63
    (4096, 512, 8, 64, (8, 8, 512)),
    (32768, 1024, 16, 64, (16, 16, 2048)),
    (5000, 1000, 4, 64, (4, 4, 1280)),  # n=5->4, len=1250->1280, live=4
])
def test_plan_worked_examples(L, kps, cap, tile, want):
    assert oracle.decode_plan(L, kps, cap, tile) == want


def test_plan_invariants():
    for L in list(range(1, 300)) + [4095, 4096, 4097, 32767, 32768]:
        for kps, cap, tile in [(16, 64, 16), (256, 8, 64), (1, 1000, 32), (64, 3, 64)]:
            live, n, sl = oracle.decode_plan(L, kps, cap, tile)
            assert 1 <= n <= cap and sl % tile == 0 and sl > 0
            assert 1 <= live <= n
            assert (live - 1) * sl < L <= live * sl      # live splits cover [0, L) exactly


def plan_by_search(L, kps, cap, tile):
    """The plan derived from what it is for, by search and enumeration rather
    than by its ceil-division formulas: n is the fewest kps-key pieces that
    hold L keys, at most cap; the split length is the shortest multiple of the
    tile with which n splits hold L keys; the live splits are those of the n
    that hold at least one key."""
    n = 1
    while n * kps < L and n < cap:
        n += 1
    sl = tile
    while n * sl < L:
        sl += tile
    live = sum(1 for i in range(n) if i * sl < L)
    return live, n, sl


def test_plan_matches_its_characterisation():
    Ls = list(range(1, 700)) + [1000, 4095, 4096, 4097, 10000, 32767, 32768, 32769, 40000]
    for L in Ls:
        for kps, cap, tile in [(64, 512, 64), (16, 64, 16), (256, 8, 64), (1, 1000, 32),
                               (64, 3, 64), (100, 7, 16)]:
            assert oracle.decode_plan(L, kps, cap, tile) == plan_by_search(L, kps, cap, tile), \
                (L, kps, cap, tile)


def test_plan_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.decode_plan(0, 16, 64, 16)


def brute_tiles(q0, q1, lo, hi, sink, win, bk):
    """Walk tiles; a tile is visited iff some query of [q0, q1] has some key of
    the tile in its key set, else skipped."""
    vis = skp = 0
    j0 = lo
    while j0 < hi and j0 <= q1:
        keys = range(j0, min(j0 + bk, hi))
        hit = any(oracle.key_in_set(j, p, sink, win)
                  for p in range(q0, q1 + 1) for j in keys)
        vis += hit
        skp += not hit
        j0 += bk
    return vis, skp


@pytest.mark.parametrize("sink,win", [(0, 0), (0, 1), (2, 3), (4, 9), (0, 20), (17, 2), (-3, 5)])
@pytest.mark.parametrize("bq,bk", [(1, 4), (3, 4), (4, 8), (16, 32)])
def test_tile_walk_matches_brute_force(sink, win, bq, bk):
    n, pos0 = 45, 6
    for b in range(0, n, bq):
        q0 = pos0 + b
        q1 = min(q0 + bq - 1, pos0 + n - 1)
        assert oracle.tile_walk(q0, q1, 0, q1 + 1, sink, win, bk) == \
            brute_tiles(q0, q1, 0, q1 + 1, sink, win, bk)
    for lo, hi in [(8, 24), (0, 5), (16, 51)]:
        q = 50
        assert oracle.tile_walk(q, q, lo, hi, sink, win, bk) == brute_tiles(q, q, lo, hi, sink, win, bk)


def test_prefill_tile_counts_sum_the_blocks():
    n, pos0, n_kv, sink, win, bq, bk = 77, 3, 2, 2, 10, 8, 16
    vis = skp = 0
    for b in range(0, n, bq):
        q0 = pos0 + b
        q1 = min(q0 + bq - 1, pos0 + n - 1)
        v_, s_ = brute_tiles(q0, q1, 0, q1 + 1, sink, win, bk)
        vis += v_
        skp += s_
    assert oracle.prefill_tile_counts(n, pos0, n_kv, sink, win, bq, bk) == (vis * n_kv, skp * n_kv)


def test_full_causal_prefill_never_skips_and_counts_triangle():
    # full causal from pos0 = 0 with bq = bk: block b walks b+1 tiles
    n, bq = 256, 16
    vis, skp = oracle.prefill_tile_counts(n, 0, 3, 0, 0, bq, bq)
    nb = n // bq
    assert skp == 0 and vis == 3 * nb * (nb + 1) // 2


def test_decode_tile_counts_sum_the_live_splits():
    pos = np.array([0, 15, 16, 100, 257, 1000], dtype=np.int32)
    kps, cap, bk, sink, win, n_kv = 64, 5, 16, 3, 40, 2
    vis = skp = 0
    for p in pos:
        live, n, sl = oracle.decode_plan(int(p) + 1, kps, cap, bk)
        for s in range(live):
            lo, hi = s * sl, min(int(p) + 1, (s + 1) * sl)
            v_, s_ = brute_tiles(int(p), int(p), lo, hi, sink, win, bk)
            vis += v_
            skp += s_
    assert oracle.decode_tile_counts(pos, n_kv, kps, cap, sink, win, bk) == (vis * n_kv, skp * n_kv)


def test_window_workload_pair_count_closed_form():
    # sink 4, win 1024 over 32768 positions: p+1 keys for p <= 1027, else 1028
    sink, win, n = 4, 1024, 32768
    pairs = sum(p + 1 for p in range(1028)) + (n - 1028) * 1028
    assert pairs == 33_157_626
    # the same count from the key-set predicate on a strided sample of rows
    for p in itertools.chain(range(0, 1100, 37), range(1027, 32768, 4093)):
        cnt = sum(oracle.key_in_set(j, p, sink, win) for j in range(p + 1))
        assert cnt == (p + 1 if p <= 1027 else 1028)
