"""Host-side logic that needs no GPU: the bench's command-line contract and
FLOP counting, and the structure of the seeded workloads (page tables,
request draws) that both the tests and the bench build on."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                    # no JSON line


@pytest.mark.parametrize("n,pos0,sink,win", [
    (1, 0, 0, 0), (37, 0, 0, 0), (20, 15, 0, 0), (40, 0, 3, 7), (25, 30, 0, 1), (50, 5, 60, 10),
])
def test_keyset_pairs_is_the_brute_force_count(n, pos0, sink, win):
    want = sum(1 for p in range(pos0, pos0 + n) for j in range(p + 1)
               if oracle.key_in_set(j, p, sink, win))
    assert bench.keyset_pairs(n, pos0, sink, win) == want


def test_paged_flops_counts_each_request_at_its_positions():
    w = workloads.BY_NAME["paged-varlen-8k"]
    reqs = workloads.paged_requests(w)
    pairs = sum((c + 1 + c + n) * n // 2 for c, n in reqs)      # keys c+1 .. c+n per token
    assert bench.paged_flops(w) == 4.0 * w.head_dim * w.n_head * pairs


def test_paged_request_draw_uses_the_token_budget():
    w = workloads.BY_NAME["paged-varlen-8k"]
    reqs = workloads.paged_requests(w)
    assert sum(n for _, n in reqs) == w.n
    assert all(n >= 1 and 0 <= c <= w.ctx_hi for c, n in reqs)
    assert reqs == workloads.paged_requests(w)                  # seeded: the same every time


def test_paged_layout_pages_are_disjoint_and_cover_every_row():
    w = workloads.BY_NAME["paged-varlen-8k"]
    table, num_blocks, seq, qsl = workloads.paged_layout(w)
    reqs = workloads.paged_requests(w)
    assert qsl[0] == 0 and qsl[-1] == w.n and np.all(np.diff(qsl) >= 0)
    used = []
    for r, (c, n) in enumerate(reqs):
        assert seq[r] == c + n
        pages = table[r, :(seq[r] + w.block_size - 1) // w.block_size]
        used.extend(pages.tolist())
        slots = workloads.paged_slots(table, r, np.arange(seq[r]), w.block_size)
        assert len(set(slots.tolist())) == seq[r]
    assert sorted(used) == list(range(num_blocks))             # a permutation of the cache


def test_decode_page_table_is_a_permutation():
    w = workloads.BY_NAME["paged-decode-64req-f32kv"]
    ctx = workloads.decode_ctx(w)
    table, num_blocks = workloads.decode_page_table(w, ctx)
    used = []
    for s, c in enumerate(ctx):
        used.extend(table[s, :(int(c) + w.block_size - 1) // w.block_size].tolist())
    assert sorted(used) == list(range(num_blocks))
    assert table.shape == (w.n_slots, int(((ctx + w.block_size - 1) // w.block_size).max()))


def test_generators_are_deterministic_and_distinct():
    w = workloads.BY_NAME["decode-64slots-q4kv"]
    a = workloads.decode_kv(w, 3, 50)
    b = workloads.decode_kv(w, 3, 50)
    c = workloads.decode_kv(w, 4, 50)
    assert np.array_equal(a[0], b[0]) and not np.array_equal(a[0], c[0])
    assert not np.array_equal(a[0], a[1])                        # K and V differ
    f32 = workloads.BY_NAME["decode-64slots-f32kv"]
    assert np.array_equal(workloads.decode_kv(f32, 3, 50)[0], a[0])   # same inputs as the Q4_0 run


def test_spread_reports_median_p90_and_relative_std():
    got = bench.spread([2.0, 1.0, 4.0, 3.0], "t")
    assert got["t_median"] == 2.5
    assert abs(got["t_p90"] - 3.7) < 1e-12                        # linear interpolation
    assert abs(got["t_rel_std"] - np.std([1, 2, 3, 4]) / 2.5) < 1e-12
