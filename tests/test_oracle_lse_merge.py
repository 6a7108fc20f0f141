"""Pins of the oracle's log-sum-exp, attention-state merge ([VT]
MergeAttnStates) and paged-cache row gather ([VT] PagedAttention)."""
import numpy as np
import pytest

import oracle


def data(seed, n_q=3, H=4, n_kv=2, hd=16, rows=30):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((n_q, H, hd)).astype(np.float32),
            rng.standard_normal((n_kv, rows, hd)).astype(np.float32),
            rng.standard_normal((n_kv, rows, hd)).astype(np.float32))


def test_lse_of_a_single_key_is_its_score():
    q, k, _ = data(1)
    lse = oracle.gqa_lse(q, [0, 0, 0], k, 0, 0, 0.3)
    want = [0.3 * float(np.dot(q[i, h].astype(np.float64), k[h // 2, 0].astype(np.float64)))
            for i in range(3) for h in range(4)]
    assert np.allclose(lse, want, rtol=0, atol=1e-12)


def test_lse_of_identical_keys_adds_log_count():
    q, k, _ = data(2)
    k[:] = k[:, :1]                      # every key equals key 0
    lse = oracle.gqa_lse(q, [4, 9, 29], k, 0, 0, 0.5)
    base = oracle.gqa_lse(q, [0, 0, 0], k, 0, 0, 0.5)
    counts = np.repeat([5, 10, 30], 4)
    assert np.allclose(lse - base, np.log(counts), rtol=0, atol=1e-12)


def test_lse_weights_reproduce_the_attention_output():
    q, k, v = data(3)
    pos = [7, 20, 29]
    lse = oracle.gqa_lse(q, pos, k, 2, 9, 0.25).reshape(3, 4)
    out = oracle.gqa_rows(q, pos, k, v, 2, 9, 0.25).reshape(3, 4, -1)
    for i, p in enumerate(pos):
        keys = [j for j in range(p + 1) if oracle.key_in_set(j, p, 2, 9)]
        for h in range(4):
            s = 0.25 * (k[h // 2, keys].astype(np.float64) @ q[i, h].astype(np.float64))
            w = np.exp(s - lse[i, h])
            assert abs(w.sum() - 1.0) < 1e-12
            assert np.allclose(w @ v[h // 2, keys].astype(np.float64), out[i, h], atol=1e-12)


@pytest.mark.parametrize("split", [1, 6, 12])
def test_merging_disjoint_key_sets_gives_the_full_attention(split):
    # keys [0, split) (a query at split-1 sees exactly those) and [split, p]
    # (a window of p - split + 1 keys ending at p) are disjoint and cover [0, p]
    q, k, v = data(4 + split, n_q=1)
    p = 12
    full = oracle.gqa_rows(q, [p], k, v, 0, 0, 0.4).reshape(1, 4, -1)
    full_lse = oracle.gqa_lse(q, [p], k, 0, 0, 0.4).reshape(4, 1)
    pre = oracle.gqa_rows(q, [split - 1], k, v, 0, 0, 0.4).reshape(1, 4, -1)
    pre_lse = oracle.gqa_lse(q, [split - 1], k, 0, 0, 0.4).reshape(4, 1)
    win = p - split + 1
    suf = oracle.gqa_rows(q, [p], k, v, 0, win, 0.4).reshape(1, 4, -1)
    suf_lse = oracle.gqa_lse(q, [p], k, 0, win, 0.4).reshape(4, 1)
    out, lse = oracle.merge_attn_states(pre, pre_lse, suf, suf_lse)
    assert np.allclose(out, full, atol=1e-12) and np.allclose(lse, full_lse, atol=1e-12)
    # the merge is symmetric in its two inputs
    out2, lse2 = oracle.merge_attn_states(suf, suf_lse, pre, pre_lse)
    assert np.allclose(out2, out, atol=1e-13) and np.allclose(lse2, lse, atol=1e-13)


def test_merge_edge_cases():
    rng = np.random.Generator(np.random.PCG64(5))
    po, so = rng.standard_normal((4, 2, 3)), rng.standard_normal((4, 2, 3))
    pl = np.array([[np.inf, -np.inf, 0.5, 1.0], [-np.inf, 2.0, 0.0, 3.0]])
    sl = np.array([[0.0, -np.inf, np.inf, 1.0], [1.0, -np.inf, 0.0, 3.0]])
    out, lse = oracle.merge_attn_states(po, pl, so, sl, prefill_tokens_with_context=3)
    assert np.array_equal(out[0, 0], so[0, 0]) and lse[0, 0] == 0.0      # +inf counts as -inf
    assert np.array_equal(out[1, 0], po[1, 0]) and lse[0, 1] == -np.inf  # both -inf: prefix
    assert np.array_equal(out[2, 0], po[2, 0]) and lse[0, 2] == 0.5
    assert np.array_equal(out[1, 1], po[1, 1]) and lse[1, 1] == 2.0
    assert np.allclose(out[2, 1], (po[2, 1] + so[2, 1]) / 2) and np.isclose(lse[1, 2], np.log(2))
    assert np.array_equal(out[3], so[3]) and np.array_equal(lse[:, 3], sl[:, 3])   # suffix only


def test_paged_rows_inverts_a_scatter():
    rng = np.random.Generator(np.random.PCG64(6))
    n_kv, hd, bs, L = 2, 8, 16, 70
    rows = rng.standard_normal((n_kv, L, hd)).astype(np.float32)
    table = rng.permutation(10)[:5]           # 5 blocks of 16 hold 70 rows
    cache = np.zeros((10, bs, n_kv, hd), np.float32)
    for j in range(L):
        cache[table[j // bs], j % bs] = rows[:, j]
    assert np.array_equal(oracle.paged_rows(cache, table, L), rows)
