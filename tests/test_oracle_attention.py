"""Pins for the oracle's attention rows.

Definition followed: vllm-cpp-sys include/vt/ops.h, vt::Attention (s_j =
scale * q.k_j for j <= i, softmax, sum of p_j v_j; q head h reads kv head
h / (Hq/Hk)) with the key set of Foundry cuda_kernels/attention.cu's file
header ([0, sink) U [p - win + 1, p] when win > 0) and the AttentionWindow
convention of ops.h ((W-1, 0) is a causal window of W tokens).

What pins it, independently of its own code: torch's scaled_dot_product_attention
in float64 (a library routine) for dense and explicitly masked cases, textbook
closed forms (two-key softmax, own-row V, arithmetic mean for q = 0), and
invariants (GQA expansion, decode == prefill row).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def rand(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(np.float32)


def sdpa_reference(q, k, v, pos0, mask_fn, scale):
    """torch SDPA (float64, CPU) with a boolean mask [n][kv_rows]."""
    n, H, hd = q.shape
    n_kv, rows, _ = k.shape
    G = H // n_kv
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)          # [H][n][hd]
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(G, 0)     # [H][rows][hd]
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(G, 0)
    mask = torch.zeros((n, rows), dtype=torch.bool)
    for t in range(n):
        for j in range(rows):
            mask[t, j] = mask_fn(j, pos0 + t)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale)
    return out.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("n,pos0,H,Hkv,hd", [(1, 0, 1, 1, 8), (37, 0, 4, 2, 16),
                                             (20, 13, 8, 1, 32), (9, 50, 6, 3, 4)])
def test_full_causal_matches_torch_sdpa(n, pos0, H, Hkv, hd):
    rows = pos0 + n
    q, k, v = rand(1, n, H, hd), rand(2, Hkv, rows, hd), rand(3, Hkv, rows, hd)
    scale = 1 / math.sqrt(hd)
    got = oracle.prefill(q, k, v, pos0, 0, 0, scale)
    want = sdpa_reference(q, k, v, pos0, lambda j, p: j <= p, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("sink,win", [(0, 1), (0, 3), (2, 4), (4, 7), (1, 1), (5, 2),
                                      (30, 2), (0, 100)])
def test_window_matches_sdpa_with_explicit_interval_mask(sink, win):
    # the dense mask is the union of two explicit intervals per query row:
    # [0, min(sink, p+1)) and [max(0, p-win+1), p]
    n, pos0, H, Hkv, hd = 40, 5, 4, 2, 8
    rows = pos0 + n
    q, k, v = rand(4, n, H, hd), rand(5, Hkv, rows, hd), rand(6, Hkv, rows, hd)
    scale = 0.37

    def in_intervals(j, p):
        return (0 <= j < min(sink, p + 1)) or (max(0, p - win + 1) <= j <= p)

    got = oracle.prefill(q, k, v, pos0, sink, win, scale)
    want = sdpa_reference(q, k, v, pos0, in_intervals, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_win_nonpositive_is_full_causal_whatever_the_sink():
    n, H, Hkv, hd = 30, 2, 1, 8
    q, k, v = rand(7, n, H, hd), rand(8, Hkv, n, hd), rand(9, Hkv, n, hd)
    full = oracle.prefill(q, k, v, 0, 0, 0, 0.5)
    for sink, win in [(0, -1), (3, 0), (100, -5)]:
        np.testing.assert_array_equal(oracle.prefill(q, k, v, 0, sink, win, 0.5), full)


def test_window_or_sink_covering_the_prefix_is_full_causal():
    n, H, Hkv, hd = 25, 2, 2, 8
    q, k, v = rand(10, n, H, hd), rand(11, Hkv, n, hd), rand(12, Hkv, n, hd)
    full = oracle.prefill(q, k, v, 0, 0, 0, 0.5)
    np.testing.assert_array_equal(oracle.prefill(q, k, v, 0, 0, n, 0.5), full)
    np.testing.assert_array_equal(oracle.prefill(q, k, v, 0, n, 1, 0.5), full)


def test_window_of_one_returns_own_value_row():
    # win = 1, sink = 0: the key set of position p is {p}, softmax weight 1
    n, H, Hkv, hd = 12, 4, 2, 16
    q, k, v = rand(13, n, H, hd), rand(14, Hkv, n, hd), rand(15, Hkv, n, hd)
    got = oracle.prefill(q, k, v, 0, 0, 1, 0.25)
    for t in range(n):
        for h in range(H):
            np.testing.assert_array_equal(got[t, h], v[h // 2, t].astype(np.float64))


def test_position_zero_returns_its_value_row():
    q, k, v = rand(16, 1, 3, 8), rand(17, 1, 1, 8), rand(18, 1, 1, 8)
    got = oracle.prefill(q, k, v, 0, 0, 0, 1.0)
    for h in range(3):
        np.testing.assert_array_equal(got[0, h], v[0, 0].astype(np.float64))


def two_key_closed_form(s_a, s_b, v_a, v_b):
    # softmax over two keys: weight of b is the logistic function of s_b - s_a
    wb = 1.0 / (1.0 + math.exp(-(s_b - s_a)))
    return (1.0 - wb) * v_a + wb * v_b


@pytest.mark.parametrize("scale", [0.125, 1.0, 2.5])
def test_two_key_window_closed_form(scale):
    # sink = 0, win = 2: position p sees exactly {p-1, p}
    hd = 4
    q = np.zeros((6, 1, hd), np.float32)
    k = np.zeros((1, 6, hd), np.float32)
    v = rand(19, 1, 6, hd)
    q[:, 0, 0] = [1.0, 2.0, -1.0, 0.5, 3.0, -2.0]
    k[0, :, 0] = [0.5, -1.0, 2.0, 1.5, -0.25, 1.0]
    got = oracle.prefill(q, k, v, 0, 0, 2, scale)
    for p in range(1, 6):
        s_a = scale * float(q[p, 0, 0]) * float(k[0, p - 1, 0])
        s_b = scale * float(q[p, 0, 0]) * float(k[0, p, 0])
        want = two_key_closed_form(s_a, s_b, v[0, p - 1].astype(np.float64),
                                   v[0, p].astype(np.float64))
        np.testing.assert_allclose(got[p, 0], want, rtol=0, atol=1e-14)


def test_sink_plus_self_closed_form():
    # sink = 1, win = 1: position p > 0 sees exactly {0, p}
    hd = 3
    q = rand(20, 8, 1, hd)
    k = rand(21, 1, 8, hd)
    v = rand(22, 1, 8, hd)
    got = oracle.prefill(q, k, v, 0, 1, 1, 0.7)
    for p in range(1, 8):
        s0 = 0.7 * float(np.dot(q[p, 0].astype(np.float64), k[0, 0].astype(np.float64)))
        sp = 0.7 * float(np.dot(q[p, 0].astype(np.float64), k[0, p].astype(np.float64)))
        want = two_key_closed_form(s0, sp, v[0, 0].astype(np.float64), v[0, p].astype(np.float64))
        np.testing.assert_allclose(got[p, 0], want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("sink,win", [(0, 0), (3, 5), (0, 4), (6, 1)])
def test_zero_query_gives_mean_of_values_over_key_set(sink, win):
    # q = 0 makes every score 0, so the output is the plain average of the V
    # rows in the key set; the set's size has its own closed form
    n, pos0, hd = 20, 7, 8
    q = np.zeros((n, 2, hd), np.float32)
    k, v = rand(23, 1, pos0 + n, hd), rand(24, 1, pos0 + n, hd)
    got = oracle.prefill(q, k, v, pos0, sink, win, 1.0)
    for t in range(n):
        p = pos0 + t
        if win <= 0:
            keys = list(range(p + 1))
        else:
            lo = max(0, p - win + 1)
            keys = sorted(set(range(min(sink, p + 1))) | set(range(lo, p + 1)))
            assert len(keys) == min(p + 1, min(sink, lo) + (p - lo + 1))
        want = v[0, keys].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(got[t, 0], want, rtol=0, atol=1e-14)
        np.testing.assert_allclose(got[t, 1], want, rtol=0, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_heads():
    n, H, Hkv, hd = 15, 8, 2, 8
    q, k, v = rand(25, n, H, hd), rand(26, Hkv, n, hd), rand(27, Hkv, n, hd)
    got = oracle.prefill(q, k, v, 0, 2, 5, 0.3)
    k_rep = np.repeat(k, H // Hkv, axis=0)
    v_rep = np.repeat(v, H // Hkv, axis=0)
    np.testing.assert_array_equal(oracle.prefill(q, k_rep, v_rep, 0, 2, 5, 0.3), got)
    # swapping kv head 0 and 1 moves the answer between the two head groups
    got_sw = oracle.prefill(q[:, ::-1].copy(), k[::-1].copy(), v[::-1].copy(), 0, 2, 5, 0.3)
    np.testing.assert_array_equal(got_sw[:, ::-1], got)


def test_decode_row_equals_prefill_row():
    n, H, Hkv, hd = 33, 4, 1, 8
    q, k, v = rand(28, n, H, hd), rand(29, Hkv, n, hd), rand(30, Hkv, n, hd)
    pre = oracle.prefill(q, k, v, 0, 0, 0, 0.4)
    for p in [0, 1, 16, 32]:
        dec = oracle.gqa_rows(q[p:p + 1], [p], k, v, 0, 0, 0.4).reshape(H, hd)
        np.testing.assert_array_equal(dec, pre[p])


def test_selected_rows_and_threads_match_full_evaluation():
    n, H, Hkv, hd = 21, 4, 2, 8
    q, k, v = rand(31, n, H, hd), rand(32, Hkv, n, hd), rand(33, Hkv, n, hd)
    full = oracle.prefill(q, k, v, 0, 1, 6, 0.4).reshape(n * H, hd)
    sel = np.array([0, 5, 83, 42, 17], dtype=np.int64)
    np.testing.assert_array_equal(oracle.prefill(q, k, v, 0, 1, 6, 0.4, sel=sel), full[sel])
    np.testing.assert_array_equal(
        oracle.prefill(q, k, v, 0, 1, 6, 0.4, threads=4).reshape(n * H, hd), full)


def test_rejects_positions_past_the_cache():
    q, k, v = rand(34, 4, 1, 8), rand(35, 1, 4, 8), rand(36, 1, 4, 8)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, 1, 0, 0, 1.0)   # row 3 at position 4, cache holds 4 rows


def test_large_scores_do_not_overflow():
    # global-max subtraction keeps exp() finite for scores far beyond 700
    q = np.full((3, 1, 4), 30.0, np.float32)
    k = np.full((1, 3, 4), 10.0, np.float32)
    v = rand(37, 1, 3, 4)
    got = oracle.prefill(q, k, v, 0, 0, 0, 1.0)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got[2, 0], v[0].astype(np.float64).mean(0), atol=1e-14)
