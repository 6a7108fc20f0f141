"""Pins of the oracle's fp16-shadow attention ([FA] "fp16 sink + recent-window
exemption", fc_kvq4_is_fp16 and the win_live_lo guard): reductions to the
plain attention, and a brute force on tiny inputs written from explicit key
sets.
"""
import math

import numpy as np
import pytest

import oracle


def rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def setup(seed, n_q=5, n_head=4, n_kv=2, hd=32, kv_rows=40):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rand(rng, n_q, n_head, hd)
    k, v = rand(rng, n_kv, kv_rows, hd), rand(rng, n_kv, kv_rows, hd)
    k16, v16 = rand(rng, n_kv, kv_rows, hd), rand(rng, n_kv, kv_rows, hd)
    pos = np.sort(rng.choice(kv_rows, n_q, replace=False)).astype(np.int32)
    return q, pos, k, v, k16, v16


@pytest.mark.parametrize("attn", [(0, 0), (3, 9)])
def test_no_shadow_is_the_plain_attention(attn):
    q, pos, k, v, k16, v16 = setup(1)
    a = oracle.gqa_rows_shadow(q, pos, k, v, k16, v16, *attn, 0.2, 0, 0, -1)
    b = oracle.gqa_rows(q, pos, k, v, *attn, 0.2)
    assert np.array_equal(a, b)


def test_shadow_over_everything_is_attention_on_the_shadow():
    q, pos, k, v, k16, v16 = setup(2)
    a = oracle.gqa_rows_shadow(q, pos, k, v, k16, v16, 0, 0, 0.3, 0, 10_000, -1)
    b = oracle.gqa_rows(q, pos, k16, v16, 0, 0, 0.3)
    assert np.array_equal(a, b)


def test_identical_sources_make_the_choice_irrelevant():
    q, pos, k, v, _, _ = setup(3)
    a = oracle.gqa_rows_shadow(q, pos, k, v, k, v, 2, 7, 0.25, 4, 6, 11)
    b = oracle.gqa_rows(q, pos, k, v, 2, 7, 0.25)
    assert np.array_equal(a, b)


def brute(q, pos, k, v, k16, v16, attn_sink, attn_win, scale, ssink, swin, live_lo):
    """Plain Python: explicit key set and explicit shadow set per query."""
    n_q, n_head, hd = q.shape
    n_kv = k.shape[0]
    g = n_head // n_kv
    out = np.zeros((n_q * n_head, hd))
    for i in range(n_q):
        p = int(pos[i])
        keys = list(range(p + 1)) if attn_win <= 0 else \
            sorted(set(range(min(attn_sink, p + 1))) | set(range(max(0, p - attn_win + 1), p + 1)))
        shadow = set(range(min(ssink, p + 1)))
        if swin > 0:
            shadow |= {s for s in range(p - swin + 1, p + 1) if s > live_lo and s >= 0}
        for h in range(n_head):
            kv = h // g
            sc = []
            for s in keys:
                kr = (k16 if s in shadow else k)[kv, s]
                sc.append(scale * sum(float(q[i, h, e]) * float(kr[e]) for e in range(hd)))
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            tot = sum(w)
            for wi, s in zip(w, keys):
                vr = (v16 if s in shadow else v)[kv, s]
                for e in range(hd):
                    out[i * n_head + h, e] += wi * float(vr[e]) / tot
    return out


@pytest.mark.parametrize("params", [
    # attn_sink, attn_win, ssink, swin, live_lo
    (0, 0, 2, 4, -1),
    (0, 0, 0, 3, 9),        # lapped ring: keys <= 9 read from the body
    (1, 5, 3, 2, -1),       # key set and shadow both windowed
    (0, 0, 8, 0, -1),       # sink only
])
def test_brute_force_tiny(params):
    attn_sink, attn_win, ssink, swin, live_lo = params
    q, pos, k, v, k16, v16 = setup(10 + sum(params), n_q=4, n_head=4, n_kv=2, hd=4, kv_rows=14)
    pos = np.array([0, 5, 10, 13], np.int32)
    a = oracle.gqa_rows_shadow(q, pos, k, v, k16, v16, attn_sink, attn_win, 0.7, ssink, swin,
                               live_lo)
    b = brute(q, pos, k, v, k16, v16, attn_sink, attn_win, 0.7, ssink, swin, live_lo)
    assert np.abs(a - b).max() < 1e-12


def test_fp16_rounding_helper_matches_the_oracle_conversion():
    rng = np.random.Generator(np.random.PCG64(4))
    x = np.concatenate([rand(rng, 4000) * 10, rand(rng, 1000) * 1e-6, rand(rng, 1000) * 6e4,
                        np.float32([0.0, -0.0, 65504.0, 2.0 ** -24, 1 + 2.0 ** -11])])
    want = np.array([oracle.f16_bits_to_f32(oracle.f32_to_f16_bits(float(t))) for t in x],
                    np.float32)
    assert np.array_equal(oracle.f16_round(x).view(np.uint32), want.view(np.uint32))
