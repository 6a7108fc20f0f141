"""Pins for the oracle's Q4_0 codec and its binary16 conversion.

The Q4_0 format and quantiser steps are those of Foundry
cuda_kernels/attention.cu ("4-bit KV cache (Q4_0 blocks)" section and the
fc_kvq4_quant_block / fc_kvq4_dequant_elem comments). Expected values come
from tests/golden/q4_blocks.txt (hand-derived), from numpy's IEEE binary16
conversion (a library routine) and from the quantiser's error bound.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4_blocks.txt")


def _num(s: str) -> float:
    return float.fromhex(s) if "0x" in s else float(s)


def load_cases():
    cases, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            rest = rest.strip()
            if key == "case":
                name, hd = rest.split()
                cur = {"name": name, "hd": int(hd), "x": {}, "deq": {}, "rest": None}
                cases.append(cur)
            elif key == "x":
                for tok in rest.split():
                    i, v = tok.split("=")
                    cur["x"][int(i)] = _num(v)
            elif key == "bytes":
                cur["bytes"] = bytes.fromhex(rest)
            elif key == "deq":
                for tok in rest.split():
                    i, v = tok.split("=")
                    if i == "rest":
                        cur["rest"] = _num(v)
                    else:
                        cur["deq"][int(i)] = _num(v)
    return cases


CASES = load_cases()


def test_golden_file_is_well_formed():
    assert len(CASES) >= 12
    for c in CASES:
        assert len(c["bytes"]) == c["hd"] // 32 * 18, c["name"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_built_blocks(case):
    hd = case["hd"]
    x = np.zeros(hd, dtype=np.float32)
    for i, v in case["x"].items():
        x[i] = np.float32(v)
        assert float(x[i]) == v or (np.isnan(v) and np.isnan(x[i])), "fixture value not exact"
    row = oracle.q4_quantize(x)
    assert row.tobytes() == case["bytes"]
    deq = oracle.q4_dequantize(row, hd)
    for e in range(hd):
        want = case["deq"].get(e, case["rest"])
        got = float(deq[e])
        if np.isnan(want):
            assert np.isnan(got), (e, got, want)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (e, got, want)


def test_f16_conversion_matches_numpy_on_all_halves():
    # every binary16 bit pattern decodes like numpy's IEEE decoder
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_bits_to_f32(int(b)) for b in bits], dtype=np.float32)
    finite = np.isfinite(want)
    assert np.array_equal(got[finite].view(np.uint32), want[finite].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(want) & (want > 0))


def test_f32_to_f16_round_to_nearest_even_matches_numpy():
    rng = np.random.Generator(np.random.PCG64(7))
    # values across the whole binary16 range: normals, subnormals, ties, overflow
    mags = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.random(20000) * 70000).astype(np.float32),
        np.float32(2.0) ** rng.integers(-30, 17, 20000).astype(np.float32)
        * rng.random(20000).astype(np.float32),
    ])
    # exact ties: a half-way significand between two binary16 neighbours
    halves = np.arange(0x0400, 0x7bff, 7, dtype=np.uint16).view(np.float16).astype(np.float32)
    nxt = (np.arange(0x0400, 0x7bff, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float32)
    ties = (halves.astype(np.float64) + nxt.astype(np.float64)) / 2
    sub_ties = (np.arange(1, 1023, dtype=np.float64) + 0.5) * 2.0 ** -24
    vals = np.concatenate([mags, -mags, ties.astype(np.float32), sub_ties.astype(np.float32),
                           np.float32([65504, 65519.99, 65520, 1e30, 0.0, -0.0, 2 ** -25,
                                       2 ** -25 * 1.0001, 2 ** -26])])
    want = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_quantise_error_bound_on_random_rows():
    # |deq(x) - x| <= |d|/2 + 8*|fp16(d) - d| (plus one ulp of slack for the
    # rounded reciprocal): code error of at most half a step, then the stored
    # scale's rounding scaled by |c - 8| <= 8.
    rng = np.random.Generator(np.random.PCG64(11))
    x = rng.standard_normal((4096, 256)).astype(np.float32)
    deq = oracle.q4_dequantize(oracle.q4_quantize(x), 256).astype(np.float64)
    blocks = x.reshape(-1, 32).astype(np.float64)
    amax = np.abs(blocks).max(axis=1)
    d32 = (amax / -8.0).astype(np.float32).astype(np.float64)
    d16 = d32.astype(np.float16).astype(np.float64)
    slack = 8 * np.abs(d16 - d32) + np.abs(d32) * 1e-6
    err = np.abs(deq.reshape(-1, 32) - blocks)
    # in range: x/d in [-8.5, 7.5] -> at most half a step
    ratio = blocks / d32[:, None]
    in_range = ratio <= 7.5
    assert np.all(err[in_range] <= np.broadcast_to((np.abs(d32) / 2 + slack)[:, None],
                                                   err.shape)[in_range])
    # clipped (x near -amax, code 15 = 7*d): at most one full step
    assert np.all(err <= (np.abs(d32) + slack)[:, None])
    assert np.any(~in_range)


def test_codes_cover_range_and_extremes_exact():
    # The block's +amax element is exact (code 0), a -amax element clips to 15.
    rng = np.random.Generator(np.random.PCG64(12))
    x = rng.standard_normal((512, 32)).astype(np.float32)
    rows = oracle.q4_quantize(x)
    deq = oracle.q4_dequantize(rows, 32)
    for r in range(512):
        i = int(np.argmax(np.abs(x[r])))
        d = float(np.float16(np.float32(np.abs(x[r]).max()) / np.float32(-8)))
        if x[r, i] > 0:
            assert deq[r, i] == np.float32(-8 * d)
        else:
            assert deq[r, i] == np.float32(7 * d)


def test_dequantised_values_are_code_times_scale():
    # (c - 8) * d is exact in fp32: every dequantised value divided by its
    # block's scale is an integer in [-8, 7].
    rng = np.random.Generator(np.random.PCG64(13))
    x = (rng.standard_normal((256, 128)) * 3).astype(np.float32)
    rows = oracle.q4_quantize(x)
    deq = oracle.q4_dequantize(rows, 128).reshape(-1, 32).astype(np.float64)
    scales = rows.reshape(-1, 18)[:, :2].copy().view(np.float16).astype(np.float64).reshape(-1, 1)
    ratio = deq / scales
    assert np.all(ratio == np.round(ratio))
    assert ratio.min() >= -8 and ratio.max() <= 7


def test_rows_are_independent_and_ordered():
    rng = np.random.Generator(np.random.PCG64(14))
    x = rng.standard_normal((3, 5, 64)).astype(np.float32)
    rows = oracle.q4_quantize(x)
    assert rows.shape == (3, 5, 36)
    for a in range(3):
        for b in range(5):
            assert np.array_equal(rows[a, b], oracle.q4_quantize(x[a, b]))
