"""The GPU dequantises a Q4_0 code c with scale d by one fused multiply-add on
a binary16 operand built from the code's nibble: (1024 + c) * d - 1032 d for a
low nibble and (1024 + 16 c) * (d / 16) - 72 d for a high nibble. Both must
equal (c - 8) * d exactly for every finite fp16 scale d and every code: the
fp32 constants d/16, 1032 d and 72 d must be exact and the fused result must
round to (c - 8) d itself. Checked exhaustively here in float64 (every value
involved has at most 20 significant bits, so float64 holds them exactly), and
compared bit for bit: the only difference is the sign of a zero. For code 8
(or a zero scale) both identities cancel exactly, and an exact cancellation
rounds to +0.0, while (c - 8) * d is -0.0 for code 8 when d is negative (as
every scale the quantiser writes is). The value is the same and no attention output can tell them apart
(a zero key element adds nothing to q.k, a zero value element nothing to the
accumulator).
"""
import numpy as np


def all_finite_fp16_scales():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    d = bits.view(np.float16).astype(np.float64)
    return d[np.isfinite(d)]


def exact_in_f32(x):
    return np.all(x.astype(np.float32).astype(np.float64) == x)


def test_binary16_operand_values():
    # 0x6400 | c and 0x6400 | (c << 4) as binary16
    for c in range(16):
        lo = np.array([0x6400 | c], dtype=np.uint16).view(np.float16)[0]
        hi = np.array([0x6400 | (c << 4)], dtype=np.uint16).view(np.float16)[0]
        assert float(lo) == 1024 + c
        assert float(hi) == 1024 + 16 * c


def test_fused_dequant_is_exact_for_every_scale_and_code():
    d = all_finite_fp16_scales()
    assert d.size == 65536 - 2048          # all patterns but inf and NaN
    d16 = d / 16.0
    assert exact_in_f32(d16) and exact_in_f32(1032.0 * d) and exact_in_f32(72.0 * d)
    for c in range(16):
        want = (c - 8) * d
        assert exact_in_f32(want)
        low = (1024 + c) * d - 1032.0 * d            # exact in float64
        high = (1024 + 16 * c) * d16 - 72.0 * d
        bits = lambda x: x.astype(np.float32).view(np.uint32)
        zero = (d == 0) | (c == 8)
        # exact cancellation: +0.0 whatever the signs; (c - 8) * d is a zero
        # of either sign there (-0.0 for code 8 with a negative scale)
        assert np.all(bits(low)[zero] == 0) and np.all(bits(high)[zero] == 0)
        if c == 8:
            assert np.all(bits(want)[d < 0] == 0x80000000)
        # elsewhere one rounding of the exact value to fp32 (what the fused op
        # does) gives (c - 8) * d bit for bit
        assert np.array_equal(bits(low)[~zero], bits(want)[~zero])
        assert np.array_equal(bits(high)[~zero], bits(want)[~zero])
