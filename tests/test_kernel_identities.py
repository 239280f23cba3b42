"""Host-side checks of arithmetic identities the HIP kernels rely on.

These do not touch the GPU or the oracle: each one restates, in numpy, a bit
or integer trick that a kernel uses in place of the plain operation, and
checks it against the plain operation over its whole input range.
"""
import numpy as np


def e4m3_value(b):
    """OCP FP8 E4M3 (no infinities, 0x7F / 0xFF are NaN): sign, 4-bit
    exponent with bias 7, 3-bit mantissa, subnormals at exponent 0."""
    s = -1.0 if b & 0x80 else 1.0
    e, m = (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return None
    return s * (m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))


def test_e4m3_bits_moved_into_fp16_fields_give_value_times_2_pow_minus_8():
    # The NVFP4 GEMM turns a block-scale byte into fp16 by moving its sign to
    # bit 15 and its exponent and mantissa to bits 7..14: the fp16 read from
    # those bits is the E4M3 value times 2^-8, for normal and subnormal
    # bytes alike.
    n = 0
    for b in range(256):
        v = e4m3_value(b)
        if v is None:
            continue
        f = ((b & 0x80) << 8) | ((b & 0x7F) << 7)
        h = np.array([f], dtype=np.uint16).view(np.float16)[0]
        assert float(h) * 256.0 == v, b
        n += 1
    assert n == 254


def test_e2m1_times_e4m3_times_2_pow_minus_8_is_exact_in_fp16():
    # Each decoded operand value of that GEMM is e2m1 x (E4M3 x 2^-8),
    # formed by one fp16 multiply: every such product must be an fp16 value.
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for b in range(256):
        v = e4m3_value(b)
        if v is None:
            continue
        sh = np.float16(v / 256.0)
        for g in grid:
            for sign in (1.0, -1.0):
                exact = sign * g * v / 256.0
                assert float(np.float16(sign * g) * sh) == exact, (b, g)


def test_multiply_high_division_is_exact_in_its_range():
    # The panel kernel divides n by the rank d (1 <= d <= 96, n < 96 * 32)
    # as the high half of n * m, m = floor((2^32 - 1) / d) + 1, with d = 1
    # returning n itself (m = 2^32 does not fit).
    n = np.arange(0, 96 * 32 * 4, dtype=np.uint64)
    for d in range(1, 97):
        q = n if d == 1 else (n * np.uint64((0xFFFFFFFF // d) + 1)) >> np.uint64(32)
        assert np.array_equal(q, n // np.uint64(d)), d
