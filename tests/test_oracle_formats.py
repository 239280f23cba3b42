"""Pins of the oracle's FP4 codecs against facts fixed outside the oracle.

Each test is chosen so that a plausible slip in ``oracle/formats.py`` (a wrong
tie rule, an off-by-one in the shared exponent, a dropped sign, a swapped
nibble, a reciprocal instead of a division) fails at least one of them.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def brute_e2m1(v):
    """Independent nearest-of-eight: minimise |v| - g over the grid, ties to
    the even code index, sign from v (also for zero)."""
    # beyond 7 the nearest point is 6 whatever the value; clipping keeps the
    # differences exact for huge inputs
    a = np.minimum(np.abs(v), 7.0)[..., None]
    d = np.abs(a - GRID)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equal distances take an even index if there is one
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return (pick | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def test_e2m1_grid_values_round_trip():
    codes = np.arange(16, dtype=np.uint8)
    vals = F.e2m1_decode(codes)
    assert list(vals[:8]) == list(GRID)
    assert np.all(F.e2m1_encode(vals) == codes)


def test_e2m1_exhaustive_near_every_decision_point():
    """Every fp32 value within 2^18 bit patterns of each rounding threshold and
    grid point in (0, 8) (both signs), a stride-13 sweep of all of [2^-3, 8),
    and a strided sweep of all 2^31 positive bit patterns below infinity,
    against the brute force."""
    points = [0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0]
    win = 1 << 18
    for p in points:
        c = int(np.float32(p).view(np.uint32))
        bits = np.arange(c - win, c + win, dtype=np.uint32)
        v = bits.view(np.float32).astype(np.float64)
        assert np.array_equal(F.e2m1_encode(v), brute_e2m1(v)), p
        assert np.array_equal(F.e2m1_encode(-v), brute_e2m1(-v)), p
    lo = int(np.float32(0.125).view(np.uint32))
    hi = int(np.float32(8.0).view(np.uint32))
    bits = np.arange(lo, hi, 13, dtype=np.uint32)
    v = bits.view(np.float32).astype(np.float64)
    assert np.array_equal(F.e2m1_encode(v), brute_e2m1(v))
    assert np.array_equal(F.e2m1_encode(-v), brute_e2m1(-v))
    bits = np.arange(0, 0x7F800000, 997, dtype=np.uint32)
    v = bits.view(np.float32).astype(np.float64)
    assert np.array_equal(F.e2m1_encode(v), brute_e2m1(v))


def test_e2m1_hand_listed_ties_and_saturation():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 1e30, -0.0, -0.25, -5.0])
    expect = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, -0.0, -0.0, -4.0]
    got = F.e2m1_decode(F.e2m1_encode(v))
    assert list(got) == expect
    assert F.e2m1_encode(np.array([-0.0]))[0] == 8  # sign of zero kept


@pytest.mark.parametrize("gmax", [6.0, 4.0, 3.0, 2.0, 1.5, 1.0, 0.5])
def test_mx_grid_times_power_of_two_round_trips_for_every_exponent(gmax):
    """Blocks of E2M1 grid values times 2^e, for every E8M0 exponent e, come back exactly."""
    g = np.random.Generator(np.random.PCG64(7))
    sub = GRID[GRID <= gmax]
    for e in range(-127, 128):
        mags = g.choice(sub, size=(3, 32))
        mags[:, 0] = gmax
        signs = g.choice([-1.0, 1.0], size=(3, 32))
        x = np.ldexp(mags * signs, e)
        codes, scales = F.mx_quantize(x)
        assert np.array_equal(F.mx_dequantize(codes, scales), x), e
        want = int(np.clip(e + int(np.floor(np.log2(gmax))) - 2, -127, 127)) + 127
        assert np.all(scales == want), e


def test_mx_scale_rule_closed_form():
    # amax = 1 -> floor(log2 1) = 0 -> shared exponent -2 -> byte 125
    x = np.zeros((1, 32)); x[0, 3] = 1.0; x[0, 4] = -0.3
    codes, scales = F.mx_quantize(x)
    assert scales[0, 0] == 125
    c = F.unpack_nibbles(codes)[0]
    assert c[3] == 6          # 1.0 * 4 = 4.0 -> code 6
    assert c[4] == 8 | 2      # -0.3 * 4 = -1.2 -> -1.0 (code 2 with sign)
    # amax just below 2: floor(log2) = 0 still
    x[0, 3] = np.nextafter(2.0, 0.0)
    assert F.mx_quantize(x)[1][0, 0] == 125
    x[0, 3] = 2.0
    assert F.mx_quantize(x)[1][0, 0] == 126
    # all-zero block (with a negative zero): scale byte 0, codes keep sign
    z = np.zeros((1, 32)); z[0, 1] = -0.0
    cz, sz = F.mx_quantize(z)
    assert sz[0, 0] == 0 and F.unpack_nibbles(cz)[0, 1] == 8 and F.unpack_nibbles(cz)[0, 0] == 0
    # tiny amax clamps at 2^-127
    t = np.full((1, 32), 2.0 ** -140)
    assert F.mx_quantize(t)[1][0, 0] == 0


def test_nibble_order():
    codes = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    assert list(F.pack_nibbles(codes)[0]) == [0x21, 0x43]
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(codes)), codes)


@pytest.mark.parametrize("dist", ["normal", "heavy", "ties", "tiny"])
def test_mx_brute_force_4x32(dist):
    """For 4x32 blocks, each code minimises |x - value(code) 2^se| over all 16
    codes (ties: the even code; zero: the sign of x), and the error is within
    half a grid step at that scale."""
    g = np.random.Generator(np.random.PCG64(11))
    if dist == "normal":
        x = g.standard_normal((4, 32))
    elif dist == "heavy":
        x = g.standard_normal((4, 32)) * np.exp(3 * g.standard_normal((4, 32)))
    elif dist == "ties":
        # values exactly on the decision points of the grid at the block's scale
        x = g.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], size=(4, 32)) * g.choice([-1, 1], size=(4, 32))
        x[:, 0] = 6.0
        x = x * 2.0 ** -3
    else:
        x = g.standard_normal((4, 32)) * 2.0 ** -135
    codes, scales = F.mx_quantize(x)
    c = F.unpack_nibbles(codes)
    se = scales.astype(np.int64) - 127
    for r in range(4):
        amax = np.max(np.abs(x[r]))
        assert se[r, 0] == (max(min(int(np.floor(np.log2(amax))) - 2, 127), -127) if amax > 0 else -127)
        cand = np.ldexp(F.e2m1_decode(np.arange(16, dtype=np.uint8)), int(se[r, 0]))
        for i in range(32):
            d = np.abs(x[r, i] - cand)
            best = np.flatnonzero(d == d.min())
            mags = set(int(b) & 7 for b in best)
            if len(mags) > 1:  # genuine tie between two magnitudes
                want_mag = [m for m in mags if m % 2 == 0][0]
            else:
                want_mag = mags.pop()
            assert c[r, i] & 7 == want_mag
            assert (c[r, i] >> 3) == int(np.signbit(x[r, i]))
        err = np.abs(F.mx_dequantize(codes, scales)[r] - x[r])
        step = np.ldexp(2.0, int(se[r, 0]))  # largest grid gap (4 -> 6) at this scale
        top = np.ldexp(6.0, int(se[r, 0]))
        # the floor scale rule lets |x| reach 8 * 2^se: those values saturate at 6
        allowed = np.where(np.abs(x[r]) > top, np.abs(x[r]) - top, step / 2)
        assert np.all(err <= allowed + 1e-300)


def test_e4m3_against_torch_float8():
    """Every finite positive E4M3 value, every midpoint and its fp32
    neighbours, and random values below 464: oracle == torch's RNE cast."""
    allv = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    mids = (allv[1:] + allv[:-1]) / 2
    pts = np.concatenate([allv, mids])
    pts32 = pts.astype(np.float32)
    near = np.concatenate([pts32, np.nextafter(pts32, np.float32(0)), np.nextafter(pts32, np.float32(1e9))])
    g = np.random.Generator(np.random.PCG64(3))
    rnd = (np.exp(g.uniform(np.log(2.0 ** -12), np.log(463.9), 20000))).astype(np.float32)
    v = np.concatenate([near, rnd]).astype(np.float32)
    v = v[(v >= 0) & (v < 464)]
    ours = F.e4m3_decode(F.e4m3_encode(v.astype(np.float64)))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    # byte-level agreement too
    ref_bytes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(v.astype(np.float64)), ref_bytes)


def test_e4m3_boundaries_by_hand():
    v = np.array([447.0, 448.0, 464.0, 1e6, 2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -10, 2.0 ** -6, 0.0])
    want = [448.0, 448.0, 448.0, 448.0, 2.0 ** -9, 0.0, 2.0 ** -9, 2.0 ** -6, 0.0]
    assert list(F.e4m3_decode(F.e4m3_encode(v))) == want
    assert F.e4m3_encode(np.array([448.0]))[0] == 0x7E  # exponent 15, mantissa 6


def _nv_by_numpy_float32(x32, s_t=None):
    """The NVFP4 chain written with numpy float32 scalars (IEEE single ops);
    s_t given: that tensor scale instead of the array's own."""
    x32 = np.asarray(x32, dtype=np.float32)
    a_t = np.max(np.abs(x32))
    if s_t is not None:
        s_t = np.float32(s_t)
    elif a_t == 0:
        s_t = np.float32(1.0)
    else:
        s_t = max(np.float32(a_t) / np.float32(2688.0), np.float32(2.0 ** -126))
    s_t = np.float32(s_t)
    rows, cols = x32.shape
    xb = x32.reshape(rows, cols // 16, 16)
    amax = np.max(np.abs(xb), axis=-1)
    d = np.float32(np.float32(6.0) * s_t)
    b = (amax / d).astype(np.float32)
    sb = F.e4m3_encode(b.astype(np.float64))
    sbv = F.e4m3_decode(sb).astype(np.float32)
    den = (sbv * s_t).astype(np.float32)
    safe = np.where(sbv > 0, den, np.float32(1.0)).astype(np.float32)
    q = (xb / safe[..., None]).astype(np.float32)
    q = np.where((sbv > 0)[..., None], q, np.float32(0.0) * xb)
    return brute_e2m1(q.astype(np.float64)).reshape(rows, cols), sb, s_t


@pytest.mark.parametrize("dist", ["normal", "wide", "outlier"])
def test_nv_matches_float32_arithmetic(dist):
    g = np.random.Generator(np.random.PCG64(5))
    x = g.standard_normal((8, 64))
    if dist == "wide":
        x *= np.exp(4 * g.standard_normal((8, 64)))
    if dist == "outlier":
        x[:, 5] *= 1e4
        x[2, :16] = 0.0
    x32 = x.astype(np.float32)
    codes, sb, s_t = F.nv_quantize(x32.astype(np.float64))
    ref_codes, ref_sb, ref_st = _nv_by_numpy_float32(x32)
    assert np.float32(s_t) == ref_st
    assert np.array_equal(sb, ref_sb)
    assert np.array_equal(F.unpack_nibbles(codes), ref_codes)


@pytest.mark.parametrize("factor", [0.75, 1.0 + 2.0 ** -20, 3.0])
def test_nv_with_a_given_tensor_scale_matches_float32_arithmetic(factor):
    """A tensor scale passed in (not the array's own max / 2688) enters the
    same fp32 chain; blocks past 6 * 448 times it saturate at scale 448."""
    g = np.random.Generator(np.random.PCG64(6))
    x32 = (g.standard_normal((8, 64)) * np.exp(3 * g.standard_normal((8, 64)))).astype(np.float32)
    own = F.nv_tensor_scale(x32.astype(np.float64))
    s_t = float(np.float32(own * factor))
    codes, sb, st = F.nv_quantize(x32.astype(np.float64), tensor_scale=s_t)
    ref_codes, ref_sb, ref_st = _nv_by_numpy_float32(x32, s_t)
    assert np.float32(st) == ref_st
    assert np.array_equal(sb, ref_sb)
    assert np.array_equal(F.unpack_nibbles(codes), ref_codes)


def test_nv_zero_tensor_and_dequant_rounding():
    codes, sb, s_t = F.nv_quantize(np.zeros((2, 32)))
    assert s_t == 1.0 and np.all(sb == 0) and np.all(codes == 0)
    x = np.array([[6.0 * 448.0] + [0.0] * 15], dtype=np.float32).astype(np.float64)
    codes, sb, s_t = F.nv_quantize(x)
    assert s_t == 1.0 and F.e4m3_decode(sb)[0, 0] == 448.0
    assert F.nv_dequantize(codes, sb, s_t)[0, 0] == 2688.0
