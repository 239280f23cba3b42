"""FP4 number formats and block codecs, written from their definitions (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the method asks for: every part of the split (dominant factors and the
long-tail residual) is block-quantized to a 4-bit float format, MXFP4 or
NVFP4 (SII open-source-week post on Metis, "Ecosystem" highlights and §2.2;
"Metis: Training LLMs with FP4 Quantization", abstract: W4A4G4). The pages
name the formats but do not define them, so the bit layouts follow the public
format descriptions:

* E2M1 (OCP Microscaling Formats v1.0, §5.3.3): sign bit 3, exponent bits 2-1
  (bias 1), mantissa bit 0. Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E8M0 block scale (OCP MX v1.0, §5.4.1 and the scale rule of §6.3): byte e
  stands for 2^(e-127); the shared exponent is floor(log2(amax)) - emax_elem
  with emax_elem = 2 for E2M1.
* E4M3 (OCP 8-bit floating point, "E4M3FN"): bias 7, max 448, subnormal
  step 2^-9, no infinities; byte 0x7F/0xFF is NaN and is never produced here.
* NVFP4 (NVIDIA's public NVFP4 description): 16-element blocks with an E4M3
  scale, plus one fp32 scale per tensor.

Readings taken where the pages are silent:
round-to-nearest-even with ties to the even code, saturation at +-6 (E2M1)
and +-448 (E4M3), the sign of zero kept, all-zero block -> scale byte 0,
NVFP4 scale arithmetic as a chain of correctly rounded fp32 operations with a
division (never a multiplication by a reciprocal).

Pins (tests/test_oracle_formats.py): exact round trip of the E2M1 grid times
2^e for every E8M0 exponent; an independent nearest-of-eight brute force over
every fp32 bit pattern near each decision point and a dense sweep of the rest; brute-force search over all 16
codes for 4x32 blocks; torch.float8_e4m3fn as a library special case for E4M3;
numpy.float32 arithmetic for the fp32 emulation; hand-listed boundary values.
"""
import numpy as np

# Magnitudes of E2M1 codes 0..7 (bit 3 is the sign).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0
# Midpoints between neighbouring magnitudes: the rounding decision points.
_E2M1_MIDPOINTS = (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:]) / 2.0

MX_BLOCK = 32
NV_BLOCK = 16
E4M3_MAX = 448.0
NV_TENSOR_DIVISOR = E2M1_MAX * E4M3_MAX  # 2688: maps the tensor max to 6 * 448
FP32_MIN_NORMAL = 2.0 ** -126


def _as_f64(x):
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("oracle inputs must be finite (NaN/Inf are undefined)")
    return x


def f32(x):
    """Round fp64 value(s) to the nearest fp32 (ties to even), back as fp64.

    An fp32 +, -, * or / of fp32 operands equals the fp64 result rounded once
    to fp32, because 53 >= 2*24 + 2; this is how fp32 steps are emulated."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------- E2M1
def e2m1_encode(v):
    """Round scaled values to E2M1 codes (uint8, sign in bit 3).

    Round to nearest; a value exactly halfway between two magnitudes takes the
    code whose mantissa bit is 0 (even code index). Magnitudes above 6
    saturate to 6. The sign bit is copied from the input, also for zero."""
    v = _as_f64(v)
    a = np.abs(v)
    # number of decision points strictly below |v|
    idx = np.searchsorted(_E2M1_MIDPOINTS, a, side="left")
    on_mid = np.zeros(a.shape, dtype=bool)
    inside = idx < _E2M1_MIDPOINTS.size
    on_mid[inside] = a[inside] == _E2M1_MIDPOINTS[idx[inside]]
    # a tie sits between idx and idx+1: keep the even one
    idx = np.where(on_mid & (idx % 2 == 1), idx + 1, idx)
    sign = np.signbit(v).astype(np.uint8)
    return (idx.astype(np.uint8) | (sign << 3)).astype(np.uint8)


def e2m1_decode(codes):
    """Value of E2M1 code(s) as fp64."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def pack_nibbles(codes):
    """codes (..., 2n) -> bytes (..., n); element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """bytes (..., n) -> codes (..., 2n)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------- E8M0
def floor_log2(a):
    """floor(log2(a)) for a > 0, exact (from the binary exponent, no log)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))  # a = f * 2^e, f in [0.5, 1)
    return e.astype(np.int64) - 1


def e8m0_decode(byte):
    return np.ldexp(1.0, np.asarray(byte, dtype=np.int64) - 127)


def mx_shared_exponent(amax):
    """Shared exponent of MXFP4 blocks with maximum magnitude amax (>= 0):
    floor(log2 amax) minus the largest E2M1 exponent (2), clamped to
    [-127, 127]; an all-zero block gets -127 (scale byte 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    shared = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    shared[nz] = np.clip(floor_log2(amax[nz]) - 2, -127, 127)
    return shared


def mx_encode_at(x, shared):
    """E2M1 codes (unpacked, (rows, cols)) of a 2-D array whose blocks of 32
    along the last axis carry the given shared exponents (rows, cols/32)."""
    x = _as_f64(x)
    rows, cols = x.shape
    xb = x.reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    scaled = np.ldexp(xb, -np.asarray(shared, dtype=np.int64)[..., None])  # exact: power-of-two scaling
    return e2m1_encode(scaled).reshape(rows, cols)


def mx_quantize(x):
    """MXFP4: blocks of 32 along the last axis of a 2-D array.

    Returns (codes, scales): codes packed two per byte (rows, cols/2) and one
    E8M0 byte per block (rows, cols/32)."""
    x = _as_f64(x)
    rows, cols = x.shape
    if cols % MX_BLOCK:
        raise ValueError("MXFP4 needs the blocked axis to be a multiple of 32")
    amax = np.max(np.abs(x.reshape(rows, cols // MX_BLOCK, MX_BLOCK)), axis=-1)
    shared = mx_shared_exponent(amax)
    return pack_nibbles(mx_encode_at(x, shared)), (shared + 127).astype(np.uint8)


def mx_dequantize(codes, scales):
    """Inverse of mx_quantize: value(code) * 2^(byte - 127), exact in fp64."""
    vals = e2m1_decode(unpack_nibbles(codes))
    rows, cols = vals.shape
    sc = e8m0_decode(scales)
    return (vals.reshape(rows, cols // MX_BLOCK, MX_BLOCK) * sc[..., None]).reshape(rows, cols)


# --------------------------------------------------------------------- E4M3
def e4m3_encode(b):
    """Non-negative value(s) -> E4M3 byte(s), round to nearest even, saturate at 448."""
    b = _as_f64(b)
    if np.any(b < 0):
        raise ValueError("E4M3 block scales are non-negative")
    out = np.zeros(b.shape, dtype=np.uint8)
    pos = b > 0
    v = np.minimum(b[pos], E4M3_MAX)
    # binade of v; below the smallest normal 2^-6 the step stays 2^-9
    e = np.maximum(floor_log2(v), -6)
    step = np.ldexp(1.0, e - 3)  # three mantissa bits
    r = np.minimum(np.round(v / step) * step, E4M3_MAX)  # np.round: ties to even
    byte = np.zeros(r.shape, dtype=np.int64)
    nz = r > 0
    rn = r[nz]
    sub = rn < 2.0 ** -6
    eb = floor_log2(rn)
    mant = np.where(sub, rn / 2.0 ** -9, (np.ldexp(rn, -eb) - 1.0) * 8.0)
    field = np.where(sub, 0, eb + 7)
    byte[nz] = (field << 3) | mant.astype(np.int64)
    out[pos] = byte.astype(np.uint8)
    return out


def e4m3_decode(byte):
    b = np.asarray(byte, dtype=np.int64)
    field = (b >> 3) & 0xF
    mant = b & 7
    mag = np.where(field == 0, mant * 2.0 ** -9, (1.0 + mant / 8.0) * np.ldexp(1.0, field - 7))
    return np.where(b & 0x80, -mag, mag)


# -------------------------------------------------------------------- NVFP4
def nv_tensor_scale_of_max(a_t):
    """Per-tensor fp32 scale from the tensor's max magnitude a_t:
    max(f32(a_t / 2688), 2^-126), and 1 for a zero tensor."""
    a_t = float(a_t)
    if a_t == 0.0:
        return 1.0
    return float(max(f32(a_t / NV_TENSOR_DIVISOR), FP32_MIN_NORMAL))


def nv_tensor_scale(x):
    """Per-tensor fp32 scale s_t of an array (see nv_tensor_scale_of_max)."""
    x = _as_f64(x)
    return nv_tensor_scale_of_max(float(np.max(np.abs(x))) if x.size else 0.0)


def nv_block_scale(amax, s_t):
    """E4M3 scale bytes of NVFP4 blocks with maximum magnitude amax, given
    the tensor scale s_t: d = f32(6 s_t), b = f32(amax / d), e4m3(b)."""
    d = f32(6.0 * s_t)
    return e4m3_encode(f32(np.asarray(amax, dtype=np.float64) / d))


def nv_encode_at(x, sb, s_t):
    """E2M1 codes (unpacked, (rows, cols)) of a 2-D fp32-valued array whose
    blocks of 16 along the last axis carry the E4M3 scale bytes sb (rows,
    cols/16), with tensor scale s_t: den = f32(value(sb) s_t), then
    e2m1(f32(x / den)); a block whose scale is 0 gets +-0 codes."""
    x = _as_f64(x)
    rows, cols = x.shape
    xb = x.reshape(rows, cols // NV_BLOCK, NV_BLOCK)
    sbv = e4m3_decode(sb)
    den = f32(sbv * s_t)
    live = sbv > 0
    q = np.where(live[..., None], f32(xb / np.where(live, den, 1.0)[..., None]), 0.0 * xb)
    return e2m1_encode(q).reshape(rows, cols)


def nv_quantize(x, tensor_scale=None):
    """NVFP4: blocks of 16 along the last axis of a 2-D fp32-valued array.

    Returns (codes, scales, s_t): packed codes (rows, cols/2), one E4M3 byte per
    block (rows, cols/16) and the fp32 tensor scale. Each scale step is one
    correctly rounded fp32 operation, in this order:
      d = f32(6 * s_t); b = f32(amax_block / d); sb = e4m3(b);
      den = f32(value(sb) * s_t); code_i = e2m1(f32(x_i / den)).
    A block whose scale rounds to 0 gets +-0 codes. tensor_scale, if given,
    replaces s_t = nv_tensor_scale(x) (a scale taken from elsewhere)."""
    x = _as_f64(x)
    if np.any(x != f32(x)):
        raise ValueError("NVFP4 oracle takes fp32-representable inputs")
    rows, cols = x.shape
    if cols % NV_BLOCK:
        raise ValueError("NVFP4 needs the blocked axis to be a multiple of 16")
    s_t = nv_tensor_scale(x) if tensor_scale is None else float(tensor_scale)
    amax = np.max(np.abs(x.reshape(rows, cols // NV_BLOCK, NV_BLOCK)), axis=-1)
    sb = nv_block_scale(amax, s_t)
    return pack_nibbles(nv_encode_at(x, sb, s_t)), sb, np.float32(s_t)


def nv_dequantize(codes, scales, s_t):
    """value(code) * value(scale) * s_t, rounded once to fp32 (the product is exact in fp64)."""
    vals = e2m1_decode(unpack_nibbles(codes))
    rows, cols = vals.shape
    sc = e4m3_decode(scales)
    prod = vals.reshape(rows, cols // NV_BLOCK, NV_BLOCK) * sc[..., None] * float(s_t)
    return f32(prod.reshape(rows, cols))


# ------------------------------------------------------------------ dispatch
MXFP4, NVFP4 = "mxfp4", "nvfp4"


def quantize(x, fmt):
    """Quantize along the last axis. Returns dict(codes, scales, tensor_scale)."""
    if fmt == MXFP4:
        c, s = mx_quantize(x)
        return {"fmt": fmt, "codes": c, "scales": s, "tensor_scale": None}
    if fmt == NVFP4:
        c, s, t = nv_quantize(x)
        return {"fmt": fmt, "codes": c, "scales": s, "tensor_scale": float(t)}
    raise ValueError(fmt)


def dequantize(q):
    if q["fmt"] == MXFP4:
        return mx_dequantize(q["codes"], q["scales"])
    if q["fmt"] == NVFP4:
        return nv_dequantize(q["codes"], q["scales"], q["tensor_scale"])
    raise ValueError(q["fmt"])
