"""Per-element check of a split's residual codes and scales against the oracle.

The HIP residual pass forms L = U W^T (W = f32(V diag(S))) on bf16 MFMA, with
U and W each carried as bf16 hi + lo and the three products Uh Wh + Uh Wl +
Ul Wh accumulated in fp32, then R = f32(A - L). Against L64 = U diag(S) V^T in
fp64 from the same fp32 factors, each element of L differs by at most
  2^-18 (the dropped Ul Wl) + 2 * 2^-18 (hi + lo leave 2^-18 of U and of W)
  + 2^-24 (W rounded to fp32) + 3 kp 2^-24 (fp32 sums over the 3 kp products,
  kp <= 96: 2^-15.8), all times sum_t |U_t| |W_t|:  below 2^-14.6 of it,
and the fp32 subtraction adds 2^-24 |R|. With R' = f32(A - L64) the check
takes, per element,
  tau = 2^-13 sum_t |U_t| |W_t| + 2^-22 |R'|        (1.5x the worst case)
and requires
  - every block scale of the GPU to lie between the oracle's scales of the
    block maxima of |R'| - tau and |R'| + tau (NVFP4: the tensor scale between
    those of max |R'| -+ tau over the whole tensor, and the block scales
    computed with the GPU's own tensor scale);
  - every code, read at the GPU's own block scale, to lie between the oracle's
    codes of R' - tau and R' + tau at that scale (E2M1 codes are monotone in
    the signed value; -0 sorts below +0).
Where the interval holds a single code (all but a small fraction of elements,
reported and bounded below), this is exact equality with the oracle."""
import numpy as np

from oracle import formats as F

TAU_REL = 2.0 ** -13   # of sum_t |U_t| |W_t|
TAU_R = 2.0 ** -22     # of |R'|
# The interval may admit two codes for at most this share of the elements: it
# is 0.1-0.2 % on the workload tensors, a few % where R is the noise floor
# thousands of times below L (a rank beyond the planted spectrum).
MAX_AMBIGUOUS = 0.05


def _key(codes):
    """Order of E2M1 codes by signed value, -0 just below +0 (injective)."""
    c = np.asarray(codes, dtype=np.uint8)
    v = 4.0 * F.e2m1_decode(c)
    return v + np.where(c == 0, 1.0, 0.0) - np.where(c == 8, 1.0, 0.0)


def residual_and_tau(A, U, S, V, idx=None, orient="n"):
    """R' = f32(A - U diag(S) V^T) and its tau, on rows idx of R (orient "n")
    or on rows idx of R^T (orient "t"), laid out along the blocked axis."""
    W = F.f32(V * S)
    if orient == "n":
        rows = np.arange(A.shape[0]) if idx is None else idx
        R = F.f32(A[rows] - (U[rows] * S) @ V.T)
        mag = np.abs(U[rows]) @ np.abs(W).T
    else:
        cols = np.arange(A.shape[1]) if idx is None else idx
        R = F.f32(A[:, cols] - (U * S) @ V[cols].T).T
        mag = (np.abs(U) @ np.abs(W[cols]).T).T
    return R, TAU_REL * mag + TAU_R * np.abs(R)


def tensor_max_bounds(A, U, S, V, chunk=1024):
    """Bounds on the GPU residual's max |R| over the whole tensor: the max
    of |R'| - tau and of |R'| + tau (rows in chunks to bound memory)."""
    lo = hi = 0.0
    for r0 in range(0, A.shape[0], chunk):
        R, tau = residual_and_tau(A, U, S, V, np.arange(r0, min(A.shape[0], r0 + chunk)))
        lo = max(lo, float(np.max(np.abs(R) - tau)))
        hi = max(hi, float(np.max(np.abs(R) + tau)))
    return max(lo, 0.0), hi


def check_codes(got, R, tau, fmt, max_bounds=None):
    """got: the GPU's fp4 dict restricted to the rows of R (codes (r, c/2),
    scales (r, c/B), tensor_scale). R, tau: from residual_and_tau.
    max_bounds: (lo, hi) from tensor_max_bounds (NVFP4 only; by default the
    rows of R are taken to be the whole tensor). Returns counts."""
    B = F.MX_BLOCK if fmt == "mxfp4" else F.NV_BLOCK
    r, c = R.shape
    gc = F.unpack_nibbles(got["codes"])
    gs = np.asarray(got["scales"])
    assert gc.shape == (r, c) and gs.shape == (r, c // B)
    Rb = np.abs(R).reshape(r, c // B, B)
    amax = Rb.max(axis=-1)
    taub = tau.reshape(r, c // B, B).max(axis=-1)
    amax_lo, amax_hi = np.maximum(amax - taub, 0.0), amax + taub
    lo_x, hi_x = R - tau, R + tau
    if fmt == "mxfp4":
        s_lo = F.mx_shared_exponent(amax_lo) + 127
        s_hi = F.mx_shared_exponent(amax_hi) + 127
        plain = F.quantize(R, fmt)
        se = gs.astype(np.int64) - 127
        c_lo, c_hi = F.mx_encode_at(lo_x, se), F.mx_encode_at(hi_x, se)
    else:
        st = float(np.float32(got["tensor_scale"]))
        whole = max_bounds is None
        if whole:
            max_bounds = (max(float(np.max(np.abs(R) - tau)), 0.0), float(np.max(np.abs(R) + tau)))
        st_lo, st_hi = (F.nv_tensor_scale_of_max(b) for b in max_bounds)
        assert st_lo <= st <= st_hi, "tensor scale %r outside [%r, %r]" % (st, st_lo, st_hi)
        s_lo, s_hi = F.nv_block_scale(amax_lo, st), F.nv_block_scale(amax_hi, st)
        plain = F.quantize(R, fmt) if whole else None
        c_lo, c_hi = F.nv_encode_at(lo_x, gs, st), F.nv_encode_at(hi_x, gs, st)
    bad_s = (gs < s_lo) | (gs > s_hi)
    assert not bad_s.any(), "%d block scales outside their interval (first at %s: got %d, allowed %d..%d)" % (
        bad_s.sum(), np.argwhere(bad_s)[0], gs[bad_s][0], s_lo[bad_s][0], s_hi[bad_s][0])
    kg, kl, kh = _key(gc), _key(c_lo), _key(c_hi)
    bad_c = (kg < kl) | (kg > kh)
    assert not bad_c.any(), "%d codes outside their interval (first at %s: got %d, allowed %d..%d)" % (
        bad_c.sum(), np.argwhere(bad_c)[0], gc[bad_c][0], c_lo[bad_c][0], c_hi[bad_c][0])
    ambiguous = float(np.mean(c_lo != c_hi))
    assert ambiguous <= MAX_AMBIGUOUS, "tau admits two codes for %.3g of the elements" % ambiguous
    out = {"codes": gc.size, "ambiguous": ambiguous, "scale_range_blocks": int(np.sum(s_lo != s_hi))}
    if plain is not None:
        out["differ_from_plain"] = int(np.sum(F.unpack_nibbles(plain["codes"]) != gc))
        out["scales_differ_from_plain"] = int(np.sum(plain["scales"] != gs))
    return out
