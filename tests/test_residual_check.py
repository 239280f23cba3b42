"""The per-element residual check used by the GPU split tests must accept the
oracle's own quantization and reject plausible mistakes: a code moved to its
neighbour, a block scale one binade off, a wrong NVFP4 tensor scale (CPU only:
the 'GPU' records here are the oracle's, with one mistake planted)."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import split as S
from tests import _residual as RC


@pytest.fixture(scope="module")
def case():
    t = synth.small_case(301, 256, 320, "bf16", "planted", k=16, l=24, n_dir=4)
    A = t.values.astype(np.float64)
    o = S.spectral_split(A, t.l, t.k, omega=t.omega_values().astype(np.float64))
    return A, F.f32(o["U"]), F.f32(o["S"]), F.f32(o["V"])


def _got(R, fmt):
    q = F.quantize(R, fmt)
    return {"codes": q["codes"].copy(), "scales": q["scales"].copy(), "tensor_scale": q["tensor_scale"]}


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("orient", ["n", "t"])
def test_oracle_quantization_passes(case, fmt, orient):
    R, tau = RC.residual_and_tau(*case, orient=orient)
    out = RC.check_codes(_got(R, fmt), R, tau, fmt)
    assert out["ambiguous"] < 0.01


def _unambiguous_element(R, tau, fmt, got):
    B = F.MX_BLOCK if fmt == "mxfp4" else F.NV_BLOCK
    gs = got["scales"]
    if fmt == "mxfp4":
        se = gs.astype(np.int64) - 127
        lo, hi = F.mx_encode_at(R - tau, se), F.mx_encode_at(R + tau, se)
    else:
        st = got["tensor_scale"]
        lo, hi = F.nv_encode_at(R - tau, gs, st), F.nv_encode_at(R + tau, gs, st)
    codes = F.unpack_nibbles(got["codes"])
    ok = (lo == hi) & ((codes & 7) > 0) & ((codes & 7) < 7)
    i, j = np.argwhere(ok)[len(np.argwhere(ok)) // 2]
    return i, j


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_a_neighbouring_code_is_rejected(case, fmt):
    R, tau = RC.residual_and_tau(*case)
    got = _got(R, fmt)
    i, j = _unambiguous_element(R, tau, fmt, got)
    codes = F.unpack_nibbles(got["codes"])
    codes[i, j] += 1
    got["codes"] = F.pack_nibbles(codes)
    with pytest.raises(AssertionError, match="codes outside"):
        RC.check_codes(got, R, tau, fmt)


def test_a_scale_one_binade_off_is_rejected(case):
    R, tau = RC.residual_and_tau(*case, orient="t")
    got = _got(R, "mxfp4")
    got["scales"][3, 2] += 1
    with pytest.raises(AssertionError, match="block scales outside"):
        RC.check_codes(got, R, tau, "mxfp4")


def test_a_wrong_tensor_scale_is_rejected(case):
    R, tau = RC.residual_and_tau(*case)
    got = _got(R, "nvfp4")
    got["tensor_scale"] = float(np.float32(got["tensor_scale"] * 1.01))
    with pytest.raises(AssertionError, match="tensor scale"):
        RC.check_codes(got, R, tau, "nvfp4")


def test_tau_bounds_the_hi_lo_product_error(case):
    """The error model behind tau: L from bf16 hi + lo U and W with the three
    products Uh Wh + Uh Wl + Ul Wh summed in fp32 (emulated here with numpy
    float32 sums) stays inside tau - 2^-22 |R'| everywhere."""
    A, U, Sg, V = case
    W = F.f32(V * Sg)

    def bf16(x):
        return synth.bf16_value(synth.bf16_bits(x)).astype(np.float64)

    Uh, Wh = bf16(U), bf16(W)
    Ul, Wl = bf16(U - Uh), bf16(W - Wh)
    L32 = np.zeros((A.shape[0], A.shape[1]), dtype=np.float32)
    for t in range(U.shape[1]):
        for a, b in ((Uh, Wh), (Uh, Wl), (Ul, Wh)):
            L32 = (L32 + np.outer(a[:, t], b[:, t]).astype(np.float32)).astype(np.float32)
    L64 = (U * Sg) @ V.T
    R, tau = RC.residual_and_tau(A, U, Sg, V)
    err = np.abs(L32.astype(np.float64) - L64)
    assert np.all(err <= tau - RC.TAU_R * np.abs(R))
    assert np.max(err / (tau - RC.TAU_R * np.abs(R))) < 0.5
