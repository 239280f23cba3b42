"""Pins of the oracle's quantized linear layer (two routes, special cases),
and the direction-only check of the method's tail-spectrum claim."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import linear as L
from oracle import split as S


def _record(seed, m, n, k, l, fmt="mxfp4", kind="planted"):
    t = synth.small_case(seed, m, n, dtype="bf16", kind=kind, k=k, l=l, fmt=fmt)
    A = t.values.astype(np.float64)
    if k == 0:
        return S.quantize_record(fmt, A)
    r = S.spectral_split(A, l, k, omega=t.omega_values().astype(np.float64))
    return S.quantize_record(fmt, r["R"], r["U"], r["S"], r["V"])


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("ka,kb", [(8, 8), (0, 8), (8, 0), (0, 0), (4, 12)])
def test_expansion_route_equals_reconstruction_route(fmt, ka, kb):
    X = _record(31, 96, 64, ka, ka + 4 if ka else 0, fmt)
    W = _record(32, 160, 64, kb, kb + 4 if kb else 0, fmt)
    dY = _record(33, 96, 160, ka, ka + 4 if ka else 0, fmt)
    for a, ao, b, bo in [(X, "n", W, "n"), (dY, "n", W, "t"), (dY, "t", X, "t")]:
        c1 = L.gemm_nt(a, ao, b, bo)
        c2 = L.gemm_nt_expanded(a, ao, b, bo)
        assert np.abs(c1 - c2).max() <= 1e-12 * np.abs(c1).max()


def test_unsplit_operands_give_a_plain_dequantized_gemm():
    X = _record(34, 64, 96, 0, 0)
    W = _record(35, 32, 96, 0, 0)
    want = F.mx_dequantize(X["R_q"]["codes"], X["R_q"]["scales"]) @ \
        F.mx_dequantize(W["R_q"]["codes"], W["R_q"]["scales"]).T
    assert np.array_equal(L.linear_fwd(X, W), want)


def test_identity_input_returns_the_dequantized_weight():
    W = _record(36, 64, 96, 8, 12)
    I = S.quantize_record("mxfp4", np.eye(96))
    assert np.array_equal(F.mx_dequantize(I["R_q"]["codes"], I["R_q"]["scales"]), np.eye(96))
    Y = L.linear_fwd(I, W)
    assert np.allclose(Y, L.operand(W, "n").T, rtol=0, atol=1e-13)


def test_sampled_rows_match_full_product():
    X = _record(37, 64, 96, 8, 12)
    W = _record(38, 64, 96, 8, 12)
    rows = np.array([0, 5, 63])
    assert np.allclose(L.linear_fwd(X, W, rows), L.linear_fwd(X, W)[rows], rtol=1e-14, atol=1e-12)


def test_orientation_records_differ_but_each_reconstructs():
    """The transposed residual is a separate quantization, close to R^T."""
    t = synth.small_case(39, 128, 96, kind="normal", k=0)
    A = t.values.astype(np.float64)
    rec = S.quantize_record("mxfp4", A)
    Rn = L.residual(rec, "n")
    Rt = L.residual(rec, "t")
    assert not np.array_equal(Rn, Rt.T)
    assert np.linalg.norm(Rt.T - A) / np.linalg.norm(A) < 0.2


def test_split_narrows_the_residual_range():
    """SII post §2.4(1): the long-tail residual has a narrow range."""
    t = synth.small_case(40, 512, 256, kind="planted", k=8, l=16, n_dir=8)
    A = t.values.astype(np.float64)
    r = S.spectral_split(A, t.l, t.k, omega=t.omega_values().astype(np.float64))
    assert np.abs(r["R"]).max() < 0.5 * np.abs(A).max()


def test_tail_spectrum_distortion_direction():
    """Direction-only check of the pages' claim (SII post §2.3 and §2.4(1);
    Metis abstract): block quantization inflates the tail singular values, and
    the split keeps them closer. Magnitudes are parity unpinned (the pages
    print none)."""
    W = synth.make_tensor(1, "W")
    A = W.values.astype(np.float64)
    sA = np.linalg.svd(A, compute_uv=False)
    direct = F.mx_dequantize(*F.mx_quantize(A))
    r = S.spectral_split(A, W.l, W.k, omega=W.omega_values().astype(np.float64))
    rec = S.quantize_record("mxfp4", r["R"], r["U"], r["S"], r["V"], orientations=("n",))
    split = L.operand(rec, "n")
    s_direct = np.linalg.svd(direct, compute_uv=False)
    s_split = np.linalg.svd(split, compute_uv=False)
    for i in (63, 127):
        infl_direct = s_direct[i] / sA[i]
        infl_split = s_split[i] / sA[i]
        assert infl_direct > 1.5 * infl_split
