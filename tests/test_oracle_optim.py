"""Pins of the optimizer-side oracle terms (oracle/optim.py), CPU only."""
import numpy as np
import pytest

from oracle import optim as O
from oracle import split as S


def _lowrank(seed, m, n, s):
    g = np.random.Generator(np.random.PCG64(seed))
    U = np.linalg.qr(g.standard_normal((m, len(s))))[0]
    V = np.linalg.qr(g.standard_normal((n, len(s))))[0]
    return U, np.asarray(s, dtype=np.float64), V


def test_gamma_is_one_down_to_the_reference_and_capped_below():
    Sv = np.array([50.0, 20.0, 10.0, 5.0, 1.0, 0.1, 0.0])
    g = O.spectral_lr_gamma(Sv, 2, 8.0)
    assert np.allclose(g, [1.0, 1.0, 1.0, 2.0, 8.0, 8.0, 1.0])
    assert np.all(np.diff(g[:-1]) >= 0)  # nondecreasing toward the tail
    assert np.all(O.spectral_lr_gamma(Sv, 0, 1.0) == 1.0)
    with pytest.raises(ValueError):
        O.spectral_lr_gamma(Sv, 7, 2.0)


def test_rescale_with_unit_gamma_is_the_identity():
    g = np.random.Generator(np.random.PCG64(3))
    G = g.standard_normal((40, 30))
    U, Sv, V = _lowrank(4, 40, 30, [9.0, 4.0, 2.0])
    assert np.array_equal(O.spectral_lr_rescale(G, U, Sv, V, 2, 4.0), G)  # all S_i >= S[2]
    assert np.array_equal(O.spectral_lr_rescale(G, U, Sv, V, 0, 1.0), G)


def test_rescaled_low_rank_spectrum_matches_lapack():
    """G exactly of rank 6: the singular values of G' are S gamma (LAPACK)."""
    U, Sv, V = _lowrank(5, 64, 48, [40.0, 30.0, 8.0, 4.0, 1.0, 0.25])
    G = (U * Sv) @ V.T
    Gp = O.spectral_lr_rescale(G, U, Sv, V, 1, 16.0)
    want = np.sort(Sv * O.spectral_lr_gamma(Sv, 1, 16.0))[::-1]
    got = np.linalg.svd(Gp, compute_uv=False)[:6]
    assert np.allclose(got, want, rtol=1e-12)
    assert np.allclose(want, [40.0, 30.0, 30.0, 30.0, 16.0, 4.0])


def test_rescale_leaves_the_residual_of_a_split_untouched():
    """With the oracle's own split of G, G' - G lies in span(U) x span(V) and
    G' keeps R = G - U S V^T."""
    g = np.random.Generator(np.random.PCG64(6))
    U0, S0, V0 = _lowrank(7, 96, 80, [30.0, 20.0, 12.0, 6.0, 3.0])
    G = (U0 * S0) @ V0.T + 0.01 * g.standard_normal((96, 80))
    sp = S.spectral_split(G, 12, 5, omega=g.standard_normal((80, 12)))
    Gp = O.spectral_lr_rescale(G, sp["U"], sp["S"], sp["V"], 0, 100.0)
    Rp = Gp - (sp["U"] * (sp["S"] * O.spectral_lr_gamma(sp["S"], 0, 100.0))) @ sp["V"].T
    assert np.allclose(Rp, sp["R"], atol=1e-12)


def test_dual_range_loss_closed_forms():
    assert O.dual_range_loss(np.array([0.2, -0.5, 0.9]), 0.1, 1.0, 3.0, 2.0) == 0.0
    assert O.dual_range_loss(np.array([0.0]), 0.1, 1.0, 3.0, 2.0) == 0.0
    w = np.array([1.5, -0.02])
    want = 2.0 * 0.5 ** 2 + 3.0 * 0.08 ** 2
    assert abs(O.dual_range_loss(w, 0.1, 1.0, 3.0, 2.0) - want) < 1e-15
    assert O.dual_range_loss(-w, 0.1, 1.0, 3.0, 2.0) == O.dual_range_loss(w, 0.1, 1.0, 3.0, 2.0)


def test_dual_range_gradient_is_the_loss_derivative():
    """Central finite differences of the loss, away from the kinks."""
    g = np.random.Generator(np.random.PCG64(8))
    w = g.standard_normal(400) * 0.8
    args = (0.15, 1.1, 2.5, 1.7)
    kink = np.minimum.reduce([np.abs(np.abs(w) - 0.15), np.abs(np.abs(w) - 1.1), np.abs(w)])
    w = w[kink > 1e-3]
    grad = O.dual_range_grad(w, *args)
    h = 1e-6
    fd = np.array([(O.dual_range_loss(np.array([x + h]), *args) - O.dual_range_loss(np.array([x - h]), *args)) / (2 * h)
                   for x in w])
    assert np.allclose(grad, fd, rtol=1e-6, atol=1e-8)
    assert np.array_equal(O.dual_range_grad(-w, *args), -grad)
    # near-zero values are pushed away from zero, oversized ones toward the band
    assert np.all(grad[(np.abs(w) < 0.15)] * w[(np.abs(w) < 0.15)] < 0)
    assert np.all(grad[(np.abs(w) > 1.1)] * w[(np.abs(w) > 1.1)] > 0)


def test_a_planted_sign_mistake_fails_the_pins():
    """The finite-difference pin catches a flipped near-zero term."""
    w = np.array([0.05, -0.07, 1.4])
    args = (0.15, 1.1, 2.5, 1.7)
    wrong = 2.0 * 1.7 * np.maximum(np.abs(w) - 1.1, 0) * np.sign(w) + 2.0 * 2.5 * np.maximum(0.15 - np.abs(w), 0) * np.sign(w)
    h = 1e-6
    fd = np.array([(O.dual_range_loss(np.array([x + h]), *args) - O.dual_range_loss(np.array([x - h]), *args)) / (2 * h)
                   for x in w])
    assert not np.allclose(wrong, fd, rtol=1e-6, atol=1e-8)
    assert np.allclose(O.dual_range_grad(w, *args), fd, rtol=1e-6, atol=1e-8)
