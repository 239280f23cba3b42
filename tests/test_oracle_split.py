"""Pins of the oracle's randomized split against LAPACK and closed forms."""
import numpy as np
import pytest

import synth
from oracle import split as S


def _rand(seed, m, n):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal((m, n))


@pytest.mark.parametrize("m,l", [(40, 7), (300, 16), (97, 33)])
def test_householder_matches_lapack_qr(m, l):
    Y = _rand(1, m, l)
    Q, R = S.householder_qr(Y)
    Qn, Rn = np.linalg.qr(Y)
    d = np.sign(np.diag(Rn)) * np.sign(np.diag(R))
    assert np.allclose(Q, Qn * d, atol=1e-12)
    assert np.allclose(R, (Rn.T * d).T, atol=1e-12)
    assert np.allclose(Q.T @ Q, np.eye(l), atol=1e-13)
    assert np.allclose(Q @ R, Y, atol=1e-12)


def test_householder_rank_deficient_keeps_orthonormal_q():
    Y = _rand(2, 50, 6)
    Y[:, 3] = 0.0
    Y[:, 5] = Y[:, 0] * 2.0
    Q, R = S.householder_qr(Y)
    assert np.allclose(Q.T @ Q, np.eye(6), atol=1e-13)
    assert np.allclose(Q @ R, Y, atol=1e-12)


@pytest.mark.parametrize("l,n", [(8, 40), (16, 300), (33, 97), (12, 12)])
def test_jacobi_svd_matches_lapack(l, n):
    B = _rand(3, l, n)
    Ub, sig, W = S.jacobi_svd(B)
    Un, sn, Vtn = np.linalg.svd(B, full_matrices=False)
    assert np.allclose(sig, sn, rtol=1e-12, atol=0)
    # each singular vector equal up to sign (distinct singular values here)
    dots = np.abs(np.sum(Ub * Un, axis=0))
    assert np.allclose(dots, 1.0, atol=1e-10)
    assert np.allclose((Ub * sig) @ W.T, B, atol=1e-12)
    assert np.allclose(Ub.T @ Ub, np.eye(l), atol=1e-13)


@pytest.mark.parametrize("l,n", [(6, 100), (16, 300)])
def test_small_svd_wide_route_equals_direct_jacobi_and_lapack(l, n):
    B = _rand(11, l, n) * np.exp(np.linspace(0, -6, l))[:, None]
    U1, s1, W1 = S.small_svd(B)          # QR-compressed route (n > 4 l)
    U2, s2, W2 = S.jacobi_svd(B)         # direct route
    sn = np.linalg.svd(B, compute_uv=False)
    assert np.allclose(s1, sn, rtol=1e-11, atol=0) and np.allclose(s1, s2, rtol=1e-11, atol=0)
    d = np.sign(np.sum(U1 * U2, axis=0))
    assert np.allclose(U1, U2 * d, atol=1e-9) and np.allclose(W1, W2 * d, atol=1e-9)
    assert np.allclose((U1 * s1) @ W1.T, B, atol=1e-12)


def test_library_route_agrees_with_own_routines_at_l160(monkeypatch):
    """Wide sketches use LAPACK for QR and SVD; on a 160-column case both
    routes give the same split (and the planted values)."""
    g = np.random.Generator(np.random.PCG64(12))
    U = synth.orthonormal(g, 640, 10)
    V = synth.orthonormal(g, 480, 10)
    s = 100.0 * np.arange(1, 11) ** -1.0
    A = (U * s) @ V.T + 1e-3 * g.standard_normal((640, 480))
    J = np.sort(g.choice(480, 160, replace=False))
    r_lib = S.spectral_split(A, 160, 12, columns=J)
    monkeypatch.setattr(S, "LIBRARY_ROUTE_MIN_L", 10 ** 9)
    r_own = S.spectral_split(A, 160, 12, columns=J)
    assert np.allclose(r_lib["S"], r_own["S"], rtol=1e-10, atol=0)
    assert np.allclose(r_lib["R"], r_own["R"], atol=1e-10)
    assert np.allclose(r_lib["S"][:10], s, rtol=1e-3)


def test_jacobi_svd_zero_row_gives_zero_sigma():
    B = _rand(4, 6, 30)
    B[2] = 0.0
    Ub, sig, W = S.jacobi_svd(B)
    assert sig[-1] == 0.0
    assert np.allclose((Ub * sig) @ W.T, B, atol=1e-12)


@pytest.mark.parametrize("m,n", [(64, 48), (48, 64)])
def test_full_rank_split_leaves_no_residual(m, n):
    A = _rand(5, m, n)
    k = min(m, n)
    omega = _rand(6, n, k)
    r = S.spectral_split(A, k, k, omega=omega)
    assert np.linalg.norm(r["R"]) / np.linalg.norm(A) <= 1e-12


def test_planted_rank8_singular_values_recovered():
    g = np.random.Generator(np.random.PCG64(8))
    U = synth.orthonormal(g, 300, 8)
    V = synth.orthonormal(g, 200, 8)
    s = np.array([90.0, 41.0, 17.0, 9.0, 5.5, 2.0, 1.25, 0.5])
    A = (U * s) @ V.T
    omega = synth.bf16_value(synth.bf16_bits(g.standard_normal((200, 16)))).astype(np.float64)
    r = S.spectral_split(A, 16, 8, omega=omega)
    assert np.allclose(r["S"], s, rtol=1e-10, atol=0)
    # and the planted subspace itself: U_k U_k^T = U U^T
    assert np.allclose(r["U"] @ r["U"].T, U @ U.T, atol=1e-10)


def test_split_invariants_noisy_powerlaw():
    t = synth.small_case(21, 384, 256, dtype="bf16", kind="powerlaw", k=16, l=24)
    A = t.values.astype(np.float64)
    r = S.spectral_split(A, t.l, t.k, omega=t.omega_values().astype(np.float64))
    Q, U, Sk, V, R = r["Q"], r["U"], r["S"], r["V"], r["R"]
    sA = np.linalg.svd(A, compute_uv=False)
    assert np.allclose(Q.T @ Q, np.eye(t.l), atol=1e-13)
    assert np.all(r["sigma_B"] <= sA[: t.l] * (1 + 1e-12))          # interlacing
    assert np.abs(U.T @ R).max() <= 1e-10 * np.abs(A).max()          # U_k^T R = 0
    lhs = np.linalg.norm(R) ** 2
    assert abs(lhs - (np.linalg.norm(A) ** 2 - np.sum(Sk ** 2))) <= 1e-10 * np.linalg.norm(A) ** 2
    assert np.linalg.norm(R) >= np.sqrt(np.sum(sA[t.k:] ** 2)) * (1 - 1e-12)  # Eckart-Young
    assert np.all(np.diff(Sk) <= 0)


def test_sign_convention():
    t = synth.small_case(22, 128, 96, dtype="f32", kind="planted", k=4, l=8, n_dir=4)
    A = t.values.astype(np.float64)
    om = t.omega_values().astype(np.float64)
    r = S.spectral_split(A, t.l, t.k, omega=om)
    U = r["U"]
    for i in range(t.k):
        j = int(np.argmax(np.abs(U[:, i])))
        assert U[j, i] > 0
    # the split of -A negates V, not U
    r2 = S.spectral_split(-A, t.l, t.k, omega=om)
    assert np.allclose(r2["U"], U, atol=1e-10) and np.allclose(r2["V"], -r["V"], atol=1e-10)


def test_column_sampling_sketch_is_a_gather():
    A = _rand(9, 30, 50)
    J = np.array([1, 4, 9, 20, 49], dtype=np.int32)
    assert np.array_equal(S.sketch(A, columns=J), A[:, J])
    r = S.spectral_split(A, 5, 3, columns=J)
    # the captured subspace is the span of the sampled columns
    P = r["Q"] @ r["Q"].T
    assert np.allclose(P @ A[:, J], A[:, J], atol=1e-12)


def test_bad_arguments():
    A = _rand(10, 20, 10)
    with pytest.raises(ValueError):
        S.spectral_split(A, 11, 4, omega=_rand(1, 10, 11))
    with pytest.raises(ValueError):
        S.spectral_split(A, 4, 5, omega=_rand(1, 10, 4))
    with pytest.raises(ValueError):
        S.sketch(A)


def test_power_iterations_reach_the_exact_top_k():
    """Subspace iteration (q >= 1): on a slowly decaying spectrum one sketch
    pass leaves a visible gap to the exact top-k singular values; a few
    iterations close it to LAPACK precision, monotonically in q."""
    g = np.random.Generator(np.random.PCG64(41))
    m, n, k, l = 200, 160, 8, 12
    U = synth.orthonormal(g, m, 60)
    V = synth.orthonormal(g, n, 60)
    A = (U * (np.arange(1, 61) ** -0.5)) @ V.T
    sA = np.linalg.svd(A, compute_uv=False)
    om = g.standard_normal((n, l))
    errs = []
    for q in range(0, 8):
        r = S.spectral_split(A, l, k, omega=om, q=q)
        errs.append(np.max(np.abs(r["S"] - sA[:k]) / sA[0]))
        # the residual never beats Eckart-Young and is monotone toward it
        assert np.linalg.norm(r["R"]) >= np.sqrt(np.sum(sA[k:] ** 2)) * (1 - 1e-12)
    assert errs[0] > 1e-3
    assert all(b <= a * 1.0001 for a, b in zip(errs, errs[1:]))
    r = S.spectral_split(A, l, k, omega=om, q=30)
    assert np.allclose(r["S"], sA[:k], rtol=1e-9, atol=0)
    assert np.allclose(np.abs(r["U"].T @ np.linalg.svd(A)[0][:, :k]), np.eye(k), atol=1e-6)


def test_mean_split_closed_form():
    """Averis split: mu is the column mean, the residual is de-meaned, and
    the parts add back to A; U = 1 and S = 1 quantize exactly."""
    from oracle import formats as F
    g = np.random.Generator(np.random.PCG64(31))
    A = g.standard_normal((96, 64)) + np.linspace(-3.0, 5.0, 64)  # columns with distinct offsets
    r = S.mean_split(A)
    assert np.allclose(r["mu"], A.mean(axis=0), rtol=0, atol=1e-14)
    assert np.allclose(r["R"].sum(axis=0), 0.0, atol=1e-12)
    assert np.array_equal(r["R"] + np.ones((96, 1)) @ r["V"].T, A) or np.allclose(
        r["R"] + np.ones((96, 1)) @ r["V"].T, A, rtol=0, atol=1e-15)
    for fmt in ("mxfp4", "nvfp4"):
        rec = S.quantize_record(fmt, r["R"], r["U"], r["S"], r["V"])
        Uq = F.dequantize(rec["Ut_q"])
        assert np.allclose(Uq, 1.0, rtol=2e-7, atol=0)
    # a constant matrix is all mean: zero residual
    r0 = S.mean_split(np.full((32, 32), 2.5))
    assert np.all(r0["R"] == 0.0) and np.all(r0["mu"] == 2.5)


# --- planted mistakes: each pin above must notice a plausible slip ---------
def test_pins_catch_a_planted_mistake_unsorted_sigma(monkeypatch):
    real = S.jacobi_svd

    def unsorted(B, **kw):
        Ub, sig, W = real(B, **kw)
        return Ub[:, ::-1], sig[::-1], W[:, ::-1]

    monkeypatch.setattr(S, "jacobi_svd", unsorted)
    with pytest.raises(AssertionError):
        test_planted_rank8_singular_values_recovered()


def test_pins_catch_a_planted_mistake_transposed_projection(monkeypatch):
    real = S.householder_qr

    def bad_qr(Y):
        Q, R = real(Y)
        return Q[:, ::-1] * 0.999, R  # slightly non-orthonormal basis

    monkeypatch.setattr(S, "householder_qr", bad_qr)
    with pytest.raises(AssertionError):
        test_split_invariants_noisy_powerlaw()
