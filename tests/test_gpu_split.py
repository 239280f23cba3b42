"""GPU parity of metis_split against the fp64 oracle on the same seeded A and
the same Omega (or column ids).

Gates: ||L_gpu - L_oracle||_F / ||A||_F <= 1e-3 with L = U S V^T from the
GPU's fp32 factors; U^T and V^T codes bit-exact against the oracle's
quantization of the GPU's own fp32 factors; every residual code and scale
(both orientations; NVFP4 tensor scales too) inside the interval the oracle
gives for R' -+ tau, R' = f32(A - U S V^T) in fp64 from the GPU factors and
tau the error bound of the kernel's bf16 hi/lo product (tests/_residual.py):
exact equality wherever that interval holds one code."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import split as S
from tests import _glue as G
from tests import _residual as RC

pytestmark = pytest.mark.gpu

import fp4_spectral_split_amd as M

L_GATE = 1e-3


def _oracle_split(t, q=0):
    A = t.values.astype(np.float64)
    if t.sketch == "gaussian":
        return A, S.spectral_split(A, t.l, t.k, omega=t.omega_values().astype(np.float64), q=q)
    return A, S.spectral_split(A, t.l, t.k, columns=t.columns, q=q)


def _sub(q, idx):
    """The rows idx of a GPU fp4 dict."""
    return {"codes": q["codes"][idx], "scales": q["scales"][idx], "tensor_scale": q["tensor_scale"]}


def _check_residuals(d, A, U, Sg, V, fmt, idx_n=None, idx_t=None, whole=True):
    """Per-element residual check of R_q (rows idx_n) and Rt_q (rows idx_t of
    R^T, i.e. columns of A); all rows when the index is None."""
    bounds = None
    if fmt == "nvfp4" and not whole:
        bounds = RC.tensor_max_bounds(A, U, Sg, V)
    for key, orient, idx in (("R_q", "n", idx_n), ("Rt_q", "t", idx_t)):
        if d[key] is None:
            continue
        R, tau = RC.residual_and_tau(A, U, Sg, V, idx, orient)
        got = d[key] if idx is None else _sub(d[key], idx)
        out = RC.check_codes(got, R, tau, fmt, max_bounds=bounds)
        print(key, out, flush=True)


def _check_split(t, rec, A, orc, fmt):
    U, Sg, V = G.factors_np(rec)
    k = t.k
    Lg = (U * Sg) @ V.T
    Lo = (orc["U"] * orc["S"]) @ orc["V"].T
    err = np.linalg.norm(Lg - Lo) / np.linalg.norm(A)
    print("L rel err %.3e   S rel err %.3e" % (err, np.max(np.abs(Sg - orc["S"]) / orc["S"][0])), flush=True)
    assert err <= L_GATE
    assert np.allclose(Sg, orc["S"], rtol=0, atol=1e-4 * orc["S"][0])
    assert int(rec.info.item()) == 0
    # sign convention on the GPU's own factors
    for i in range(k):
        j = int(np.argmax(np.abs(U[:, i])))
        assert U[j, i] >= 0
    assert np.allclose(U.T @ U, np.eye(k), atol=1e-5)
    d = G.record_to_dict(rec)
    # factor codes: oracle quantization of the GPU's fp32 factors, bit-exact
    for key, X in (("Ut_q", U.T), ("Vt_q", V.T)):
        want = F.quantize(F.f32(X), fmt)
        assert np.array_equal(d[key]["codes"], want["codes"]), key
        assert np.array_equal(d[key]["scales"], want["scales"]), key
        if fmt == "nvfp4":
            assert np.float32(d[key]["tensor_scale"]) == np.float32(want["tensor_scale"])
    _check_residuals(d, A, U, Sg, V, fmt)
    return err


CASES = {
    "cfg1-W-f32": lambda: synth.make_tensor(1, "W"),
    "ragged-powerlaw-bf16": lambda: synth.small_case(101, 288, 416, "bf16", "powerlaw", k=16, l=24),
    "planted-f32": lambda: synth.small_case(102, 320, 192, "f32", "planted", k=8, l=16, n_dir=4),
    "wide-l96": lambda: synth.small_case(103, 512, 384, "bf16", "planted", k=64, l=96, n_dir=8),
    "sampled-columns": lambda: synth.small_case(104, 256, 320, "bf16", "planted", k=8, l=24, n_dir=4,
                                                sketch="columns"),
    "nvfp4": lambda: synth.small_case(105, 288, 256, "bf16", "powerlaw", k=16, l=32, fmt="nvfp4"),
    "wide-columns-l160": lambda: synth.small_case(108, 640, 448, "bf16", "planted", k=32, l=160, n_dir=8,
                                                  sketch="columns"),
    "wide-gaussian-l128-nvfp4": lambda: synth.small_case(109, 384, 320, "bf16", "powerlaw", k=16, l=128,
                                                         fmt="nvfp4"),
    # factor rank 65..96: the residual's KP = 96 instance
    "k80-l96": lambda: synth.small_case(110, 384, 352, "bf16", "planted", k=80, l=96, n_dir=8),
    "k80-l96-nvfp4-f32": lambda: synth.small_case(111, 320, 288, "f32", "powerlaw", k=80, l=96, fmt="nvfp4"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_split_parity_small(name):
    t = CASES[name]()
    if t.k and not t.orientations:
        t.orientations = ("n", "t")
    print("case", name, t.shape, flush=True)
    A, orc = _oracle_split(t)
    rec = G.split_gpu(t, orientations=("n", "t"))
    torch.cuda.synchronize()
    _check_split(t, rec, A, orc, t.fmt)


def test_split_is_bitwise_deterministic():
    t = CASES["ragged-powerlaw-bf16"]()
    r1 = G.record_to_dict(G.split_gpu(t, orientations=("n", "t")))
    r2 = G.record_to_dict(G.split_gpu(t, orientations=("n", "t")))
    for key in ("Ut_q", "Vt_q", "R_q", "Rt_q"):
        assert np.array_equal(r1[key]["codes"], r2[key]["codes"])
        assert np.array_equal(r1[key]["scales"], r2[key]["scales"])
    assert np.array_equal(r1["S"], r2["S"])


def test_split_zero_matrix_reports_rank_deficiency():
    t = synth.small_case(106, 128, 96, "bf16", "zero", k=4, l=8)
    rec = G.split_gpu(t, orientations=("n", "t"))
    torch.cuda.synchronize()
    assert int(rec.info.item()) == 1
    assert np.all(rec.S.cpu().numpy() == 0)
    d = G.record_to_dict(rec)
    assert np.all(F.dequantize(d["R_q"]) == 0) and np.all(F.dequantize(d["Rt_q"]) == 0)


def test_split_rank_deficient_input_keeps_reconstruction():
    """A with rank 3 < l: the sketch is rank deficient; L still matches the oracle."""
    g = np.random.Generator(np.random.PCG64(107))
    A = (synth.orthonormal(g, 192, 3) * np.array([9.0, 4.0, 1.0])) @ synth.orthonormal(g, 160, 3).T
    t = synth.Tensor("T", A, "f32", k=4, l=8, sketch="gaussian",
                     omega=synth.bf16_bits(g.standard_normal((160, 8))), orientations=("n", "t"))
    Ao, orc = _oracle_split(t)
    rec = G.split_gpu(t)
    torch.cuda.synchronize()
    U, Sg, V = G.factors_np(rec)
    err = np.linalg.norm((U * Sg) @ V.T - (orc["U"] * orc["S"]) @ orc["V"].T) / np.linalg.norm(Ao)
    assert err <= L_GATE


def _sampled(n, seed, count=256):
    return np.sort(np.random.Generator(np.random.PCG64(seed)).choice(n, min(count, n), replace=False))


def _full_size(t, q=0):
    """Split at full size in both orientations; the L gate, the U^T codes, and
    the residual codes of R on 256 sampled rows and of R^T on 256 sampled
    columns (multi-tile residual runs: the paired tiles, the prefetch and the
    U reload all take part)."""
    print("case", t.name, t.shape, "k", t.k, "l", t.l, t.fmt, "q", q, flush=True)
    A, orc = _oracle_split(t, q=q)
    rec = G.split_gpu(t, orientations=("n", "t"), q=q)
    torch.cuda.synchronize()
    U, Sg, V = G.factors_np(rec)
    Lg = (U * Sg) @ V.T
    Lo = (orc["U"] * orc["S"]) @ orc["V"].T
    err = np.linalg.norm(Lg - Lo) / np.linalg.norm(A)
    gap = (orc["sigma_B"][t.k - 1] - orc["sigma_B"][t.k]) / orc["sigma_B"][t.k - 1]
    print("L rel err %.3e  (sigma_k relative gap %.2e)" % (err, gap), flush=True)
    assert err <= L_GATE
    assert int(rec.info.item()) == 0
    d = G.record_to_dict(rec)
    for key, X in (("Ut_q", U.T), ("Vt_q", V.T)):
        want = F.quantize(F.f32(X), t.fmt)
        assert np.array_equal(d[key]["codes"], want["codes"]), key
        assert np.array_equal(d[key]["scales"], want["scales"]), key
        if t.fmt == "nvfp4":
            assert np.float32(d[key]["tensor_scale"]) == np.float32(want["tensor_scale"])
    _check_residuals(d, A, U, Sg, V, t.fmt, _sampled(t.shape[0], 5), _sampled(t.shape[1], 6), whole=False)


@pytest.mark.parametrize("cfg,name", [(2, "W"), (3, "W"), (3, "X"), (4, "W_up"), (4, "X_down"), (4, "dY_up")])
def test_split_parity_full_size(cfg, name):
    """Full workload sizes (MXFP4, Gaussian sketch, k = 32 / 64)."""
    _full_size(synth.make_tensor(cfg, name))


def test_split_parity_full_size_k80_l96():
    """8192 x 4096 bf16 (the FFN input's shape) at k = 80, l = 96: the
    residual's KP = 96 instance at full size."""
    t = synth.make_tensor(4, "X_up")
    t.k, t.l = 80, 96
    t.omega = synth.gaussian_omega(4, "omega.X", t.shape[1], 96)
    _full_size(t)


@pytest.mark.parametrize("name", ["dY", "W", "X"])
def test_split_parity_full_size_nvfp4_sampled_512(name):
    """NVFP4 + 512 sampled columns (wide sketch, global-memory small SVD):
    factor codes and tensor scales bit-exact, the residual's tensor scale and
    codes of both orientations per element."""
    _full_size(synth.make_tensor(5, name))


@pytest.mark.parametrize("q", [1, 2])
@pytest.mark.parametrize("name", ["ragged-powerlaw-bf16", "planted-f32", "sampled-columns", "nvfp4", "wide-l96"])
def test_split_power_iterations_parity_small(name, q):
    """q power iterations (metis_split_power) against the oracle's subspace
    iteration with the same q, to the same gates as q = 0."""
    t = CASES[name]()
    t.orientations = ("n", "t")
    print("case", name, "q", q, t.shape, flush=True)
    A, orc = _oracle_split(t, q=q)
    rec = G.split_gpu(t, orientations=("n", "t"), q=q)
    torch.cuda.synchronize()
    _check_split(t, rec, A, orc, t.fmt)


def test_split_power_iterations_full_size():
    """8192 x 4096 bf16 (LLaMA-3-8B FFN input), k = 64, l = 80, q = 1."""
    _full_size(synth.make_tensor(4, "X_up"), q=1)
