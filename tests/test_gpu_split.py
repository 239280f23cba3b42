"""GPU parity of metis_split against the fp64 oracle on the same seeded A and
the same Omega (or column ids).

Gates: ||L_gpu - L_oracle||_F / ||A||_F <= 1e-3 with L = U S V^T from the
GPU's fp32 factors; U^T and V^T codes bit-exact against the oracle's
quantization of the GPU's own fp32 factors; residual codes equal to the
oracle's quantization of R' = A - U S V^T (fp64 from the GPU factors) except
at values that sit on a rounding decision point within the fp32 accuracy of
R (adjacent codes only, at most 1e-3 of them)."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import split as S
from tests import _glue as G

pytestmark = pytest.mark.gpu

import fp4_spectral_split_amd as M

L_GATE = 1e-3


def _oracle_split(t, q=0):
    A = t.values.astype(np.float64)
    if t.sketch == "gaussian":
        return A, S.spectral_split(A, t.l, t.k, omega=t.omega_values().astype(np.float64), q=q)
    return A, S.spectral_split(A, t.l, t.k, columns=t.columns, q=q)


def _check_codes_near(got, want, fmt, rows=None):
    """Residual codes: equal, or adjacent where the fp32 R sits on a decision point."""
    gc = F.unpack_nibbles(got["codes"])
    wc = F.unpack_nibbles(want["codes"])
    gs, ws = got["scales"], want["scales"]
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    assert gc.shape == wc.shape
    code_mis = gc != wc
    scale_mis = gs != ws
    assert scale_mis.mean() <= 1e-3, "scale mismatch rate %g" % scale_mis.mean()
    assert code_mis.mean() <= 1e-3, "code mismatch rate %g" % code_mis.mean()
    # mismatching codes are neighbours on the grid (or a signed zero)
    dm = np.abs((gc & 7).astype(int) - (wc & 7).astype(int))
    assert np.all(dm[code_mis] <= 1)


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
    Rp = F.f32(A - Lg)
    if d["R_q"] is not None:
        _check_codes_near(d["R_q"], F.quantize(Rp, fmt), fmt)
    if d["Rt_q"] is not None:
        _check_codes_near(d["Rt_q"], F.quantize(Rp.T, fmt), fmt)
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


@pytest.mark.parametrize("cfg,name", [(2, "W"), (3, "W"), (3, "X"), (4, "W_up"), (4, "X_down")])
def test_split_parity_full_size(cfg, name):
    """Full workload sizes; residual codes compared on 256 sampled rows."""
    t = synth.make_tensor(cfg, name)
    print("case cfg", cfg, name, t.shape, flush=True)
    A, orc = _oracle_split(t)
    rec = G.split_gpu(t, orientations=("n",))
    torch.cuda.synchronize()
    U, Sg, V = G.factors_np(rec)
    Lg = (U * Sg) @ V.T
    Lo = (orc["U"] * orc["S"]) @ orc["V"].T
    err = np.linalg.norm(Lg - Lo) / np.linalg.norm(A)
    gap = (orc["sigma_B"][t.k - 1] - orc["sigma_B"][t.k]) / orc["sigma_B"][t.k - 1]
    print("L rel err %.3e  (sigma_k relative gap %.2e)" % (err, gap), flush=True)
    assert err <= L_GATE
    d = G.record_to_dict(rec)
    want = F.quantize(F.f32(U.T), "mxfp4")
    assert np.array_equal(d["Ut_q"]["codes"], want["codes"])
    rows = np.sort(np.random.Generator(np.random.PCG64(5)).choice(t.shape[0], 256, replace=False))
    Rp = F.f32(A[rows] - (U[rows] * Sg) @ V.T)
    _check_codes_near(d["R_q"], F.quantize(Rp, "mxfp4"), "mxfp4", rows=rows)


@pytest.mark.parametrize("name", ["dY", "W", "X"])
def test_split_parity_full_size_nvfp4_sampled_512(name):
    """NVFP4 + 512 sampled columns (wide sketch, global-memory small SVD)."""
    t = synth.make_tensor(5, name)
    print("case cfg5", name, t.shape, flush=True)
    A, orc = _oracle_split(t)
    rec = G.split_gpu(t, orientations=("n",))
    torch.cuda.synchronize()
    U, Sg, V = G.factors_np(rec)
    err = np.linalg.norm((U * Sg) @ V.T - (orc["U"] * orc["S"]) @ orc["V"].T) / np.linalg.norm(A)
    print("L rel err %.3e" % err, flush=True)
    assert err <= L_GATE
    assert int(rec.info.item()) == 0
    d = G.record_to_dict(rec)
    want = F.quantize(F.f32(V.T), "nvfp4")
    assert np.array_equal(d["Vt_q"]["codes"], want["codes"]) and np.array_equal(d["Vt_q"]["scales"], want["scales"])
    assert np.float32(d["Vt_q"]["tensor_scale"]) == np.float32(want["tensor_scale"])


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
    t = synth.make_tensor(4, "X_up")
    A, orc = _oracle_split(t, q=1)
    rec = G.split_gpu(t, orientations=("n",), q=1)
    torch.cuda.synchronize()
    U, Sg, V = G.factors_np(rec)
    Lg = (U * Sg) @ V.T
    err = np.linalg.norm(Lg - (orc["U"] * orc["S"]) @ orc["V"].T) / np.linalg.norm(A)
    print("L rel err %.3e" % err, flush=True)
    assert err <= L_GATE
    rows = np.sort(np.random.Generator(np.random.PCG64(7)).choice(t.shape[0], 256, replace=False))
    Rp = F.f32(A[rows] - (U[rows] * Sg) @ V.T)
    _check_codes_near(G.record_to_dict(rec)["R_q"], F.quantize(Rp, "mxfp4"), "mxfp4", rows=rows)


@pytest.mark.parametrize("name", ["ragged-powerlaw-bf16", "planted-f32", "sampled-columns", "nvfp4", "wide-columns-l160"])
def test_split_in_two_calls_equals_one_call(name):
    """metis_split_begin + metis_split_finish (each on its own stream, the
    second waiting for the first) give metis_split's record bit for bit."""
    t = CASES[name]()
    print("case", name, t.shape, flush=True)
    A = G.to_gpu(t)
    kw = {"omega": G.omega_gpu(t)} if t.sketch == "gaussian" else {"columns": G.columns_gpu(t)}
    ref = M.metis_split(A, t.l, t.k, t.fmt, orientations=("n", "t"), **kw)
    two = M.SplitInTwo(A, t.l, t.k, t.fmt, orientations=("n", "t"), **kw)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        two.begin()
    e = torch.cuda.Event()
    e.record(s1)
    s2.wait_event(e)
    with torch.cuda.stream(s2):
        rec = two.finish()
    torch.cuda.synchronize()
    a, b = G.record_to_dict(rec), G.record_to_dict(ref)
    assert np.array_equal(a["S"], b["S"])
    for key in ("Ut_q", "Vt_q", "R_q", "Rt_q"):
        assert np.array_equal(a[key]["codes"], b[key]["codes"]), key
        assert np.array_equal(a[key]["scales"], b[key]["scales"]), key
        assert a[key]["tensor_scale"] == b[key]["tensor_scale"], key
    assert torch.equal(rec.U, ref.U) and torch.equal(rec.V, ref.V)
    assert int(rec.info.item()) == int(ref.info.item())
