"""GPU parity of metis_mean_split (the mean-residual split) against the
fp64 oracle (oracle.split.mean_split).

Gates: U == 1 and S == 1 exactly; V (the column mean, summed in fp64 and
rounded once) within one fp32 ulp of the oracle's mean; factor and residual
codes bit-exact against the oracle's quantization of the GPU's own fp32
factors and of f32(A - 1 V^T), which the GPU forms as one correctly rounded
fp32 subtraction. A linear layer with mean-split operands matches the
oracle's fp64 GEMM over the same records (relative error <= 1e-5)."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import linear as OL
from oracle import split as S
from tests import _glue as G

pytestmark = pytest.mark.gpu

import fp4_spectral_split_amd as M


def _mean_dominated(seed, rows, cols, offset=4.0, dtype="bf16"):
    """N(0,1) entries plus a per-column offset: activations whose extremes
    come from the mean, the case the split targets."""
    g = np.random.Generator(np.random.PCG64(seed))
    A = g.standard_normal((rows, cols)) + offset * g.standard_normal(cols)
    if dtype == "bf16":
        bits = synth.bf16_bits(A)
        return synth.bf16_value(bits).astype(np.float64), torch.from_numpy(bits.view(np.int16).copy()).view(
            torch.bfloat16).to(G.device())
    A32 = A.astype(np.float32)
    return A32.astype(np.float64), torch.from_numpy(A32).to(G.device())


def _check(A, rec, fmt, rows=None):
    U, Sg, V = G.factors_np(rec)
    assert np.all(U == 1.0) and np.all(Sg == 1.0)
    mu = S.mean_split(A)["mu"]
    ulp = np.spacing(np.abs(mu).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(V[:, 0] - mu) <= ulp), np.max(np.abs(V[:, 0] - mu) / ulp)
    d = G.record_to_dict(rec)
    for key, X in (("Ut_q", U.T), ("Vt_q", V.T)):
        want = F.quantize(F.f32(X), fmt)
        assert np.array_equal(d[key]["codes"], want["codes"]), key
        assert np.array_equal(d[key]["scales"], want["scales"]), key
    Rp = F.f32(A - U @ V.T)
    for key, X in (("R_q", Rp), ("Rt_q", Rp.T)):
        if d[key] is None:
            continue
        want = F.quantize(X, fmt)
        got = d[key]
        if rows is not None and key == "R_q":
            assert np.array_equal(got["codes"][rows], want["codes"][rows]), key
            assert np.array_equal(got["scales"][rows], want["scales"][rows]), key
        else:
            assert np.array_equal(got["codes"], want["codes"]), key
            assert np.array_equal(got["scales"], want["scales"]), key
        if fmt == "nvfp4":
            assert np.float32(got["tensor_scale"]) == np.float32(want["tensor_scale"])


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(288, 416), (160, 96), (32, 32)])
def test_mean_split_parity(rows, cols, dtype, fmt):
    A, Ag = _mean_dominated(300 + rows + cols, rows, cols, dtype=dtype)
    print("case", rows, cols, dtype, fmt, flush=True)
    rec = M.metis_mean_split(Ag, fmt)
    torch.cuda.synchronize()
    _check(A, rec, fmt)


def test_mean_split_constant_matrix_has_zero_residual():
    Ag = torch.full((64, 64), 3.0, dtype=torch.float32, device=G.device())
    rec = M.metis_mean_split(Ag, "mxfp4")
    torch.cuda.synchronize()
    assert torch.all(rec.V == 3.0)
    d = G.record_to_dict(rec)
    assert np.all(F.dequantize(d["R_q"]) == 0) and np.all(F.dequantize(d["Rt_q"]) == 0)


def test_mean_split_full_size_activation():
    """8192 x 4096 bf16 (the LLaMA-3-8B FFN input at 8192 tokens); residual
    codes compared on 256 sampled rows, the transposed orientation whole."""
    A, Ag = _mean_dominated(311, 8192, 4096)
    rec = M.metis_mean_split(Ag, "mxfp4")
    torch.cuda.synchronize()
    rows = np.sort(np.random.Generator(np.random.PCG64(6)).choice(8192, 256, replace=False))
    _check(A, rec, "mxfp4", rows=rows)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_linear_with_mean_split_operands(fmt):
    """Y = X W^T, dX = dY W, dW = dY^T X with X and dY mean-split and W
    spectrally split, against the oracle's GEMM over the same records."""
    Mt, K, N = 288, 512, 416
    X, Xg = _mean_dominated(320, Mt, K)
    dY, dYg = _mean_dominated(321, Mt, N, offset=0.5)
    W = synth.small_case(322, N, K, "bf16", "powerlaw", k=8, l=16, fmt=fmt)
    rx = M.metis_mean_split(Xg, fmt)
    rd = M.metis_mean_split(dYg, fmt)
    rw = G.split_gpu(W, orientations=("n", "t"), fmt=fmt)
    Y = M.spectral_fp4_linear_fwd(rx, rw)
    dX, dW = M.spectral_fp4_linear_bwd(rd, rx, rw)
    torch.cuda.synchronize()
    dx_, dw_, dd_ = G.record_to_dict(rx), G.record_to_dict(rw), G.record_to_dict(rd)
    for name, got, want in (("Y", Y, OL.linear_fwd(dx_, dw_)), ("dX", dX, OL.linear_bwd_dx(dd_, dw_)),
                            ("dW", dW, OL.linear_bwd_dw(dd_, dx_))):
        g = got.cpu().numpy().astype(np.float64)
        err = np.linalg.norm(g - want) / np.linalg.norm(want)
        print("%s rel err %.3e" % (name, err), flush=True)
        assert err <= 1e-5, name


def test_mean_split_is_bitwise_deterministic():
    A, Ag = _mean_dominated(330, 256, 256)
    a = G.record_to_dict(M.metis_mean_split(Ag, "mxfp4"))
    b = G.record_to_dict(M.metis_mean_split(Ag, "mxfp4"))
    for key in ("Vt_q", "R_q", "Rt_q"):
        assert np.array_equal(a[key]["codes"], b[key]["codes"])
