"""GPU parity of spectral_fp4_linear_fwd / _bwd against the oracle's fp64
GEMM over the same (GPU-produced) quantized records.

Gate: ||C_gpu - C_oracle||_F / ||C_oracle||_F <= 1e-3 (the GPU accumulates
exact FP4 products in fp32 and carries the low-rank correction with 16
significant bits, so the measured error is expected near 1e-6)."""
import numpy as np
import pytest
import torch

import synth
from oracle import linear as OL
from tests import _glue as G

pytestmark = pytest.mark.gpu

import fp4_spectral_split_amd as M

C_GATE = 1e-3


def _rel(got, want):
    return np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)


def _operand(t, orientations):
    if t.k:
        return G.split_gpu(t, orientations=orientations)
    return M.plain_operand(G.to_gpu(t), t.fmt, orientations)


def _small(seed, rows, cols, k, l, kind="planted", dtype="bf16", fmt="mxfp4"):
    return synth.small_case(seed, rows, cols, dtype, kind, k=k, l=l, n_dir=4, fmt=fmt)


# (288, 320, 416): contraction lengths that are not multiples of 128 and
# output tiles that are ragged against 256 x 256; (288, 512, 416): the forward
# contraction a multiple of 512 (the MXFP4 kernel with asynchronous LDS loads)
# with ragged output tiles; (512, 512, 1024): every contraction a multiple of
# 512, several stage groups deep.
SHAPES = {"ragged-k": (288, 320, 416), "fwd-k512": (288, 512, 416), "k512": (512, 512, 1024)}


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("kx,kw,kdy", [(8, 8, 8), (0, 8, 0), (8, 0, 8), (0, 0, 0), (16, 8, 4), (80, 72, 80)])
def test_linear_fwd_bwd_small(kx, kw, kdy, fmt, shape):
    Mt, K, N = SHAPES[shape]
    X = _small(201, Mt, K, kx, kx + 8, fmt=fmt)
    W = _small(202, N, K, kw, kw + 8, kind="powerlaw", fmt=fmt)
    dY = _small(203, Mt, N, kdy, kdy + 8, fmt=fmt)
    print("case", kx, kw, kdy, fmt, shape, flush=True)
    rx, rw, rd = _operand(X, ("n", "t")), _operand(W, ("n", "t")), _operand(dY, ("n", "t"))
    Y = M.spectral_fp4_linear_fwd(rx, rw)
    dX, dW = M.spectral_fp4_linear_bwd(rd, rx, rw)
    torch.cuda.synchronize()
    dx_, dw_, dd_ = G.record_to_dict(rx), G.record_to_dict(rw), G.record_to_dict(rd)
    for name, got, want in (("Y", Y, OL.linear_fwd(dx_, dw_)), ("dX", dX, OL.linear_bwd_dx(dd_, dw_)),
                            ("dW", dW, OL.linear_bwd_dw(dd_, dx_))):
        err = _rel(got.cpu().numpy().astype(np.float64), want)
        print("%s rel err %.3e" % (name, err), flush=True)
        assert err <= C_GATE, name
        assert err <= 1e-5, name  # far inside the gate: fp32-accurate everywhere


# NVFP4 forwards whose contraction is one to three 128-element stages of the
# ring kernel (its waits take their short-pipeline forms), with no correction
# stage, with two, and with ranks that differ; ragged rows and columns.
@pytest.mark.parametrize("K", [128, 256, 384])
@pytest.mark.parametrize("kx,kw", [(0, 0), (8, 8), (16, 8)])
def test_linear_nvfp4_short_contraction(K, kx, kw):
    X = _small(211, 288, K, kx, kx + 8, fmt="nvfp4")
    W = _small(212, 416, K, kw, kw + 8, kind="powerlaw", fmt="nvfp4")
    print("case", K, kx, kw, flush=True)
    rx, rw = _operand(X, ("n",)), _operand(W, ("n",))
    Y = M.spectral_fp4_linear_fwd(rx, rw)
    torch.cuda.synchronize()
    want = OL.linear_fwd(G.record_to_dict(rx), G.record_to_dict(rw))
    err = _rel(Y.cpu().numpy().astype(np.float64), want)
    print("Y rel err %.3e" % err, flush=True)
    assert err <= 1e-5


def test_linear_unsplit_is_a_plain_fp4_gemm_and_handles_empty():
    X = _small(204, 64, 256, 0, 0, kind="normal")
    W = _small(205, 96, 256, 0, 0, kind="normal")
    rx, rw = _operand(X, ("n",)), _operand(W, ("n",))
    Y = M.spectral_fp4_linear_fwd(rx, rw).cpu().numpy().astype(np.float64)
    want = OL.linear_fwd(G.record_to_dict(rx), G.record_to_dict(rw))
    assert _rel(Y, want) <= 1e-6
    e = M.plain_operand(torch.empty(0, 256, device="cuda"), "mxfp4", ("n",))
    out = M.spectral_fp4_linear_fwd(e, rw)
    assert out.shape == (0, 96)


def test_linear_deterministic():
    X = _small(206, 256, 256, 8, 16)
    W = _small(207, 256, 256, 8, 16, kind="powerlaw")
    rx, rw = _operand(X, ("n",)), _operand(W, ("n",))
    a = M.spectral_fp4_linear_fwd(rx, rw).clone()
    b = M.spectral_fp4_linear_fwd(rx, rw)
    assert torch.equal(a, b)


@pytest.mark.parametrize("K", [1024, 1536, 2560])
def test_linear_persistent_grid_with_ragged_tiles(K):
    """More output tiles than the MXFP4 kernel's persistent grid of 256
    workgroups (17 x 17 = 289), the last tile row and column ragged: the
    workgroups that take a second tile take the ragged ones, and the last
    stages of their first tile load the first stages of the second. K = 1536
    and 2560 give an odd number of four-stage scale groups per tile, so the
    second tile's scale groups sit in the other buffer of each pair. Rows of
    the first tile row, of tile row 8 (whose last two tiles are second
    tiles) and of the last two tile rows are checked against the oracle."""
    Mt, N = 4128, 4160
    X = _small(211, Mt, K, 8, 16)
    W = _small(212, N, K, 8, 16, kind="powerlaw")
    rx, rw = _operand(X, ("n",)), _operand(W, ("n",))
    Y = M.spectral_fp4_linear_fwd(rx, rw)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(0, 64), np.arange(2048, 2112), np.arange(Mt - 96, Mt)])
    got = Y[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    want = OL.gemm_nt(G.record_to_dict(rx), "n", G.record_to_dict(rw), "n", rows=rows)
    err = _rel(got, want)
    print("persistent ragged K=%d rel err %.3e" % (K, err), flush=True)
    assert err <= 1e-5


def _full(cfg, gemms, nrows=512):
    names = set()
    for _, a, _, b, _ in gemms:
        names |= {a, b}
    tens = {n: synth.make_tensor(cfg, n) for n in sorted(names)}
    recs = {n: _operand(t, ("n", "t")) for n, t in tens.items()}
    torch.cuda.synchronize()
    dicts = {n: G.record_to_dict(r) for n, r in recs.items()}
    for out, a, ao, b, bo in gemms:
        if ao == "n" and bo == "n":
            C = M.spectral_fp4_linear_fwd(recs[a], recs[b])
        elif ao == "n":
            C = _bwd_dx(recs[a], recs[b])
        else:
            C = _bwd_dw(recs[a], recs[b])
        torch.cuda.synchronize()
        rows = np.sort(np.random.Generator(np.random.PCG64(9)).choice(C.shape[0], min(nrows, C.shape[0]),
                                                                       replace=False))
        got = C[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        want = OL.gemm_nt(dicts[a], ao, dicts[b], bo, rows=rows)
        err = _rel(got, want)
        print("cfg %d %s rel err %.3e on %d rows" % (cfg, out, err, len(rows)), flush=True)
        assert err <= C_GATE
        del C


def _bwd_dx(dY, W):
    """dX through the public bwd entry point (dW skipped)."""
    fake_x = M.SplitRecord(dY.m, W.n, 0, W.fmt)
    return M.spectral_fp4_linear_bwd(dY, fake_x, W, need_dx=True, need_dw=False)[0]


def _bwd_dw(dY, X):
    """dW through the public bwd entry point (dX skipped)."""
    fake_w = M.SplitRecord(dY.n, X.n, 0, X.fmt)
    return M.spectral_fp4_linear_bwd(dY, X, fake_w, need_dx=False, need_dw=True)[1]


def test_linear_full_size_cfg2():
    """1.1B-class layer: X 4096 x 2048 unsplit with eight x20 outlier
    channels, W^T 5632 x 2048 split at k = 32 (K = 2048: the asynchronous-load
    MXFP4 kernel with a one-sided correction)."""
    _full(2, synth.GEMMS[2])


def test_linear_full_size_cfg3():
    _full(3, synth.GEMMS[3])


def test_linear_full_size_cfg4_up():
    _full(4, [g for g in synth.GEMMS[4] if g[0].endswith("_up")])


def test_linear_full_size_cfg4_down():
    _full(4, [g for g in synth.GEMMS[4] if g[0].endswith("_down")], nrows=256)


def test_linear_full_size_cfg5_nvfp4():
    """NVFP4 GEMMs (bf16 MFMA on exactly decoded operands) on the
    512-column-sampled splits of the FFN down projection."""
    _full(5, synth.GEMMS[5], nrows=256)
