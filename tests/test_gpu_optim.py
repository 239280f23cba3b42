"""GPU parity of the optimizer-side kernels (metis_spectral_lr_rescale,
metis_dual_range_reg) against the fp64 oracle (oracle/optim.py).

Dual-range regularizer: the gradient is formed in fp64 in the oracle's
operation order and rounded once, so it must equal f32(oracle) bit for bit
(also when accumulated into an existing fp32 gradient: f32(g0 + oracle));
the loss, an fp64 sum in another order, within 1e-12 relative.

Spectral learning rate: the GPU sums the rank-k term in fp32 (ascending i)
with gamma from an fp32 division; against f32(oracle) from the GPU's own
split factors each element may differ by at most
  2^-22 |G'| + (k + 4) 2^-24 sum_i |U_i| |S_i (gamma_i - 1) V_i| * gamma_max
(fp32 rounding of the sum, of its terms and of gamma), stated in the test."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import optim as O
from tests import _glue as G

pytestmark = pytest.mark.gpu

import fp4_spectral_split_amd as M


def _dev(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda(), \
            synth.bf16_value(synth.bf16_bits(x)).astype(np.float64)
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    return torch.from_numpy(x32).cuda(), x32.astype(np.float64)


REG = (0.05, 1.5, 3.0, 0.7)  # tau_lo, tau_hi, lam_lo, lam_hi


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(96, 160), (1, 8), (257, 1032)])
def test_dual_range_matches_oracle(dtype, shape):
    g = np.random.Generator(np.random.PCG64(401))
    w = g.standard_normal(shape) * np.exp(g.standard_normal(shape))
    w[0, :4] = [0.0, -0.0, 0.05, -1.5]  # zero, signed zero, both band edges
    Wd, W64 = _dev(w, dtype)
    print("case dual-range", dtype, shape, flush=True)
    loss, grad = M.metis_dual_range_reg(Wd, *REG)
    torch.cuda.synchronize()
    want_g = F.f32(O.dual_range_grad(W64, *[float(np.float32(v)) for v in REG]))
    want_l = O.dual_range_loss(W64, *[float(np.float32(v)) for v in REG])
    assert np.array_equal(grad.cpu().numpy().astype(np.float64), want_g)
    assert abs(loss.item() - want_l) <= 1e-12 * max(abs(want_l), 1e-300)
    # accumulate into an existing gradient
    g0 = torch.from_numpy(g.standard_normal(shape).astype(np.float32)).cuda()
    base = g0.cpu().numpy().astype(np.float64)
    M.metis_dual_range_reg(Wd, *REG, grad=g0, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(g0.cpu().numpy().astype(np.float64),
                          F.f32(base + O.dual_range_grad(W64, *[float(np.float32(v)) for v in REG])))


def test_dual_range_full_size_weight():
    """The LLaMA-3-8B FFN up-projection weight (14336 x 4096 bf16), gradient
    checked on 256 sampled rows, loss in full."""
    t = synth.make_tensor(4, "W_up")
    Wd = G.to_gpu(t)
    reg = (0.002, 0.05, 10.0, 100.0)
    loss, grad = M.metis_dual_range_reg(Wd, *reg)
    torch.cuda.synchronize()
    W64 = t.values.astype(np.float64)
    reg32 = [float(np.float32(v)) for v in reg]
    rows = np.sort(np.random.Generator(np.random.PCG64(11)).choice(W64.shape[0], 256, replace=False))
    got = grad[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    assert np.array_equal(got, F.f32(O.dual_range_grad(W64[rows], *reg32)))
    want_l = O.dual_range_loss(W64, *reg32)
    print("loss %.6e (oracle %.6e)" % (loss.item(), want_l), flush=True)
    assert abs(loss.item() - want_l) <= 1e-12 * abs(want_l)


def _check_rescale(Gd, G64, rec, r_ref, gmax):
    U, Sg, V = G.factors_np(rec)
    want = F.f32(O.spectral_lr_rescale(G64, U, Sg, V, r_ref, gmax))
    got = Gd.cpu().numpy().astype(np.float64)
    c = Sg * (O.spectral_lr_gamma(Sg, r_ref, gmax) - 1.0)
    mag = np.abs(U) @ np.abs(V * c).T
    tol = 2.0 ** -22 * np.abs(want) + (rec.k + 4) * 2.0 ** -24 * gmax * mag
    err = np.abs(got - want)
    print("rescale max err / tol %.3f, changed %.3g of G" % (np.max(err / np.maximum(tol, 1e-300)),
                                                              np.mean(got != G64)), flush=True)
    assert np.all(err <= tol)
    return got


@pytest.mark.parametrize("r_ref,gmax", [(0, 4.0), (3, 16.0), (7, 1.0)])
def test_spectral_lr_rescale_small(r_ref, gmax):
    """The split of a ragged fp32 gradient-like matrix, then the rescale."""
    g = np.random.Generator(np.random.PCG64(402))
    A = g.standard_normal((320, 224)) * 0.01
    U0 = np.linalg.qr(g.standard_normal((320, 8)))[0]
    V0 = np.linalg.qr(g.standard_normal((224, 8)))[0]
    A += (U0 * np.array([8.0, 5.0, 3.0, 2.0, 1.0, 0.5, 0.25, 0.125])) @ V0.T
    t = synth.Tensor("G", A, "f32", k=8, l=16, sketch="gaussian", omega=synth.bf16_bits(g.standard_normal((224, 16))),
                     orientations=("n",))
    rec = G.split_gpu(t)
    Gd = torch.from_numpy(t.values.copy()).cuda()
    print("case rescale", r_ref, gmax, flush=True)
    M.metis_spectral_lr_rescale(Gd, rec, r_ref, gmax)
    torch.cuda.synchronize()
    got = _check_rescale(Gd, t.values.astype(np.float64), rec, r_ref, gmax)
    if gmax == 1.0:
        assert np.array_equal(got, t.values.astype(np.float64))


def test_spectral_lr_rescale_full_size_dw():
    """dW of the LLaMA-3-8B FFN down projection (4096 x 14336 fp32, the
    backward GEMM's output), split at k = 64, l = 80, then rescaled with the
    reference at rank 8; checked on 256 sampled rows."""
    tw, tx, td = synth.make_tensor(4, "W_down"), synth.make_tensor(4, "X_down"), synth.make_tensor(4, "dY_down")
    rw = G.split_gpu(tw, orientations=("n", "t"))
    rx = G.split_gpu(tx, orientations=("n", "t"))
    rd = G.split_gpu(td, orientations=("n", "t"))
    _, dW = M.spectral_fp4_linear_bwd(rd, rx, rw, need_dx=False, need_dw=True)
    torch.cuda.synchronize()
    dW64 = dW.cpu().numpy().astype(np.float64)
    del rw, rx, rd
    om = synth.gaussian_omega(4, "omega.W", dW.shape[1], 80)
    t = synth.Tensor("dW", dW64, "f32", k=64, l=80, sketch="gaussian", omega=om, orientations=("n",))
    rec = G.split_gpu(t)
    print("case rescale full-size dW", dW.shape, flush=True)
    M.metis_spectral_lr_rescale(dW, rec, 8, 8.0)
    torch.cuda.synchronize()
    rows = np.sort(np.random.Generator(np.random.PCG64(12)).choice(dW.shape[0], 256, replace=False))
    U, Sg, V = G.factors_np(rec)

    class Sub:
        pass
    sub = Sub()
    sub.k = rec.k
    sub.U, sub.S, sub.V = (torch.from_numpy(U[rows].astype(np.float32)), torch.from_numpy(Sg.astype(np.float32)),
                           torch.from_numpy(V.astype(np.float32)))
    got_rows = dW[torch.from_numpy(rows).cuda()]
    _check_rescale(got_rows, dW64[rows], sub, 8, 8.0)
