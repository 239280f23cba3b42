"""Out-of-range stores: every output of the split, the mean split, the
quantizer and the GEMMs is placed inside a larger buffer filled with a
sentinel, on shapes whose tiles are ragged against every kernel's tiling
(edge workgroups run on clamped loads and must drop their stores). The
guard bytes before and after each output, and the columns between the
output's width and its leading dimension, must come back untouched, and the
results must equal those of a run on plainly allocated outputs bit for bit."""
import numpy as np
import pytest
import torch

import synth
from tests import _glue as G

pytestmark = pytest.mark.gpu

import fp4_spectral_split_amd as M

PAD = 256          # guard bytes on each side (keeps every view 256-byte aligned)
SENT = 0xA5


class Guarded:
    """A device buffer of PAD + nbytes + PAD sentinel bytes and a typed view
    of its middle."""

    def __init__(self, numel, dtype, device):
        esz = torch.empty(0, dtype=dtype).element_size()
        nbytes = numel * esz
        self.raw = torch.full((PAD + nbytes + PAD,), SENT, dtype=torch.uint8, device=device)
        self.view = self.raw[PAD:PAD + nbytes].view(dtype)

    def intact(self):
        r = self.raw.cpu().numpy()
        return bool(np.all(r[:PAD] == SENT) and np.all(r[len(r) - PAD:] == SENT))


def _guarded_fp4(fmt, rows, cols, device, guards):
    B = M.BLOCK[fmt]
    codes = Guarded(rows * cols // 2, torch.uint8, device)
    scales = Guarded(rows * (cols // B), torch.uint8, device)
    guards += [codes, scales]
    ts = None
    if fmt == M.NVFP4:
        g = Guarded(1, torch.float32, device)
        guards.append(g)
        ts = g.view
    return M.Fp4Tensor(fmt, rows, cols, codes.view, scales.view, ts)


def _guarded_split(m, n, k, fmt, orientations, device):
    fmt = M._FMT[fmt]
    guards = []
    rec = M.SplitRecord(m, n, k, fmt)
    if k:
        for name, numel in (("U", m * k), ("S", k), ("V", n * k)):
            g = Guarded(numel, torch.float32, device)
            guards.append(g)
            setattr(rec, name, g.view)
        rec.U, rec.V = rec.U.view(m, k), rec.V.view(n, k)
        rec.Ut_q = _guarded_fp4(fmt, k, m, device, guards)
        rec.Vt_q = _guarded_fp4(fmt, k, n, device, guards)
    if "n" in orientations:
        rec.R_q = _guarded_fp4(fmt, m, n, device, guards)
    if "t" in orientations:
        rec.Rt_q = _guarded_fp4(fmt, n, m, device, guards)
    g = Guarded(1, torch.int32, device)
    g.view.zero_()
    guards.append(g)
    rec.info = g.view
    return rec, guards


def _same_record(a, b):
    da, db = G.record_to_dict(a), G.record_to_dict(b)
    assert np.array_equal(da["S"], db["S"])
    for key in ("Ut_q", "Vt_q", "R_q", "Rt_q"):
        if da[key] is None:
            assert db[key] is None
            continue
        assert np.array_equal(da[key]["codes"], db[key]["codes"]), key
        assert np.array_equal(da[key]["scales"], db[key]["scales"]), key
        assert da[key]["tensor_scale"] == db[key]["tensor_scale"], key
    if a.k:
        assert torch.equal(a.U, b.U) and torch.equal(a.V, b.V)
    assert int(a.info.item()) == int(b.info.item())


# (rows, cols): 288 and 416 leave partial 128 x 64 residual tiles and an odd
# count of row tiles against the residual's 2 x 4 tile blocks; 160 x 96 is
# smaller than one block; 544 x 224 gives a 32-row tail; 352 x 224 an odd
# count of row tiles, each partial against a 64-column tile edge.
SPLIT_CASES = {
    "ragged-288x416": lambda: synth.small_case(301, 288, 416, "bf16", "powerlaw", k=16, l=24),
    "tiny-160x96-f32": lambda: synth.small_case(302, 160, 96, "f32", "planted", k=4, l=8, n_dir=2),
    "tail-544x224-columns": lambda: synth.small_case(303, 544, 224, "bf16", "planted", k=8, l=24, n_dir=4,
                                                     sketch="columns"),
    "nvfp4-352x224": lambda: synth.small_case(304, 352, 224, "bf16", "powerlaw", k=8, l=16, fmt="nvfp4"),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_split_writes_stay_inside_outputs(name):
    t = SPLIT_CASES[name]()
    m, n = t.shape
    print("case", name, t.shape, flush=True)
    A = G.to_gpu(t)
    om = G.omega_gpu(t) if t.sketch == "gaussian" else None
    cols = G.columns_gpu(t) if t.sketch != "gaussian" else None
    rec, guards = _guarded_split(m, n, t.k, t.fmt, ("n", "t"), A.device)
    M.metis_split(A, t.l, t.k, t.fmt, omega=om, columns=cols, out=rec)
    ref = M.metis_split(A, t.l, t.k, t.fmt, omega=om, columns=cols, orientations=("n", "t"))
    torch.cuda.synchronize()
    assert all(g.intact() for g in guards)
    _same_record(rec, ref)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_mean_split_and_quant_writes_stay_inside_outputs(fmt):
    t = synth.small_case(305, 288, 416, "bf16", "powerlaw", k=4, l=8, fmt=fmt)
    m, n = t.shape
    A = G.to_gpu(t)
    rec, guards = _guarded_split(m, n, 1, fmt, ("n", "t"), A.device)
    M.metis_mean_split(A, fmt, out=rec)
    ref = M.metis_mean_split(A, fmt, orientations=("n", "t"))
    f = M._FMT[fmt]
    for transpose in (False, True):
        rows, cols = (n, m) if transpose else (m, n)
        qg = []
        q = M.fp4_block_quant(A, fmt, transpose=transpose, out=_guarded_fp4(f, rows, cols, A.device, qg))
        qr = M.fp4_block_quant(A, fmt, transpose=transpose)
        torch.cuda.synchronize()
        assert all(g.intact() for g in qg), transpose
        assert torch.equal(q.codes, qr.codes) and torch.equal(q.scales, qr.scales)
    torch.cuda.synchronize()
    assert all(g.intact() for g in guards)
    _same_record(rec, ref)


def _padded_out(rows, cols, extra, device):
    """rows x cols view (leading dimension cols + extra) of a NaN-filled
    buffer with one spare row on each side."""
    buf = torch.full((rows + 2, cols + extra), float("nan"), dtype=torch.float32, device=device)
    return buf, buf[1:rows + 1, :cols]


def _outside_untouched(buf, rows, cols):
    b = buf.cpu()
    return bool(torch.isnan(b[0]).all() and torch.isnan(b[rows + 1]).all() and torch.isnan(b[1:rows + 1, cols:]).all())


# (M, K, N) as in the GEMM parity tests: ragged contraction and output tiles,
# and a forward contraction that is a multiple of 512 (the MXFP4 kernel with
# asynchronous LDS loads) with ragged output tiles.
@pytest.mark.parametrize("shape", [(288, 320, 416), (288, 512, 416)])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_gemm_writes_stay_inside_outputs(shape, fmt):
    Mt, K, N = shape
    print("case", shape, fmt, flush=True)
    X = synth.small_case(311, Mt, K, "bf16", "planted", k=8, l=16, n_dir=4, fmt=fmt)
    W = synth.small_case(312, N, K, "bf16", "powerlaw", k=8, l=16, fmt=fmt)
    dY = synth.small_case(313, Mt, N, "bf16", "planted", k=8, l=16, n_dir=4, fmt=fmt)
    rx, rw, rd = (G.split_gpu(t, orientations=("n", "t")) for t in (X, W, dY))
    dev = rx.R_q.codes.device
    yb, y = _padded_out(Mt, N, 7, dev)
    xb, dx = _padded_out(Mt, K, 5, dev)
    wb, dw = _padded_out(N, K, 3, dev)
    M.spectral_fp4_linear_fwd(rx, rw, out=y)
    M.spectral_fp4_linear_bwd(rd, rx, rw, dx=dx, dw=dw)
    y0 = M.spectral_fp4_linear_fwd(rx, rw)
    dx0, dw0 = M.spectral_fp4_linear_bwd(rd, rx, rw)
    torch.cuda.synchronize()
    for name, buf, view, ref in (("Y", yb, y, y0), ("dX", xb, dx, dx0), ("dW", wb, dw, dw0)):
        assert _outside_untouched(buf, *ref.shape), name
        assert torch.equal(view.cpu(), ref.cpu()), name


def test_dequant_writes_stay_inside_output():
    t = synth.small_case(314, 288, 416, "bf16", "powerlaw", k=4, l=8)
    A = G.to_gpu(t)
    q = M.fp4_block_quant(A, "mxfp4")
    buf, view = _padded_out(288, 416, 9, A.device)
    M.fp4_block_dequant(q, out=view)
    ref = M.fp4_block_dequant(q)
    torch.cuda.synchronize()
    assert _outside_untouched(buf, 288, 416)
    assert torch.equal(view.cpu(), ref.cpu())
