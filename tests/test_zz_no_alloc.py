"""spectral_fp4_linear_fwd_noalloc (the forward with its workspace in the
library's static per-GPU scratch) against spectral_fp4_linear_fwd (workspace
argument) through the C ABI: the same kernels, so the outputs must agree bit
for bit. Two calls in a row, the second on smaller operands, so the second
reads scratch that still holds the first call's larger contents."""
import numpy as np
import pytest
import torch

import synth
from tests import _glue as G

pytestmark = pytest.mark.gpu

import fp4_spectral_split_amd as M


def _records(seed, rows, K, N, kx, kw, fmt):
    X = synth.small_case(seed, rows, K, "bf16", "planted", k=kx, l=kx + 8, n_dir=4, fmt=fmt)
    W = synth.small_case(seed + 1, N, K, "bf16", "powerlaw", k=kw, l=kw + 8, fmt=fmt)
    rx = G.split_gpu(X, orientations=("n",)) if kx else M.plain_operand(G.to_gpu(X), fmt, ("n",))
    rw = G.split_gpu(W, orientations=("n",)) if kw else M.plain_operand(G.to_gpu(W), fmt, ("n",))
    return rx, rw


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_noalloc_fwd_equals_fwd_twice_shrinking(fmt):
    first = _records(801, 1024, 1536, 1280, 16, 24, fmt)
    second = _records(803, 288, 512, 416, 8, 8, fmt)
    outs = []
    for rx, rw in (first, second):
        print("case noalloc", fmt, rx.m, rx.n, rw.m, flush=True)
        y_na = torch.full((rx.m, rw.m), float("nan"), dtype=torch.float32, device="cuda")
        M.spectral_fp4_linear_fwd_noalloc(rx, rw, y_na)
        outs.append(y_na)
    for (rx, rw), y_na in zip((first, second), outs):
        y = M.spectral_fp4_linear_fwd(rx, rw)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        assert torch.equal(y_na, y)


def test_noalloc_fwd_full_size_then_small():
    """A 8192-token forward of the LLaMA-3-8B FFN up projection (both operands
    split, k = 64: 30 MB of scratch), then a small unsplit one."""
    tx, tw = synth.make_tensor(4, "X_up"), synth.make_tensor(4, "W_up")
    rx = G.split_gpu(tx, orientations=("n",))
    rw = G.split_gpu(tw, orientations=("n",))
    small = _records(805, 64, 256, 96, 0, 0, "mxfp4")
    y_big = torch.empty(rx.m, rw.m, dtype=torch.float32, device="cuda")
    print("case noalloc full size", rx.m, rx.n, rw.m, flush=True)
    M.spectral_fp4_linear_fwd_noalloc(rx, rw, y_big)
    y_small = torch.empty(64, 96, dtype=torch.float32, device="cuda")
    M.spectral_fp4_linear_fwd_noalloc(small[0], small[1], y_small)
    ref_big = M.spectral_fp4_linear_fwd(rx, rw)
    ref_small = M.spectral_fp4_linear_fwd(small[0], small[1])
    torch.cuda.synchronize()
    assert torch.equal(y_big, ref_big)
    assert torch.equal(y_small, ref_small)


def test_noalloc_fwd_rejects_requests_beyond_its_scratch():
    """k = 96 on 32768 x 4096 by 65536 x 4096 needs more than 64 MiB: the
    call returns METIS_ERR_TOO_LARGE and launches nothing."""
    L = M.load()
    fake = 256

    def rec(m, n, k):
        s = M._Split()
        s.m, s.n, s.k = m, n, k
        s.U = s.S = s.V = fake
        for name, (r, c) in (("Ut_q", (k, m)), ("Vt_q", (k, n)), ("R_q", (m, n))):
            q = getattr(s, name)
            q.fmt, q.rows, q.cols, q.codes, q.scales = 0, r, c, fake, fake
        return s

    x, w = rec(32768, 4096, 96), rec(65536, 4096, 96)
    import ctypes
    assert L.metis_linear_workspace_bytes(ctypes.byref(x), ctypes.byref(w), None) > (64 << 20)
    st = L.spectral_fp4_linear_fwd_noalloc(ctypes.byref(x), ctypes.byref(w), ctypes.c_void_p(fake), 65536, None)
    assert st == 5 and L.metis_status_str(st) == b"METIS_ERR_TOO_LARGE"
