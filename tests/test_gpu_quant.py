"""GPU parity of fp4_block_quant / fp4_block_dequant against the oracle:
codes, scales and tensor scales bit-exact on identical fp32 inputs."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from tests import _glue as G

pytestmark = pytest.mark.gpu

import fp4_spectral_split_amd as M


def _inputs(seed, rows, cols, kind):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((rows, cols))
    if kind == "wide":
        x *= np.exp(4.0 * g.standard_normal((rows, cols)))
    elif kind == "special":
        x[:, :32] = 0.0                       # all-zero blocks
        x[0, 1] = -0.0
        x[1, 32:64] = 2.0 ** -140             # subnormal fp32 block
        x[2, 64:96] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4)  # exact ties at scale 1
        x[3, 96:128] = 1e30 * g.standard_normal(32)
    return x


def _check_fp4(q, want, fmt):
    got = G.fp4_to_dict(q)
    assert np.array_equal(got["codes"], want["codes"]), "codes differ"
    assert np.array_equal(got["scales"], want["scales"]), "scales differ"
    if fmt == "nvfp4":
        assert np.float32(got["tensor_scale"]) == np.float32(want["tensor_scale"])


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("shape,kind", [((96, 160), "normal"), ((224, 384), "wide"), ((160, 256), "special"),
                                        ((1056, 4128), "normal")])
def test_quant_bit_exact(fmt, dtype, transpose, shape, kind):
    rows, cols = shape
    x = _inputs(rows * 7 + cols + len(kind), rows, cols, kind)
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        xv = synth.bf16_value(bits).astype(np.float64)
        xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        xv = x.astype(np.float32).astype(np.float64)
        xt = torch.from_numpy(xv.astype(np.float32)).cuda()
    print("case", fmt, dtype, transpose, shape, kind, flush=True)
    q = M.fp4_block_quant(xt, fmt, transpose=transpose)
    src = xv.T if transpose else xv
    want = F.quantize(src, fmt)
    _check_fp4(q, want, fmt)
    y = M.fp4_block_dequant(q).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, F.dequantize(want))


def test_quant_strided_input_and_empty():
    x = torch.randn(64, 96, device="cuda")
    sub = x[:, :64]  # leading dimension 96
    q = M.fp4_block_quant(sub, "mxfp4")
    want = F.quantize(sub.cpu().double().numpy(), "mxfp4")
    _check_fp4(q, want, "mxfp4")
    e = M.fp4_block_quant(torch.empty(0, 64, device="cuda"), "mxfp4")
    assert e.rows == 0 and e.cols == 64


def test_quant_full_size_activation():
    """cfg 4 X_up (8192 x 4096 bf16) in both orientations, on 64 sampled rows."""
    t = synth.make_tensor(4, "X_up")
    xt = G.to_gpu(t)
    xv = t.values.astype(np.float64)
    rows = np.random.Generator(np.random.PCG64(1)).choice(8192, 64, replace=False)
    q = G.fp4_to_dict(M.fp4_block_quant(xt, "mxfp4"))
    want = F.quantize(xv[rows], "mxfp4")
    assert np.array_equal(q["codes"][rows], want["codes"]) and np.array_equal(q["scales"][rows], want["scales"])
    cols = np.random.Generator(np.random.PCG64(2)).choice(4096, 64, replace=False)
    qt = G.fp4_to_dict(M.fp4_block_quant(xt, "mxfp4", transpose=True))
    want = F.quantize(xv.T[cols], "mxfp4")
    assert np.array_equal(qt["codes"][cols], want["codes"]) and np.array_equal(qt["scales"][cols], want["scales"])
