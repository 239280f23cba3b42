"""Python binding of libmetis_fp4 (the spectral-domain FP4 linear layer for
MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmetis_fp4.so``. PyTorch supplies device memory and streams.
There is no fallback: if the library is missing or a call fails, an
exception is raised.

Calls (same names as the C ABI in include/metis_fp4.h):
  fp4_block_quant(x, fmt, transpose)          -> Fp4Tensor
  fp4_block_dequant(q)                         -> fp32 tensor
  metis_split(A, l, k, fmt, omega=, columns=)  -> SplitRecord
  spectral_fp4_linear_fwd(X, W)                -> Y = X W^T
  spectral_fp4_linear_fwd_noalloc(X, W, out)   -> the same, static scratch
  spectral_fp4_linear_bwd(dY, X, W)            -> (dX = dY W, dW = dY^T X)
  metis_spectral_lr_rescale(G, rec, r, gmax)   -> G rescaled in place
  metis_dual_range_reg(W, ...)                 -> (loss, grad)
"""
import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmetis_fp4.so")

MXFP4, NVFP4 = 0, 1
F32, BF16 = 0, 1
OMEGA_GAUSSIAN, OMEGA_COLUMNS = 0, 1
_FMT = {"mxfp4": MXFP4, "nvfp4": NVFP4, MXFP4: MXFP4, NVFP4: NVFP4}
_FMT_NAME = {MXFP4: "mxfp4", NVFP4: "nvfp4"}
BLOCK = {MXFP4: 32, NVFP4: 16}


class MetisError(RuntimeError):
    pass


class _Fp4(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("reserved", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class _Split(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("U", ctypes.c_void_p), ("S", ctypes.c_void_p), ("V", ctypes.c_void_p),
                ("Ut_q", _Fp4), ("Vt_q", _Fp4), ("R_q", _Fp4), ("Rt_q", _Fp4)]


_lib = None


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MetisError("libmetis_fp4.so not built: run fp4_spectral_split_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.metis_status_str.restype = ctypes.c_char_p
    L.metis_status_str.argtypes = [i32]
    L.metis_abi_version.restype = i32
    L.fp4_block_quant_workspace_bytes.restype = sz
    L.fp4_block_quant_workspace_bytes.argtypes = [i64, i64, i32]
    L.fp4_block_quant.restype = i32
    L.fp4_block_quant.argtypes = [vp, i32, i64, i64, i64, i32, ctypes.POINTER(_Fp4), vp, sz, vp]
    L.fp4_block_dequant.restype = i32
    L.fp4_block_dequant.argtypes = [ctypes.POINTER(_Fp4), vp, i64, vp]
    L.metis_split_workspace_bytes.restype = sz
    L.metis_split_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
    L.metis_split.restype = i32
    L.metis_split.argtypes = [vp, i32, i64, i64, i64, vp, i32, i32, i32, i32, ctypes.POINTER(_Split), vp, vp, sz, vp]
    L.metis_split_power_workspace_bytes.restype = sz
    L.metis_split_power_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32, i32]
    L.metis_split_power.restype = i32
    L.metis_split_power.argtypes = [vp, i32, i64, i64, i64, vp, i32, i32, i32, i32, i32, ctypes.POINTER(_Split), vp,
                                    vp, sz, vp]
    L.metis_mean_split_workspace_bytes.restype = sz
    L.metis_mean_split_workspace_bytes.argtypes = [i64, i64, i32]
    L.metis_mean_split.restype = i32
    L.metis_mean_split.argtypes = [vp, i32, i64, i64, i64, i32, ctypes.POINTER(_Split), vp, sz, vp]
    L.metis_linear_workspace_bytes.restype = sz
    L.metis_linear_workspace_bytes.argtypes = [ctypes.POINTER(_Split)] * 3
    L.spectral_fp4_linear_fwd.restype = i32
    L.spectral_fp4_linear_fwd.argtypes = [ctypes.POINTER(_Split), ctypes.POINTER(_Split), vp, i64, vp, sz, vp]
    L.spectral_fp4_linear_fwd_noalloc.restype = i32
    L.spectral_fp4_linear_fwd_noalloc.argtypes = [ctypes.POINTER(_Split), ctypes.POINTER(_Split), vp, i64, vp]
    L.spectral_fp4_linear_bwd.restype = i32
    L.spectral_fp4_linear_bwd.argtypes = [ctypes.POINTER(_Split)] * 3 + [vp, i64, vp, i64, vp, sz, vp]
    L.metis_spectral_lr_rescale.restype = i32
    L.metis_spectral_lr_rescale.argtypes = [vp, i64, i64, i64, vp, vp, vp, i32, i32, ctypes.c_float, vp]
    L.metis_dual_range_workspace_bytes.restype = sz
    L.metis_dual_range_workspace_bytes.argtypes = []
    L.metis_dual_range_reg.restype = i32
    L.metis_dual_range_reg.argtypes = [vp, i32, i64, i64, i64, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_float, vp, i64, i32, vp, vp, sz, vp]
    sp = ctypes.POINTER(_Split)
    L.metis_gemm_nt_workspace_bytes.restype = sz
    L.metis_gemm_nt_workspace_bytes.argtypes = [sp, i32, sp, i32]
    L.metis_gemm_nt_prepare.restype = i32
    L.metis_gemm_nt_prepare.argtypes = [sp, i32, sp, i32, vp, sz, vp]
    L.metis_gemm_nt_main.restype = i32
    L.metis_gemm_nt_main.argtypes = [sp, i32, sp, i32, vp, i64, vp, sz, vp]
    _lib = L
    return L


EXPORTS = ["metis_status_str", "metis_abi_version", "fp4_block_quant_workspace_bytes", "fp4_block_quant",
           "fp4_block_dequant", "metis_split_workspace_bytes", "metis_split", "metis_split_power_workspace_bytes",
           "metis_split_power", "metis_mean_split_workspace_bytes",
           "metis_mean_split", "metis_linear_workspace_bytes",
           "spectral_fp4_linear_fwd", "spectral_fp4_linear_fwd_noalloc", "spectral_fp4_linear_bwd", "metis_gemm_nt_workspace_bytes",
           "metis_gemm_nt_prepare", "metis_gemm_nt_main", "metis_spectral_lr_rescale",
           "metis_dual_range_workspace_bytes", "metis_dual_range_reg"]


def _check(status):
    if status != 0:
        raise MetisError(load().metis_status_str(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise MetisError("dense inputs must be float32 or bfloat16")


_ws_cache = {}


def workspace(nbytes, device):
    """A cached uint8 device buffer of at least nbytes (per device and stream)."""
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


@dataclass
class Fp4Tensor:
    """rows x cols FP4 matrix, blocks along cols (see metis_fp4_t)."""
    fmt: int
    rows: int
    cols: int
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: Optional[torch.Tensor] = None

    @staticmethod
    def empty(fmt, rows, cols, device):
        fmt = _FMT[fmt]
        B = BLOCK[fmt]
        return Fp4Tensor(fmt, rows, cols,
                         torch.empty(rows * cols // 2, dtype=torch.uint8, device=device),
                         torch.empty(rows * (cols // B), dtype=torch.uint8, device=device),
                         torch.empty(1, dtype=torch.float32, device=device) if fmt == NVFP4 else None)

    def c(self):
        return _Fp4(self.fmt, 0, self.rows, self.cols, _ptr(self.codes), _ptr(self.scales), _ptr(self.tensor_scale))

    @property
    def fmt_name(self):
        return _FMT_NAME[self.fmt]


def _none_fp4():
    return _Fp4(0, 0, 0, 0, None, None, None)


def fp4_block_quant(x, fmt="mxfp4", transpose=False, out=None):
    """Quantize a 2-D fp32/bf16 CUDA tensor (blocks along its last axis, or
    along its first axis with transpose=True, giving x^T)."""
    L = load()
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1
    fmt = _FMT[fmt]
    rows, cols = x.shape
    if out is None:
        out = Fp4Tensor.empty(fmt, cols if transpose else rows, rows if transpose else cols, x.device)
    c = out.c()
    nws = L.fp4_block_quant_workspace_bytes(rows, cols, fmt)
    ws = workspace(nws, x.device) if nws else None
    _check(L.fp4_block_quant(_ptr(x), _dtype_code(x), rows, cols, x.stride(0), int(transpose), ctypes.byref(c),
                             _ptr(ws), nws, _stream(x.device)))
    out.rows, out.cols = c.rows, c.cols
    return out


def fp4_block_dequant(q, out=None):
    L = load()
    if out is None:
        out = torch.empty(q.rows, q.cols, dtype=torch.float32, device=q.codes.device)
    c = q.c()
    _check(L.fp4_block_dequant(ctypes.byref(c), _ptr(out), out.stride(0), _stream(out.device)))
    return out


@dataclass
class SplitRecord:
    """Quantized split of an m x n tensor (see metis_split_t)."""
    m: int
    n: int
    k: int
    fmt: int
    U: Optional[torch.Tensor] = None
    S: Optional[torch.Tensor] = None
    V: Optional[torch.Tensor] = None
    Ut_q: Optional[Fp4Tensor] = None
    Vt_q: Optional[Fp4Tensor] = None
    R_q: Optional[Fp4Tensor] = None
    Rt_q: Optional[Fp4Tensor] = None
    info: Optional[torch.Tensor] = None
    keep: list = field(default_factory=list)

    def c(self):
        s = _Split()
        s.m, s.n, s.k = self.m, self.n, self.k
        s.U, s.S, s.V = _ptr(self.U), _ptr(self.S), _ptr(self.V)
        s.Ut_q = self.Ut_q.c() if self.Ut_q is not None else _none_fp4()
        s.Vt_q = self.Vt_q.c() if self.Vt_q is not None else _none_fp4()
        s.R_q = self.R_q.c() if self.R_q is not None else _none_fp4()
        s.Rt_q = self.Rt_q.c() if self.Rt_q is not None else _none_fp4()
        for name in ("Ut_q", "Vt_q", "R_q", "Rt_q"):
            getattr(s, name).fmt = self.fmt
        return s


def empty_split(m, n, k, fmt, orientations, device):
    fmt = _FMT[fmt]
    rec = SplitRecord(m, n, k, fmt)
    if k:
        rec.U = torch.empty(m, k, dtype=torch.float32, device=device)
        rec.S = torch.empty(k, dtype=torch.float32, device=device)
        rec.V = torch.empty(n, k, dtype=torch.float32, device=device)
        rec.Ut_q = Fp4Tensor.empty(fmt, k, m, device)
        rec.Vt_q = Fp4Tensor.empty(fmt, k, n, device)
    if "n" in orientations:
        rec.R_q = Fp4Tensor.empty(fmt, m, n, device)
    if "t" in orientations:
        rec.Rt_q = Fp4Tensor.empty(fmt, n, m, device)
    rec.info = torch.zeros(1, dtype=torch.int32, device=device)
    return rec


def metis_split(A, l, k, fmt="mxfp4", omega=None, columns=None, orientations=("n", "t"), out=None, q=0):
    """Split a 2-D fp32/bf16 CUDA tensor A (m x n) into U diag(S) V^T + R and
    quantize the parts. omega: n x l bf16 tensor (Gaussian sketch) or
    columns: int32 tensor of l column ids (sampling sketch); q: power
    iterations after the sketch (metis_split_power)."""
    L = load()
    assert A.dim() == 2 and A.is_cuda and A.stride(1) == 1
    m, n = A.shape
    fmt = _FMT[fmt]
    if (omega is None) == (columns is None):
        raise MetisError("give exactly one of omega or columns")
    if omega is not None:
        assert omega.dtype == torch.bfloat16 and omega.is_contiguous() and tuple(omega.shape) == (n, l)
        kind, om = OMEGA_GAUSSIAN, omega
    else:
        assert columns.dtype == torch.int32 and columns.is_contiguous() and columns.numel() == l
        kind, om = OMEGA_COLUMNS, columns
    rec = out if out is not None else empty_split(m, n, k, fmt, orientations, A.device)
    c = rec.c()
    if q == 0:
        nws = L.metis_split_workspace_bytes(m, n, l, k, kind, fmt)
        ws = workspace(nws, A.device)
        _check(L.metis_split(_ptr(A), _dtype_code(A), m, n, A.stride(0), _ptr(om), kind, l, k, fmt,
                             ctypes.byref(c), _ptr(rec.info), _ptr(ws), nws, _stream(A.device)))
    else:
        nws = L.metis_split_power_workspace_bytes(m, n, l, k, kind, q, fmt)
        ws = workspace(nws, A.device)
        _check(L.metis_split_power(_ptr(A), _dtype_code(A), m, n, A.stride(0), _ptr(om), kind, l, k, q, fmt,
                                   ctypes.byref(c), _ptr(rec.info), _ptr(ws), nws, _stream(A.device)))
    return rec


def metis_mean_split(A, fmt="mxfp4", orientations=("n", "t"), out=None):
    """Mean-residual split of a 2-D fp32/bf16 CUDA tensor A (m x n): the
    column mean mu and A - mu, quantized separately, as a rank-1 record
    (U = 1, S = 1, V = mu) that the GEMMs take like any split operand."""
    L = load()
    assert A.dim() == 2 and A.is_cuda and A.stride(1) == 1
    m, n = A.shape
    fmt = _FMT[fmt]
    rec = out if out is not None else empty_split(m, n, 1, fmt, orientations, A.device)
    c = rec.c()
    nws = L.metis_mean_split_workspace_bytes(m, n, fmt)
    ws = workspace(nws, A.device)
    _check(L.metis_mean_split(_ptr(A), _dtype_code(A), m, n, A.stride(0), fmt, ctypes.byref(c), _ptr(ws), nws,
                              _stream(A.device)))
    return rec


def plain_operand(x, fmt="mxfp4", orientations=("n",)):
    """An unsplit (k = 0) operand: the tensor quantized in each orientation."""
    m, n = x.shape
    rec = SplitRecord(m, n, 0, _FMT[fmt])
    if "n" in orientations:
        rec.R_q = fp4_block_quant(x, fmt, transpose=False)
    if "t" in orientations:
        rec.Rt_q = fp4_block_quant(x, fmt, transpose=True)
    return rec


def _linear_ws(X, W, dY, device):
    L = load()
    cx, cw = X.c(), W.c()
    cd = dY.c() if dY is not None else None
    n = L.metis_linear_workspace_bytes(ctypes.byref(cx), ctypes.byref(cw), ctypes.byref(cd) if cd else None)
    return workspace(n, device), n


def spectral_fp4_linear_fwd(X, W, out=None):
    """Y = X_hat W_hat^T (M x N, fp32)."""
    L = load()
    dev = (X.R_q or X.Rt_q).codes.device
    if out is None:
        out = torch.empty(X.m, W.m, dtype=torch.float32, device=dev)
    ws, n = _linear_ws(X, W, None, dev)
    cx, cw = X.c(), W.c()
    _check(L.spectral_fp4_linear_fwd(ctypes.byref(cx), ctypes.byref(cw), _ptr(out), out.stride(0), _ptr(ws), n,
                                     _stream(dev)))
    return out


def spectral_fp4_linear_fwd_noalloc(X, W, out):
    """Y = X_hat W_hat^T into the caller's fp32 tensor out (M x N), with the
    workspace taken from the library's static per-GPU scratch: the C call
    allocates nothing (the binding allocates nothing either). Calls that
    overlap on one GPU race on that scratch."""
    L = load()
    assert out.dtype == torch.float32 and out.is_cuda and out.stride(1) == 1
    cx, cw = X.c(), W.c()
    _check(L.spectral_fp4_linear_fwd_noalloc(ctypes.byref(cx), ctypes.byref(cw), _ptr(out), out.stride(0),
                                             _stream(out.device)))
    return out


def spectral_fp4_linear_bwd(dY, X, W, need_dx=True, need_dw=True, dx=None, dw=None):
    """dX = dY_hat W_hat (M x K) and dW = dY_hat^T X_hat (N x K), fp32."""
    L = load()
    dev = (dY.R_q or dY.Rt_q).codes.device
    if need_dx and dx is None:
        dx = torch.empty(X.m, X.n, dtype=torch.float32, device=dev)
    if need_dw and dw is None:
        dw = torch.empty(W.m, W.n, dtype=torch.float32, device=dev)
    ws, n = _linear_ws(X, W, dY, dev)
    cd, cx, cw = dY.c(), X.c(), W.c()
    _check(L.spectral_fp4_linear_bwd(ctypes.byref(cd), ctypes.byref(cx), ctypes.byref(cw),
                                     _ptr(dx) if need_dx else None, dx.stride(0) if need_dx else 0,
                                     _ptr(dw) if need_dw else None, dw.stride(0) if need_dw else 0,
                                     _ptr(ws), n, _stream(dev)))
    return dx, dw


def _dev(rec):
    q = rec.R_q if rec.R_q is not None else rec.Rt_q
    return q.codes.device


class GemmNT:
    """One GEMM C = A_hat B_hat^T split into prepare (skinny FP4 products and
    correction panels) and main (FP4 GEMM + correction), sharing a workspace
    owned by this object. trans_a / trans_b pick the orientation of each
    operand (False: R_q, contraction over n; True: Rt_q, over m)."""

    def __init__(self, a, trans_a, b, trans_b):
        L = load()
        self.a, self.b = a, b
        self.ta, self.tb = int(bool(trans_a)), int(bool(trans_b))
        self.ca, self.cb = a.c(), b.c()
        self.rows = a.n if trans_a else a.m
        self.cols = b.n if trans_b else b.m
        dev = _dev(a)
        self.nbytes = L.metis_gemm_nt_workspace_bytes(ctypes.byref(self.ca), self.ta, ctypes.byref(self.cb), self.tb)
        self.ws = torch.empty(max(self.nbytes, 256), dtype=torch.uint8, device=dev)

    def prepare(self):
        _check(load().metis_gemm_nt_prepare(ctypes.byref(self.ca), self.ta, ctypes.byref(self.cb), self.tb,
                                            _ptr(self.ws), self.nbytes, _stream(self.ws.device)))

    def main(self, out):
        assert out.shape[0] >= self.rows and out.stride(1) == 1
        _check(load().metis_gemm_nt_main(ctypes.byref(self.ca), self.ta, ctypes.byref(self.cb), self.tb, _ptr(out),
                                         out.stride(0), _ptr(self.ws), self.nbytes, _stream(out.device)))
        return out

    def __call__(self, out=None):
        if out is None:
            out = torch.empty(self.rows, self.cols, dtype=torch.float32, device=self.ws.device)
        self.prepare()
        return self.main(out)


def metis_spectral_lr_rescale(G, rec, r_ref, gamma_max):
    """Adaptive spectral learning rate: G (fp32, m x n) rescaled in place along
    the split rec of G (its fp32 U, S, V): G += U diag(S (gamma - 1)) V^T."""
    L = load()
    assert G.dtype == torch.float32 and G.is_cuda and G.stride(1) == 1 and rec.k > 0
    m, n = G.shape
    _check(L.metis_spectral_lr_rescale(_ptr(G), m, n, G.stride(0), _ptr(rec.U), _ptr(rec.S), _ptr(rec.V), rec.k,
                                       int(r_ref), float(gamma_max), _stream(G.device)))
    return G


def metis_dual_range_reg(W, tau_lo, tau_hi, lam_lo, lam_hi, grad=None, accumulate=False, want_grad=True):
    """Dual-range regularizer of a 2-D fp32/bf16 CUDA tensor W: returns
    (loss as a 1-element fp64 tensor, grad as fp32 or None). With grad given
    and accumulate=True the gradient is added to it."""
    L = load()
    assert W.dim() == 2 and W.is_cuda and W.stride(1) == 1
    rows, cols = W.shape
    if want_grad and grad is None:
        grad = torch.empty(rows, cols, dtype=torch.float32, device=W.device)
        accumulate = False
    loss = torch.empty(1, dtype=torch.float64, device=W.device)
    nws = L.metis_dual_range_workspace_bytes()
    ws = workspace(nws, W.device)
    _check(L.metis_dual_range_reg(_ptr(W), _dtype_code(W), rows, cols, W.stride(0), float(tau_lo), float(tau_hi),
                                  float(lam_lo), float(lam_hi), _ptr(grad) if want_grad else None,
                                  grad.stride(0) if want_grad else 0, int(bool(accumulate)), _ptr(loss), _ptr(ws), nws,
                                  _stream(W.device)))
    return loss, grad
