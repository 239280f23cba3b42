"""The C-ABI library loads without a GPU, exports every function that
include/*.h declares, and rejects bad arguments on the host before any HIP
call (no compute is launched here)."""
import ctypes
import glob
import os
import re

import pytest

import fp4_spectral_split_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    L = M.load()
    declared = _declared()
    assert {"metis_split", "fp4_block_quant", "spectral_fp4_linear_fwd"} <= declared
    for name in declared:
        assert hasattr(L, name), name
    assert set(M.EXPORTS) == declared


def test_status_strings_and_version():
    L = M.load()
    assert L.metis_status_str(0) == b"METIS_OK"
    assert L.metis_status_str(3) == b"METIS_ERR_WORKSPACE"
    assert L.metis_abi_version() == 2


def _fp4(fmt=0, codes=None, scales=None):
    return M._Fp4(fmt, 0, 0, 0, codes, scales, None)


def test_quant_rejects_bad_arguments_on_host():
    L = M.load()
    out = _fp4()
    # null output
    assert L.fp4_block_quant(ctypes.c_void_p(16), 0, 4, 64, 64, 0, None, None, 0, None) == 1
    # ldx < cols
    assert L.fp4_block_quant(ctypes.c_void_p(16), 0, 4, 64, 32, 0, ctypes.byref(out), None, 0, None) == 1
    # blocked axis not a multiple of 32
    assert L.fp4_block_quant(ctypes.c_void_p(16), 0, 4, 48, 48, 0, ctypes.byref(out), None, 0, None) == 1
    # bad dtype / fmt
    assert L.fp4_block_quant(ctypes.c_void_p(16), 7, 4, 64, 64, 0, ctypes.byref(out), None, 0, None) == 1
    bad = _fp4(fmt=5)
    assert L.fp4_block_quant(ctypes.c_void_p(16), 0, 4, 64, 64, 0, ctypes.byref(bad), None, 0, None) == 1
    # empty input is valid and launches nothing
    assert L.fp4_block_quant(None, 0, 0, 64, 64, 0, ctypes.byref(out), None, 0, None) == 0
    assert out.rows == 0 and out.cols == 64
    # NVFP4 needs its workspace word
    nv = M._Fp4(1, 0, 0, 0, ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256))
    assert L.fp4_block_quant(ctypes.c_void_p(256), 0, 4, 64, 64, 0, ctypes.byref(nv), None, 0, None) == 3
    assert L.fp4_block_quant_workspace_bytes(4, 64, 0) == 0 and L.fp4_block_quant_workspace_bytes(4, 64, 1) > 0


def test_dequant_rejects_bad_arguments_on_host():
    L = M.load()
    q = M._Fp4(0, 0, 4, 48, ctypes.c_void_p(256), ctypes.c_void_p(256), None)
    assert L.fp4_block_dequant(ctypes.byref(q), ctypes.c_void_p(256), 48, None) == 1  # cols % 32
    q = M._Fp4(0, 0, 4, 64, ctypes.c_void_p(256), ctypes.c_void_p(256), None)
    assert L.fp4_block_dequant(ctypes.byref(q), ctypes.c_void_p(256), 32, None) == 1  # ldy < cols
    e = M._Fp4(0, 0, 0, 64, None, None, None)
    assert L.fp4_block_dequant(ctypes.byref(e), None, 64, None) == 0


def _split_rec():
    s = M._Split()
    for name in ("Ut_q", "Vt_q", "R_q", "Rt_q"):
        getattr(s, name).codes = ctypes.c_void_p(256)
        getattr(s, name).scales = ctypes.c_void_p(256)
    s.U = s.S = s.V = ctypes.c_void_p(256)
    return s


def test_split_rejects_bad_arguments_on_host():
    L = M.load()
    s = _split_rec()
    A, om, ws = ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256)
    nbytes = L.metis_split_workspace_bytes(256, 256, 16, 8, 0, 0)
    assert nbytes > 0
    ok = lambda **kw: L.metis_split(kw.get("A", A), kw.get("dt", 1), kw.get("m", 256), kw.get("n", 256),
                                     kw.get("lda", 256), om, kw.get("kind", 0), kw.get("l", 16), kw.get("k", 8),
                                     kw.get("fmt", 0), ctypes.byref(s), None, kw.get("ws", ws),
                                     kw.get("ws_bytes", nbytes), None)
    assert ok(m=250) == 1            # not a multiple of 32
    assert ok(lda=128) == 1          # lda < n
    assert ok(k=17) == 1             # k > l
    assert ok(l=300) == 1            # l > min(m, n)
    assert ok(k=0) == 1
    assert ok(A=None) == 1
    assert ok(A=ctypes.c_void_p(258)) == 1   # misaligned A
    assert ok(ws=None) == 3
    assert ok(ws_bytes=1024) == 3   # far below either dtype's plan
    assert ok(l=544, k=8, m=1024, n=1024, lda=1024) == 2  # sketch wider than this build handles
    assert ok(l=128, k=100, m=512, n=512, lda=512) == 2  # rank above what the GEMMs take
    bad = _split_rec()
    bad.R_q.fmt = 1
    assert L.metis_split(A, 1, 256, 256, 256, om, 0, 16, 8, 0, ctypes.byref(bad), None, ws, nbytes, None) == 1


def test_mean_split_rejects_bad_arguments_on_host():
    L = M.load()
    s = _split_rec()
    A, ws = ctypes.c_void_p(256), ctypes.c_void_p(256)
    nbytes = L.metis_mean_split_workspace_bytes(256, 256, 0)
    assert nbytes > 0
    ok = lambda **kw: L.metis_mean_split(kw.get("A", A), kw.get("dt", 1), kw.get("m", 256), kw.get("n", 256),
                                          kw.get("lda", 256), kw.get("fmt", 0), ctypes.byref(s), kw.get("ws", ws),
                                          kw.get("ws_bytes", nbytes), None)
    assert ok(m=250) == 1            # not a multiple of 32
    assert ok(lda=128) == 1          # lda < n
    assert ok(A=None) == 1
    assert ok(A=ctypes.c_void_p(258)) == 1   # misaligned A
    assert ok(dt=7) == 1
    assert ok(ws=None) == 3
    assert ok(ws_bytes=64) == 3
    bad = _split_rec()
    bad.Vt_q.fmt = 1
    assert L.metis_mean_split(A, 1, 256, 256, 256, 0, ctypes.byref(bad), ws, nbytes, None) == 1


def test_split_power_rejects_bad_arguments_on_host():
    L = M.load()
    s = _split_rec()
    A, om, ws = ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256)
    n1 = L.metis_split_power_workspace_bytes(256, 256, 16, 8, 0, 1, 0)
    n0 = L.metis_split_power_workspace_bytes(256, 256, 16, 8, 0, 0, 0)
    assert n1 > n0 == L.metis_split_workspace_bytes(256, 256, 16, 8, 0, 0)
    assert L.metis_split_power_workspace_bytes(256, 256, 16, 8, 0, -1, 0) == 0
    ok = lambda **kw: L.metis_split_power(A, 1, kw.get("m", 256), kw.get("n", 256), kw.get("m", 256), om, 0,
                                          kw.get("l", 16), 8, kw.get("q", 1), 0, ctypes.byref(s), None, ws,
                                          kw.get("ws_bytes", n1), None)
    assert ok(q=-1) == 1
    assert ok(q=17) == 2                                   # more iterations than this build takes
    assert ok(q=1, l=128, m=1024, n=1024, ws_bytes=1 << 40) == 2  # wide sketches take no iterations
    assert ok(q=1, ws_bytes=n0) == 3                       # the q = 0 workspace is too small


def test_optim_calls_reject_bad_arguments_on_host():
    L = M.load()
    f = ctypes.c_void_p(256)
    # spectral rescale: k out of range, r_ref out of range, gamma_max < 1, k > 96
    assert L.metis_spectral_lr_rescale(f, 8, 8, 8, f, f, f, 0, 0, 2.0, None) == 1
    assert L.metis_spectral_lr_rescale(f, 8, 8, 8, f, f, f, 4, 4, 2.0, None) == 1
    assert L.metis_spectral_lr_rescale(f, 8, 8, 8, f, f, f, 4, 1, 0.5, None) == 1
    assert L.metis_spectral_lr_rescale(f, 8, 8, 8, f, f, f, 97, 1, 2.0, None) == 2
    assert L.metis_spectral_lr_rescale(f, 8, 8, 4, f, f, f, 4, 1, 2.0, None) == 1  # ldg < n
    assert L.metis_spectral_lr_rescale(None, 0, 8, 8, None, None, None, 4, 1, 2.0, None) == 0  # empty
    # dual-range: cols % 8, tau order, negative lambda, missing workspace for the loss
    ws = L.metis_dual_range_workspace_bytes()
    assert ws > 0
    assert L.metis_dual_range_reg(f, 1, 4, 12, 12, 0.1, 1.0, 1.0, 1.0, f, 12, 0, None, None, 0, None) == 1
    assert L.metis_dual_range_reg(f, 1, 4, 16, 16, 1.0, 0.1, 1.0, 1.0, f, 16, 0, None, None, 0, None) == 1
    assert L.metis_dual_range_reg(f, 1, 4, 16, 16, 0.1, 1.0, -1.0, 1.0, f, 16, 0, None, None, 0, None) == 1
    assert L.metis_dual_range_reg(f, 1, 4, 16, 16, 0.1, 1.0, 1.0, 1.0, f, 16, 0, f, None, 0, None) == 3
    assert L.metis_dual_range_reg(f, 7, 4, 16, 16, 0.1, 1.0, 1.0, 1.0, f, 16, 0, None, None, 0, None) == 1

