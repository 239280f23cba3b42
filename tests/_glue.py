"""Test glue: moves seeded inputs to the GPU and GPU records back into the
oracle's dict layout. Holds no arithmetic of the method."""
import numpy as np
import torch

import fp4_spectral_split_amd as M

FMT_NAME = {M.MXFP4: "mxfp4", M.NVFP4: "nvfp4"}


def device():
    return torch.device("cuda:0")


def to_gpu(t):
    """synth.Tensor -> CUDA tensor of its storage type."""
    if t.dtype == "bf16":
        return torch.from_numpy(t.bits.view(np.int16).copy()).view(torch.bfloat16).to(device())
    return torch.from_numpy(np.ascontiguousarray(t.values)).to(device())


def omega_gpu(t):
    return torch.from_numpy(t.omega.view(np.int16).copy()).view(torch.bfloat16).to(device()).contiguous()


def columns_gpu(t):
    return torch.from_numpy(t.columns.astype(np.int32)).to(device())


def split_gpu(t, orientations=None, fmt=None, q=0):
    A = to_gpu(t)
    o = orientations or t.orientations
    f = fmt or t.fmt
    if t.sketch == "gaussian":
        return M.metis_split(A, t.l, t.k, f, omega=omega_gpu(t), orientations=o, q=q)
    return M.metis_split(A, t.l, t.k, f, columns=columns_gpu(t), orientations=o, q=q)


def fp4_to_dict(q):
    if q is None:
        return None
    B = M.BLOCK[q.fmt]
    return {"fmt": FMT_NAME[q.fmt],
            "codes": q.codes.cpu().numpy().reshape(q.rows, q.cols // 2),
            "scales": q.scales.cpu().numpy().reshape(q.rows, q.cols // B),
            "tensor_scale": float(q.tensor_scale.cpu().item()) if q.tensor_scale is not None else None}


def record_to_dict(rec):
    return {"fmt": FMT_NAME[rec.fmt], "m": rec.m, "n": rec.n, "k": rec.k,
            "S": rec.S.cpu().numpy().astype(np.float64) if rec.k else np.zeros(0),
            "Ut_q": fp4_to_dict(rec.Ut_q) if rec.k else None,
            "Vt_q": fp4_to_dict(rec.Vt_q) if rec.k else None,
            "R_q": fp4_to_dict(rec.R_q), "Rt_q": fp4_to_dict(rec.Rt_q)}


def factors_np(rec):
    return (rec.U.cpu().numpy().astype(np.float64), rec.S.cpu().numpy().astype(np.float64),
            rec.V.cpu().numpy().astype(np.float64))
