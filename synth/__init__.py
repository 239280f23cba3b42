"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark. This module holds none of the method's arithmetic: it only
draws random tensors with the shapes and spectra of the workloads below and
rounds them to the storage type (bf16 with round-to-nearest-even, or fp32).

Workloads (layer shapes of the 1.1B model and of LLaMA-3 8B named by the Metis
pages; the training data and trained weights those pages use are replaced by
these synthetic stand-ins):

  cfg 1  tiny forward      W 256x256 fp32 = U diag(100 i^-1.5) V^T, X 128x256 N(0,1),
                           Gaussian Omega 256x16, k = 8, l = 16, MXFP4; X unsplit
  cfg 2  1.1B-class layer  W^T 5632x2048 bf16 (s_i = 50 i^-1.2 + N(0, 0.02^2) noise),
                           X 4096x2048 N(0,1) with 8 outlier channels x20,
                           k = 32, l = 48, MXFP4; X unsplit
  cfg 3  8B attention      W 4096x4096 (s_i = 50/i + noise), X 8192x4096 N(0,1)
                           + 16 planted directions, dY 8192x4096 N(0,1);
                           W and X split k = 64, l = 80; dY unsplit; fwd + dX
  cfg 4  8B FFN up + down  W_up 14336x4096, W_down 4096x14336 (s_i = 50/i + noise),
                           X_up 8192x4096, X_down 8192x14336, dY_up 8192x14336,
                           dY_down 8192x4096 (N(0,1) + 8 planted directions);
                           all six split k = 64, l = 80, MXFP4; six GEMMs
  cfg 5  NVFP4 + sampling  W_down 4096x14336, X 8192x14336 = silu(a) * b,
                           dY 8192x4096; all split by 512 sampled columns, k = 64

Planted directions have singular value 10 (sqrt(rows) + sqrt(cols)), ten times
the edge of the N(0,1) noise bulk. Power-law weights are planted up to rank
min(cols, 512); the omitted terms (s_i < 0.1 for i > 512) sit far below the
noise bulk edge of about 3.7.

Seeds: numpy Generator(PCG64(1000 * cfg + id)), with ids listed in ``_IDS``
and +100 for the down layer of cfg 4/5.
"""
import numpy as np

_IDS = {
    "W.U": 1, "W.V": 2, "W.noise": 3,
    "X": 4, "X.outliers": 5, "dY": 6,
    "omega.W": 7, "omega.X": 8, "omega.dY": 9,
    "X.U": 10, "X.V": 11, "dY.U": 12, "dY.V": 13,
    "cols.W": 14, "cols.X": 15, "cols.dY": 16,
    "X.a": 17, "X.b": 18,
}

POWERLAW_RANK_CAP = 512


def rng(cfg, key, layer_offset=0):
    return np.random.Generator(np.random.PCG64(1000 * cfg + _IDS[key] + layer_offset))


def bf16_bits(x):
    """Round fp32/fp64 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_value(bits):
    """bfloat16 bits -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def orthonormal(gen, rows, cols):
    q, r = np.linalg.qr(gen.standard_normal((rows, cols)))
    return q * np.sign(np.diag(r))


def powerlaw(cfg, rows, cols, s1, alpha, noise, layer_offset=0, rank_cap=POWERLAW_RANK_CAP):
    r = min(rows, cols, rank_cap)
    U = orthonormal(rng(cfg, "W.U", layer_offset), rows, r)
    V = orthonormal(rng(cfg, "W.V", layer_offset), cols, r)
    s = s1 * np.arange(1, r + 1, dtype=np.float64) ** (-alpha)
    A = (U * s) @ V.T
    if noise:
        A += noise * rng(cfg, "W.noise", layer_offset).standard_normal((rows, cols))
    return A


def planted(cfg, key, rows, cols, n_dir, layer_offset=0):
    """N(0,1) noise plus n_dir planted directions of singular value
    10 (sqrt(rows) + sqrt(cols))."""
    A = rng(cfg, key, layer_offset).standard_normal((rows, cols))
    if n_dir:
        sig = 10.0 * (np.sqrt(rows) + np.sqrt(cols))
        U = orthonormal(rng(cfg, key + ".U", layer_offset), rows, n_dir)
        V = orthonormal(rng(cfg, key + ".V", layer_offset), cols, n_dir)
        A += (U * sig) @ V.T
    return A


def gaussian_omega(cfg, key, n, l, layer_offset=0):
    """N(0,1) test matrix rounded to bf16 (n x l), as uint16 bits."""
    return bf16_bits(rng(cfg, key, layer_offset).standard_normal((n, l)))


def sampled_columns(cfg, key, n, l, layer_offset=0):
    """l distinct column ids drawn uniformly without replacement, sorted (int32)."""
    return np.sort(rng(cfg, key, layer_offset).choice(n, size=l, replace=False)).astype(np.int32)


class Tensor:
    """One workload tensor: storage dtype, values and how it is split."""

    def __init__(self, name, values, dtype, k=0, l=0, sketch=None, omega=None, columns=None,
                 orientations=("n",), fmt="mxfp4"):
        self.name = name
        self.dtype = dtype  # "bf16" or "f32"
        if dtype == "bf16":
            self.bits = bf16_bits(values)
            self.values = bf16_value(self.bits)
        else:
            self.bits = None
            self.values = np.ascontiguousarray(values, dtype=np.float32)
        self.k, self.l, self.sketch = k, l, sketch
        self.omega = omega  # uint16 bf16 bits (n x l) or None
        self.columns = columns  # int32 (l,) or None
        self.orientations = tuple(orientations)
        self.fmt = fmt

    @property
    def shape(self):
        return self.values.shape

    def omega_values(self):
        return None if self.omega is None else bf16_value(self.omega)


CONFIG_NAMES = {1: "tiny-256", 2: "1.1B-layer", 3: "8B-attn-proj", 4: "8B-ffn-w4a4g4", 5: "8B-ffn-down-nvfp4-sampled"}

# GEMMs per config: (output name, a tensor, a orientation, b tensor, b orientation)
GEMMS = {
    1: [("Y", "X", "n", "W", "n")],
    2: [("Y", "X", "n", "W", "n")],
    3: [("Y", "X", "n", "W", "n"), ("dX", "dY", "n", "W", "t")],
    4: [("Y_up", "X_up", "n", "W_up", "n"), ("dX_up", "dY_up", "n", "W_up", "t"),
        ("dW_up", "dY_up", "t", "X_up", "t"),
        ("Y_down", "X_down", "n", "W_down", "n"), ("dX_down", "dY_down", "n", "W_down", "t"),
        ("dW_down", "dY_down", "t", "X_down", "t")],
    5: [("Y", "X", "n", "W", "n"), ("dX", "dY", "n", "W", "t"), ("dW", "dY", "t", "X", "t")],
}

TENSOR_NAMES = {
    1: ["W", "X"], 2: ["W", "X"], 3: ["W", "X", "dY"],
    4: ["W_up", "W_down", "X_up", "X_down", "dY_up", "dY_down"], 5: ["W", "X", "dY"],
}


def _orientations(cfg, name):
    need = set()
    for _, a, ao, b, bo in GEMMS[cfg]:
        if a == name:
            need.add(ao)
        if b == name:
            need.add(bo)
    return tuple(o for o in ("n", "t") if o in need)


def make_tensor(cfg, name):
    """Build one named tensor of workload ``cfg`` (1..5)."""
    o = _orientations(cfg, name)
    if cfg == 1:
        if name == "W":
            U = orthonormal(rng(1, "W.U"), 256, 256)
            V = orthonormal(rng(1, "W.V"), 256, 256)
            s = 100.0 * np.arange(1, 257, dtype=np.float64) ** -1.5
            return Tensor("W", (U * s) @ V.T, "f32", k=8, l=16, sketch="gaussian",
                          omega=gaussian_omega(1, "omega.W", 256, 16), orientations=o)
        if name == "X":
            return Tensor("X", rng(1, "X").standard_normal((128, 256)), "f32", orientations=o)
    if cfg == 2:
        if name == "W":  # stored out x in (W^T of a 2048 x 5632 in x out matrix)
            return Tensor("W", powerlaw(2, 5632, 2048, 50.0, 1.2, 0.02), "bf16", k=32, l=48,
                          sketch="gaussian", omega=gaussian_omega(2, "omega.W", 2048, 48), orientations=o)
        if name == "X":
            X = rng(2, "X").standard_normal((4096, 2048))
            cols = rng(2, "X.outliers").choice(2048, size=8, replace=False)
            X[:, cols] *= 20.0
            return Tensor("X", X, "bf16", orientations=o)
    if cfg == 3:
        if name == "W":
            return Tensor("W", powerlaw(3, 4096, 4096, 50.0, 1.0, 0.02), "bf16", k=64, l=80,
                          sketch="gaussian", omega=gaussian_omega(3, "omega.W", 4096, 80), orientations=o)
        if name == "X":
            return Tensor("X", planted(3, "X", 8192, 4096, 16), "bf16", k=64, l=80, sketch="gaussian",
                          omega=gaussian_omega(3, "omega.X", 4096, 80), orientations=o)
        if name == "dY":
            return Tensor("dY", rng(3, "dY").standard_normal((8192, 4096)), "bf16", orientations=o)
    if cfg == 4:
        shapes = {"W_up": (14336, 4096), "W_down": (4096, 14336), "X_up": (8192, 4096),
                  "X_down": (8192, 14336), "dY_up": (8192, 14336), "dY_down": (8192, 4096)}
        if name not in shapes:
            raise KeyError(name)
        rows, cols = shapes[name]
        off = 100 if name.endswith("_down") else 0
        base = name.split("_")[0]
        if base == "W":
            vals = powerlaw(4, rows, cols, 50.0, 1.0, 0.02, off)
        else:
            vals = planted(4, base, rows, cols, 8, off)
        return Tensor(name, vals, "bf16", k=64, l=80, sketch="gaussian",
                      omega=gaussian_omega(4, "omega." + base, cols, 80, off), orientations=o)
    if cfg == 5:
        if name == "W":
            vals = powerlaw(4, 4096, 14336, 50.0, 1.0, 0.02, 100)
        elif name == "X":
            a = rng(5, "X.a").standard_normal((8192, 14336))
            b = rng(5, "X.b").standard_normal((8192, 14336))
            vals = a / (1.0 + np.exp(-a)) * b
        elif name == "dY":
            vals = planted(4, "dY", 8192, 4096, 8, 100)
        else:
            raise KeyError(name)
        cols = vals.shape[1]
        return Tensor(name, vals, "bf16", k=64, l=512, sketch="columns",
                      columns=sampled_columns(5, "cols." + name, cols, 512), orientations=o, fmt="nvfp4")
    raise KeyError((cfg, name))


def small_case(seed, rows, cols, dtype="bf16", kind="powerlaw", k=8, l=16, n_dir=4,
               orientations=("n", "t"), fmt="mxfp4", sketch="gaussian"):
    """Reduced-size stand-in with the same structure (for fast parity tests)."""
    g = np.random.Generator(np.random.PCG64(seed))
    if kind == "powerlaw":
        r = min(rows, cols, 64)
        U = orthonormal(g, rows, r)
        V = orthonormal(g, cols, r)
        vals = (U * (50.0 * np.arange(1, r + 1) ** -1.0)) @ V.T + 0.02 * g.standard_normal((rows, cols))
    elif kind == "planted":
        vals = g.standard_normal((rows, cols))
        sig = 10.0 * (np.sqrt(rows) + np.sqrt(cols))
        vals += (orthonormal(g, rows, n_dir) * sig) @ orthonormal(g, cols, n_dir).T
    elif kind == "normal":
        vals = g.standard_normal((rows, cols))
    elif kind == "zero":
        vals = np.zeros((rows, cols))
    else:
        raise ValueError(kind)
    omega = columns = None
    if k:
        if sketch == "gaussian":
            omega = bf16_bits(g.standard_normal((cols, l)))
        else:
            columns = np.sort(g.choice(cols, size=l, replace=False)).astype(np.int32)
    return Tensor("T", vals, dtype, k=k, l=l if k else 0, sketch=sketch if k else None,
                  omega=omega, columns=columns, orientations=orientations, fmt=fmt)
