"""W4A4G4 linear layer on quantized split operands, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages ("Metis: Training LLMs with FP4 Quantization", abstract) train with
FP4 weights, activations and gradients: the three GEMMs of a linear layer,
Y = X W^T, dX = dY W and dW = dY^T X, take FP4 operands. They do not spell out
how a split operand enters a GEMM; the plain reading is that the operand is
the sum of its dequantized parts:

  normal orientation (contraction along the columns n):
      A_hat   = R_hat + U_hat diag(S) V_hat^T                       (m x n)
  transposed orientation (contraction along the rows m):
      A_hat^T = Rt_hat + V_hat diag(S) U_hat^T                      (n x m)

where R_hat, Rt_hat, U_hat, V_hat are dequantized from the record's FP4 codes.
The residual is quantized separately per orientation (blocks run along the
contraction axis), so Rt_hat is not the transpose of R_hat.

Route 1 (the definition): form both operands in fp64 and multiply.
Route 2 (a second, independent route used as a pin): the four-term expansion
  C = Ra Rb^T + Ra Fb Sb Gb^T + Ga Sa Fa^T Rb^T + Ga Sa (Fa^T Fb) Sb Gb^T
with G the factor along the output axis and F the factor along the
contraction axis. Pins (tests/test_oracle_linear.py): the two routes agree
to 1e-12; k = 0 is a plain dequantized GEMM; an identity X returns W_hat.
"""
import numpy as np

from .formats import dequantize


def factors(rec):
    """Dequantized (U_hat m x k, S, V_hat n x k) of a split record."""
    if rec["k"] == 0:
        return None, None, None
    U = dequantize(rec["Ut_q"]).T
    V = dequantize(rec["Vt_q"]).T
    return U, np.asarray(rec["S"], dtype=np.float64), V


def residual(rec, orientation):
    key = "R_q" if orientation == "n" else "Rt_q"
    if rec[key] is None:
        raise ValueError("record has no %s orientation" % orientation)
    return dequantize(rec[key])


def operand(rec, orientation, rows=None):
    """Dequantized GEMM operand, rows along the output axis, columns along the
    contraction axis. ``rows`` optionally selects output rows."""
    Rh = residual(rec, orientation)
    if rows is not None:
        Rh = Rh[rows]
    if rec["k"] == 0:
        return Rh
    U, S, V = factors(rec)
    G, F = (U, V) if orientation == "n" else (V, U)
    if rows is not None:
        G = G[rows]
    return Rh + (G * S) @ F.T


def gemm_nt(a, a_orient, b, b_orient, rows=None):
    """C = A_hat B_hat^T in fp64 (route 1). ``rows`` samples rows of C."""
    return operand(a, a_orient, rows) @ operand(b, b_orient).T


def gemm_nt_expanded(a, a_orient, b, b_orient):
    """The same product by the four-term expansion (route 2)."""
    Ra = residual(a, a_orient)
    Rb = residual(b, b_orient)
    C = Ra @ Rb.T
    Ga = Fa = Gb = Fb = None
    if a["k"]:
        U, Sa, V = factors(a)
        Ga, Fa = (U, V) if a_orient == "n" else (V, U)
    if b["k"]:
        U, Sb, V = factors(b)
        Gb, Fb = (U, V) if b_orient == "n" else (V, U)
    if b["k"]:
        C = C + ((Ra @ Fb) * Sb) @ Gb.T
    if a["k"]:
        C = C + (Ga * Sa) @ (Rb @ Fa).T
    if a["k"] and b["k"]:
        C = C + (Ga * Sa) @ ((Fa.T @ Fb) * Sb) @ Gb.T
    return C


def linear_fwd(X, W, rows=None):
    """Y = X_hat W_hat^T: both operands contract along the input features."""
    return gemm_nt(X, "n", W, "n", rows)


def linear_bwd_dx(dY, W, rows=None):
    """dX = dY_hat W_hat: contraction along the output features (W transposed)."""
    return gemm_nt(dY, "n", W, "t", rows)


def linear_bwd_dw(dY, X, rows=None):
    """dW = dY_hat^T X_hat: contraction along the tokens (both transposed)."""
    return gemm_nt(dY, "t", X, "t", rows)
