"""Optimizer-side terms of Metis, in fp64 (plain numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Two mechanisms the pages name next to the spectral split (SII open-source-week
post on Metis, §2 "architecture" strategies 2 and 3 and §2.4 items 2 and 3;
the earlier version's abstract on the chatpaper.ai page, items (ii) and (iii)).
The pages give neither formula; the readings below are the plainest ones the
text supports.

Adaptive spectral learning rate (§2.4 item 2): large singular directions
learn strongly by themselves while small ones are neglected, so the gradient
along the mid and low singular directions is rescaled by the inverse of its
normalized singular value, which strengthens those updates without
amplifying noise. Reading: with the split of a gradient G = U diag(S) V^T + R
(S descending, k directions), a reference rank r fixes the level S[r];
direction i keeps its component when S_i >= S[r] and otherwise has it scaled
by gamma_i = min(gamma_max, S[r] / S_i) (its singular value raised to the
reference level, at most gamma_max times); the residual R (the tail beyond
the k resolved directions, where the noise sits) is left as it is:
    G' = G + U diag(S (gamma - 1)) V^T.

Dual-range regularizer (§2.4 item 3): a penalty that both restrains
oversized values and suppresses near-zero ones, compressing the parameter
range (lower variance, smaller quantization error). Reading: a two-sided
hinge on the magnitude of every element w of a parameter tensor,
    loss = lam_hi sum relu(|w| - tau_hi)^2 + lam_lo sum_{w != 0} relu(tau_lo - |w|)^2,
    dloss/dw = 2 lam_hi relu(|w| - tau_hi) sign(w) - 2 lam_lo relu(tau_lo - |w|) sign(w)
(the second term pushes small values away from zero; an exact zero has no
sign and contributes neither loss nor gradient).

Pins (tests/test_oracle_optim.py): gamma = 1 leaves G unchanged; on an
exactly low-rank G the rescaled singular values are S gamma (LAPACK);
gamma is capped and ordered; the regularizer is zero inside the band, even in
w, its gradient odd and equal to a central finite difference of the loss.
"""
import numpy as np


def spectral_lr_gamma(S, r_ref, gamma_max):
    """Per-direction factors gamma_i = min(gamma_max, max(1, S[r_ref] / S_i))
    (1 for S_i = 0, where the component is zero anyway)."""
    S = np.asarray(S, dtype=np.float64)
    k = S.size
    if not (0 <= r_ref < k):
        raise ValueError("reference rank must lie in [0, k)")
    if gamma_max < 1.0:
        raise ValueError("gamma_max must be at least 1")
    ref = S[r_ref]
    g = np.ones(k)
    pos = S > 0
    g[pos] = np.minimum(gamma_max, np.maximum(1.0, ref / S[pos]))
    return g


def spectral_lr_rescale(G, U, S, V, r_ref, gamma_max):
    """G' = G + U diag(S (gamma - 1)) V^T for the split (U, S, V) of G."""
    G = np.asarray(G, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    g = spectral_lr_gamma(S, r_ref, gamma_max)
    return G + (U * (S * (g - 1.0))) @ V.T


def dual_range_loss(W, tau_lo, tau_hi, lam_lo, lam_hi):
    """The two-sided hinge penalty of the module docstring (a float)."""
    a = np.abs(np.asarray(W, dtype=np.float64))
    hi = np.maximum(a - tau_hi, 0.0)
    lo = np.where(a > 0.0, np.maximum(tau_lo - a, 0.0), 0.0)
    return float(lam_hi * np.sum(hi * hi) + lam_lo * np.sum(lo * lo))


def dual_range_grad(W, tau_lo, tau_hi, lam_lo, lam_hi):
    """Its gradient with respect to W (same shape, fp64)."""
    W = np.asarray(W, dtype=np.float64)
    a = np.abs(W)
    s = np.sign(W)
    return 2.0 * lam_hi * np.maximum(a - tau_hi, 0.0) * s - 2.0 * lam_lo * np.maximum(tau_lo - a, 0.0) * s
