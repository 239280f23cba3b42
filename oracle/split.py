"""Randomized spectral split A = U_k diag(S_k) V_k^T + R, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages say (SII post on Metis, §2.4 item 1; "Metis: Training LLMs
with FP4 Quantization", abstract and the method summary of its digest page):
a matrix is split into a dominant part, made of the largest singular values
and their vectors, and a long-tail residual; the parts are quantized
separately. The dominant subspace is found cheaply in a low-dimensional space,
either by a random projection or by sparse random sampling of columns.

The pages give no formulas, so the steps follow the textbook randomized SVD
(Halko, Martinsson & Tropp, "Finding structure with randomness", SIAM Review
2011: Alg. 4.1 range finder without power iterations, Alg. 5.1 direct SVD):

  1. sketch    Y = A Omega (Gaussian Omega, n x l), or Y = A[:, J] (sampled columns)
  2. range     Y = Q R_Y by Householder reflections; keep Q (m x l, orthonormal)
  3. project   B = Q^T A (l x n)
  4. small SVD B = Ub diag(sigma) W^T by one-sided (Hestenes) Jacobi rotations
               (on B, or for wide B on the triangular factor of B^T's QR)
  5. factors   U_k = Q Ub[:, :k], S_k = sigma[:k], V_k = W[:, :k]
  6. signs     each column of U_k is flipped (with the same column of V_k) so
               that its entry of largest magnitude (lowest row on ties) is positive
  7. residual  R = A - U_k diag(S_k) V_k^T, from the unquantized factors

Sketches wider than 128 columns (the 512-column sampling workload) run steps
2 and 4 through LAPACK (numpy.linalg.qr / svd) as library primitives; the
own routines below are pinned against LAPACK, and both routes are pinned to
agree on a 160-column case.

Pins (tests/test_oracle_split.py): Householder Q and R against
numpy.linalg.qr (LAPACK) up to column signs; singular values and subspaces
against numpy.linalg.svd; full rank k = l = min(m, n) gives ||R||/||A|| <= 1e-12;
an exactly rank-8 matrix returns its planted singular values to 1e-10; the
invariants Q^T Q = I, sigma_i(B) <= sigma_i(A), U_k^T R = 0,
||R||^2 = ||A||^2 - sum S_k^2 and the Eckart-Young lower bound on ||R||.
"""
import numpy as np

from .formats import f32, quantize

JACOBI_TOL = 1e-15
JACOBI_MAX_SWEEPS = 60


def householder_qr(Y):
    """Thin QR of a tall matrix by Householder reflections.

    Returns Q (m x l) with orthonormal columns and upper-triangular R (l x l),
    Y = Q R. A column that is already zero below the diagonal gets no
    reflection (its R diagonal is 0 and Q still has orthonormal columns)."""
    A = np.array(Y, dtype=np.float64)
    m, l = A.shape
    if l > m:
        raise ValueError("householder_qr needs rows >= columns")
    reflectors = []
    for j in range(l):
        x = A[j:, j]
        norm_x = np.sqrt(x @ x)
        if norm_x == 0.0:
            reflectors.append(None)
            continue
        # reflect x onto -sign(x0) ||x|| e1 (no cancellation in v0)
        alpha = -norm_x if x[0] >= 0 else norm_x
        v = x.copy()
        v[0] -= alpha
        v /= np.sqrt(v @ v)
        A[j:, j:] -= 2.0 * np.outer(v, v @ A[j:, j:])
        reflectors.append(v)
    # Q = H_0 H_1 ... H_{l-1} applied to the first l columns of the identity,
    # accumulated from the last reflector: before H_j is applied, columns
    # 0..j-1 are still unit vectors with zeros in rows >= j, so H_j only
    # changes the block Q[j:, j:].
    Q = np.zeros((m, l))
    Q[np.arange(l), np.arange(l)] = 1.0
    for j in reversed(range(l)):
        v = reflectors[j]
        if v is None:
            continue
        Q[j:, j:] -= 2.0 * np.outer(v, v @ Q[j:, j:])
    return Q, np.triu(A[:l, :])


def _round_robin_pairs(N, rnd):
    """Pairs of round ``rnd`` of the round-robin (Brent-Luk) ordering of N
    indices (N even): index 0 stays, the others rotate one position per
    round; position i meets position N-1-i. Every pair meets once per sweep."""
    pos = np.arange(N)
    player = np.where(pos == 0, 0, 1 + (pos - 1 + rnd) % (N - 1))
    a, b = player[: N // 2], player[::-1][: N // 2]
    return np.minimum(a, b), np.maximum(a, b)


def jacobi_svd(B, tol=JACOBI_TOL, max_sweeps=JACOBI_MAX_SWEEPS):
    """SVD of a wide matrix B (l x n, l <= n) by one-sided Jacobi rotations.

    The rows of B (the columns of B^T) are rotated in pairs until every pair
    is orthogonal to relative tolerance ``tol``: |g_p . g_q| <= tol ||g_p|| ||g_q||.
    Pairs are visited in the round-robin ordering; the pairs of one round are
    disjoint, so they are rotated together. With G = J^T B after convergence,
    B = J G, the row norms of G are the singular values and the normalized
    rows are the right singular vectors. Returns (Ub, sigma, W) with
    B = Ub diag(sigma) W^T, sigma in descending order, W n x l.
    Rows of zero norm give sigma = 0 and a zero column of W."""
    B = np.asarray(B, dtype=np.float64)
    l, n = B.shape
    N = l + (l % 2)  # an odd count gets one zero row, which never rotates
    G = np.zeros((N, n))
    G[:l] = B
    J = np.eye(N)
    for _ in range(max_sweeps):
        rotated = False
        for rnd in range(N - 1):
            P, Q = _round_robin_pairs(N, rnd)
            gp, gq = G[P], G[Q]
            alpha = np.einsum("ij,ij->i", gp, gp)
            beta = np.einsum("ij,ij->i", gq, gq)
            gamma = np.einsum("ij,ij->i", gp, gq)
            act = (np.abs(gamma) > tol * np.sqrt(alpha * beta)) & (gamma != 0.0)
            if not act.any():
                continue
            rotated = True
            # rotation angle that makes each active pair orthogonal (smaller root)
            zeta = np.where(act, (beta - alpha) / np.where(act, 2.0 * gamma, 1.0), 0.0)
            t = np.where(zeta >= 0, 1.0, -1.0) / (np.abs(zeta) + np.sqrt(1.0 + zeta * zeta))
            c = np.where(act, 1.0 / np.sqrt(1.0 + t * t), 1.0)
            s = np.where(act, c * t, 0.0)
            G[P], G[Q] = c[:, None] * gp - s[:, None] * gq, s[:, None] * gp + c[:, None] * gq
            jp, jq = J[:, P], J[:, Q]
            J[:, P], J[:, Q] = c * jp - s * jq, s * jp + c * jq
        if not rotated:
            break
    G, J = G[:l], J[:l, :l]
    sigma = np.sqrt(np.einsum("ij,ij->i", G, G))
    order = np.argsort(-sigma, kind="stable")
    sigma = sigma[order]
    J = J[:, order]
    G = G[order]
    W = np.zeros((n, l))
    live = sigma > 0
    W[:, live] = (G[live] / sigma[live, None]).T
    return J, sigma, W


LIBRARY_ROUTE_MIN_L = 129  # sketches this wide use LAPACK for the same steps


def range_basis(Y, force=None):
    """Orthonormal basis Q of range(Y) by Householder QR (step 2). Sketches
    wider than 128 columns call LAPACK's Householder QR (numpy.linalg.qr) as
    a library primitive for the same step; ``force`` picks a route."""
    use_lib = Y.shape[1] >= LIBRARY_ROUTE_MIN_L if force is None else force == "library"
    if use_lib:
        Q, _ = np.linalg.qr(np.asarray(Y, dtype=np.float64))
        return Q
    Q, _ = householder_qr(Y)
    return Q


def small_svd(B, force=None):
    """SVD of the projected matrix B (l x n).

    For n up to 4 l, one-sided Jacobi on B itself. For wider B, the rows of B
    are first compressed by a Householder QR of B^T = Qb Rb (the usual QR
    step ahead of an SVD of a very wide matrix, Golub & Van Loan §8.6):
    B = Rb^T Qb^T, so one-sided Jacobi on the l x l matrix Rb^T gives the same
    left singular vectors and values, and W = Qb times its right singular
    vectors. Both routes are exact SVDs; the second only shortens the rows
    that the rotations touch."""
    l, n = B.shape
    use_lib = l >= LIBRARY_ROUTE_MIN_L if force is None else force == "library"
    if use_lib:  # LAPACK SVD as the library primitive for the same step
        Ub, sigma, Wt = np.linalg.svd(np.asarray(B, dtype=np.float64), full_matrices=False)
        return Ub, sigma, Wt.T
    if n <= 4 * l:
        return jacobi_svd(B)
    Qb, Rb = householder_qr(np.asarray(B, dtype=np.float64).T)
    Ub, sigma, Wr = jacobi_svd(Rb.T)
    return Ub, sigma, Qb @ Wr


def sign_convention(U, V):
    """Flip column pairs so that each column of U has its largest-magnitude
    entry (lowest row index on ties) positive."""
    U = np.array(U, dtype=np.float64)
    V = np.array(V, dtype=np.float64)
    for i in range(U.shape[1]):
        j = int(np.argmax(np.abs(U[:, i])))  # first maximum = lowest index
        if U[j, i] < 0:
            U[:, i] = -U[:, i]
            V[:, i] = -V[:, i]
    return U, V


def sketch(A, omega=None, columns=None):
    """Y = A Omega (Gaussian projection) or Y = A[:, J] (sampled columns)."""
    if (omega is None) == (columns is None):
        raise ValueError("give exactly one of omega or columns")
    if omega is not None:
        return np.asarray(A, dtype=np.float64) @ np.asarray(omega, dtype=np.float64)
    J = np.asarray(columns, dtype=np.int64)
    return np.asarray(A, dtype=np.float64)[:, J]


def spectral_split(A, l, k, omega=None, columns=None, q=0):
    """The seven steps of the module docstring. Returns a dict with the
    fp64 factors U (m x k), S (k), V (n x k), the residual R and the
    intermediates Q, B and sigma_B (all l singular values of B).

    q >= 1 adds power (subspace) iterations to step 2, as in Halko,
    Martinsson & Tropp's randomized subspace iteration (their Alg. 4.4):
    with Q = orth(Y), each iteration forms Z = orth(A^T Q) and then
    Y = A Z, Q = orth(Y), re-orthonormalizing after every product so that
    small singular directions are not lost to rounding. The pages fix no q;
    the configurations here all use q = 0 (none)."""
    A = np.asarray(A, dtype=np.float64)
    if not np.all(np.isfinite(A)):
        raise ValueError("split input must be finite")
    m, n = A.shape
    if not (1 <= k <= l <= min(m, n)):
        raise ValueError("need 1 <= k <= l <= min(m, n)")
    if q < 0:
        raise ValueError("q must be >= 0")
    Y = sketch(A, omega, columns)
    if Y.shape != (m, l):
        raise ValueError("sketch width must equal l")
    Q = range_basis(Y)
    for _ in range(q):
        Z = range_basis(A.T @ Q)
        Q = range_basis(A @ Z)
    B = Q.T @ A
    Ub, sigma, W = small_svd(B)
    U = Q @ Ub[:, :k]
    S = sigma[:k].copy()
    V = W[:, :k]
    U, V = sign_convention(U, V)
    R = A - (U * S) @ V.T
    return {"U": U, "S": S, "V": V, "R": R, "Q": Q, "B": B, "sigma_B": sigma}


def mean_split(A):
    """Mean-residual split (Averis, "Averaging-Induced Residual Splitting", as
    retold on the zhu318.com page, its method paragraphs): the mean over all
    rows of A is a vector mu (one value per column); the residual is A minus
    mu broadcast to every row; the mean vector and the residual are quantized
    separately, and the operand is their recombination.

    Written as a rank-1 split record so that it enters the GEMMs like any
    split operand: U = the all-ones column (exact in FP4), S = [1], V = mu,
    R = A - 1 mu^T (from the unquantized mu, as for the spectral split).
    Pins (tests/test_oracle_split.py): mu equals numpy's column mean, the
    residual's column sums vanish, R + 1 mu^T == A."""
    A = np.asarray(A, dtype=np.float64)
    if not np.all(np.isfinite(A)):
        raise ValueError("split input must be finite")
    m, n = A.shape
    if m < 1 or n < 1:
        raise ValueError("empty input")
    mu = A.sum(axis=0) / m
    U = np.ones((m, 1))
    S = np.ones(1)
    V = mu[:, None].copy()
    R = A - U @ V.T
    return {"U": U, "S": S, "V": V, "R": R, "mu": mu}


def quantize_record(fmt, R, U=None, S=None, V=None, orientations=("n", "t")):
    """Quantized split record of one tensor.

    The quantizers act on fp32 tensors: U, V and R are rounded to fp32 first.
    Ut_q: U^T (k x m) blocked along m; Vt_q: V^T (k x n) blocked along n;
    R_q: R (m x n) blocked along n; Rt_q: R^T (n x m) blocked along m.
    S stays fp32 and is not quantized. With U = None the record is an
    unsplit operand (k = 0) whose "residual" is the tensor itself."""
    R32 = f32(R)
    m, n = R32.shape
    rec = {"fmt": fmt, "m": m, "n": n, "k": 0, "S": np.zeros(0),
           "Ut_q": None, "Vt_q": None, "R_q": None, "Rt_q": None}
    if U is not None:
        rec["k"] = U.shape[1]
        rec["S"] = f32(S)
        rec["Ut_q"] = quantize(f32(U).T, fmt)
        rec["Vt_q"] = quantize(f32(V).T, fmt)
    if "n" in orientations:
        rec["R_q"] = quantize(R32, fmt)
    if "t" in orientations:
        rec["Rt_q"] = quantize(R32.T, fmt)
    return rec
