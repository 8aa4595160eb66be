"""Oracle of outer orthogonalisation.

TEST INFRASTRUCTURE ONLY: never imported by the product library.

The DiffuRefill-1B technical report (section "What we measured",
"Optimisers") replaced the averaged outer update of each weight matrix by its
polar factor.  For A = U S V^T (thin SVD, fp64 here) the polar factor is
U V^T: the orthonormal-columns (or orthonormal-rows) matrix nearest to A,
the factor P of A = P H with H symmetric positive semi-definite.  The SVD is
a library step (numpy.linalg.svd); nothing else is involved.

The report names the factor only.  The library reaches it by a fixed
polynomial iteration on X0 = A / ||A||_F (quintic steps X(aI + bG + cG^2),
then cubic steps X(1.5I - 0.5G), G the Gram matrix of X).  Every step is a
polynomial in A^T A applied to A, so in exact arithmetic the iteration keeps
the singular vectors and maps each singular value s to phi(s / ||A||_F),
where phi is the same steps applied to a scalar.  `iterated_factor` is that
exact result, U phi(S / ||A||_F) V^T: it equals U V^T wherever the
iteration has converged (phi = 1 to fp64 precision for s >= 2e-7 ||A||_F at
12 + 6 steps) and says what the method gives in the directions it has not.
"""
from __future__ import annotations

import numpy as np

# the published quintic coefficients (a, b, c) and the cubic step's (1.5, -0.5)
QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5)


def polar_factor(a: np.ndarray) -> np.ndarray:
    """U V^T of the thin SVD of a (rows x cols), in fp64.  The zero matrix
    has no direction; its factor is taken as zero (the outer step is then a
    no-op)."""
    a = np.asarray(a, dtype=np.float64)
    if not np.any(a):
        return np.zeros_like(a)
    u, _, vt = np.linalg.svd(a, full_matrices=False)
    return u @ vt


def outer_orthogonal_step(theta: np.ndarray, averaged: np.ndarray, scale: float) -> np.ndarray:
    """theta - scale * polar(theta - averaged), in fp64: the outer step whose
    update (the workers' averaged move away from theta) is replaced by its
    polar factor."""
    t = np.asarray(theta, dtype=np.float64)
    return t - float(scale) * polar_factor(t - np.asarray(averaged, dtype=np.float64))


def polar_factor_rows(a: np.ndarray, rows) -> np.ndarray:
    """Selected rows of the polar factor of a full-column-rank tall matrix,
    from the closed form P = A (A^T A)^(-1/2), in fp64: the eigendecomposition
    A^T A = V diag(l) V^T gives (A^T A)^(-1/2) = V diag(l^-1/2) V^T, and row i
    of P is row i of A times that.  For matrices too large for a full SVD."""
    a = np.asarray(a, dtype=np.float64)
    if a.shape[0] < a.shape[1]:
        raise ValueError("tall matrices only (use the transpose)")
    lam, v = np.linalg.eigh(a.T @ a)
    if lam[0] <= 0:
        raise ValueError("rank deficient")
    inv_sqrt = (v / np.sqrt(lam)) @ v.T
    return a[np.asarray(rows)] @ inv_sqrt


def iteration_map(x, quintic: int = 12, cubic: int = 6) -> np.ndarray:
    """phi(x): the iteration's steps applied to a scalar x = s / ||A||_F in
    fp64, first `quintic` steps x <- a x + b x^3 + c x^5, then `cubic` steps
    x <- 1.5 x - 0.5 x^3."""
    x = np.array(x, dtype=np.float64)
    qa, qb, qc = QUINTIC
    ca, cb = CUBIC
    for _ in range(quintic):
        x = qa * x + qb * x ** 3 + qc * x ** 5
    for _ in range(cubic):
        x = ca * x + cb * x ** 3
    return x


def iterated_factor(a: np.ndarray, quintic: int = 12, cubic: int = 6) -> np.ndarray:
    """U phi(S / ||A||_F) V^T in fp64: what the iteration computes in exact
    arithmetic (module docstring).  Zero for the zero matrix."""
    a = np.asarray(a, dtype=np.float64)
    if not np.any(a):
        return np.zeros_like(a)
    u, s, vt = np.linalg.svd(a, full_matrices=False)
    return (u * iteration_map(s / np.linalg.norm(a), quintic, cubic)) @ vt


def iterated_factor_rows(a: np.ndarray, rows, quintic: int = 12, cubic: int = 6) -> np.ndarray:
    """Selected rows of iterated_factor for a full-column-rank tall matrix,
    through the eigendecomposition A^T A = V diag(s^2) V^T: row i is
    A[i] V diag(phi(s / ||A||_F) / s) V^T."""
    a = np.asarray(a, dtype=np.float64)
    if a.shape[0] < a.shape[1]:
        raise ValueError("tall matrices only (use the transpose)")
    lam, v = np.linalg.eigh(a.T @ a)
    if lam[0] <= 0:
        raise ValueError("rank deficient")
    s = np.sqrt(lam)
    f = iteration_map(s / np.linalg.norm(a), quintic, cubic)
    return a[np.asarray(rows)] @ ((v * (f / s)) @ v.T)
