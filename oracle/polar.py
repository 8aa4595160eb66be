"""Oracle of outer orthogonalisation.

TEST INFRASTRUCTURE ONLY: never imported by the product library.

The DiffuRefill-1B technical report (section "What we measured",
"Optimisers") replaced the averaged outer update of each weight matrix by its
polar factor.  For A = U S V^T (thin SVD, fp64 here) the polar factor is
U V^T: the orthonormal-columns (or orthonormal-rows) matrix nearest to A,
the factor P of A = P H with H symmetric positive semi-definite.  The SVD is
a library step (numpy.linalg.svd); nothing else is involved.
"""
from __future__ import annotations

import numpy as np


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
