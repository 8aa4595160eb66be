"""Per-element tolerance of the fp32 polar iteration against the fp64 oracle.

The outer orthogonalisation (DiffuRefill-1B technical report, "What we
measured", "Optimisers") computes a polar factor by an fp32 polynomial
iteration.  Its result cannot match U V^T to a fixed relative error per
element.  An fp32 rounding of the first iterate alone moves the factor by
about u / (sigma_i + sigma_j) in the plane of singular pairs i, j, so the
error scales with the conditioning.  It lands on whole singular directions,
not on single elements, so an element of P near zero has no relative
accuracy at all.  The tolerance here is instead the first-order propagation
of the iteration's rounding errors, element by element.

Model (random rounding: each rounding error is an independent zero-mean
variable; the error of a length-r fp32 dot product grows like sqrt(r) u).
The computed factor is F(A + dA) + dF:

* F(A) = U f(S) V^T with f(s) = phi(s / ||A||_F) is the iteration's exact
  result (oracle.polar.iterated_factor).
* dA is a backward error whose coefficients in A's singular bases,
  E = [U U_perp]^T dA V, are independent with standard deviation
  s_b = C_S u sqrt(r) rms(A).  Its source is the early steps.  There the
  iterate is still as ill-conditioned as A, and each product's rounding acts
  like a perturbation of A itself.
* dF is a forward error of the late, well-conditioned steps: independent per
  element, standard deviation s_f = C_ETA u sqrt(r) rms(P).  These steps no
  longer amplify anything, and their rotation errors are not undone either.

First-order perturbation of a spectral map A -> U f(S) V^T (tall A; wide
matrices are transposed) gives, in the singular bases, for i != j:

    O_ij = sym(E)_ij (f_i - f_j)/(s_i - s_j) + skew(E)_ij (f_i + f_j)/(s_i + s_j)

Also O_ii = f'(s_i) E_ii, and the complement part is
(I - U U^T) dA V diag(f/s) V^T.  sym(E) and skew(E) each have standard
deviation s_b / sqrt(2) off the diagonal.  Element (k, l) of dA's effect
therefore has variance

    s_b^2 [ sum_ij U_ki^2 V_lj^2 w_ij + (1 - |U_k|^2) sum_j V_lj^2 f_j^2 / s_j^2 ]

up to cross terms, with w_ij = ((f_i-f_j)/(s_i-s_j))^2/2 +
((f_i+f_j)/(s_i+s_j))^2/2 and w_ii = f'(s_i)^2.  The cross terms pair
U_ki V_lj with U_kj V_li.  They average to zero over elements, and for each
singular pair they are at most that pair's terms (by 2|xy| <= x^2 + y^2).
So twice the bracket bounds the exact first-order variance.  The tolerance
uses

    var_kl = 2 s_b^2 [ ... ] + s_f^2 + (u P_kl)^2 / 12,

where the last term is the final rounding of P to binary32.  Where the
iteration has converged (f = 1, f' = 0), w_ij is 2 / (s_i + s_j)^2: the
classic sensitivity of the polar factor.

Constants.
* C_S = 2 and C_ETA = 3.  The derivation gives about 0.4 per step from one
  length-r product, with a few steps contributing before the spectrum
  saturates, so about 1 for both.  With these constants the GPU tests'
  largest ratio |error| / std is 4.2, at the 5632 x 2048 and 2048 x 5632
  shapes (every element; limit Z below).  On constructed spectra up to
  kappa 1e4 and the reduced step schedules it stays under 2.  So the
  constants carry a margin of about 2.
* Z = 8.  The error of an element is then within Z standard deviations.
  Under the Gaussian model that fails with probability 1.2e-15 per element,
  below 1e-7 for any matrix here.

`test_oracle_polar.py` pins the first-order formula against a Monte Carlo
of the fp64 oracle under random perturbations.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from oracle import polar as opolar

U32 = 2.0 ** -24
C_S = 2.0
C_ETA = 3.0
Z = 8.0


def iteration_map_derivative(x, quintic: int = 12, cubic: int = 6) -> np.ndarray:
    """d phi / dx by the chain rule through the same steps."""
    x = np.array(x, dtype=np.float64)
    d = np.ones_like(x)
    qa, qb, qc = opolar.QUINTIC
    ca, cb = opolar.CUBIC
    for _ in range(quintic):
        d = d * (qa + 3 * qb * x ** 2 + 5 * qc * x ** 4)
        x = qa * x + qb * x ** 3 + qc * x ** 5
    for _ in range(cubic):
        d = d * (ca + 3 * cb * x ** 2)
        x = ca * x + cb * x ** 3
    return d


def _pair_weights(s, f, fp):
    """w_ij of the module docstring (converged, unconverged and equal
    singular values alike)."""
    ds = s[:, None] - s[None, :]
    close = np.abs(ds) <= 1e-12 * s[0]
    with np.errstate(divide="ignore", invalid="ignore"):
        sym = np.where(close, 0.5 * (fp[:, None] + fp[None, :]),
                       (f[:, None] - f[None, :]) / np.where(close, 1.0, ds))
    skw = (f[:, None] + f[None, :]) / (s[:, None] + s[None, :])
    w = 0.5 * (sym ** 2 + skw ** 2)
    np.fill_diagonal(w, fp ** 2)
    return w


@dataclass
class Expected:
    """The oracle's factors and the per-element standard deviation of the
    fp32 result about iterated (all arrays shaped like the requested rows of
    the matrix)."""
    svd: np.ndarray          # U V^T (the definition)
    iterated: np.ndarray     # U phi(S/||A||_F) V^T (the iteration in exact arithmetic)
    std: np.ndarray          # per-element standard deviation of the fp32 result
    sigma: np.ndarray        # singular values of A, descending

    @property
    def tol(self) -> np.ndarray:
        return Z * self.std


def backward_variance(U, s, V, quintic: int = 12, cubic: int = 6) -> np.ndarray:
    """The bracket of the module docstring per unit s_b^2: the first-order
    variance of each element of U f(S) V^T when A (tall, A = U S V^T with U
    holding the wanted rows) is perturbed by dA with independent
    coefficients of unit variance in its singular bases, cross terms
    dropped."""
    norm_f = float(np.sqrt(np.sum(s ** 2)))
    f = opolar.iteration_map(s / norm_f, quintic, cubic)
    fp = iteration_map_derivative(s / norm_f, quintic, cubic) / norm_f
    var_b = (U ** 2) @ _pair_weights(s, f, fp) @ (V ** 2).T
    rest = np.maximum(0.0, 1.0 - np.sum(U ** 2, axis=1))
    return var_b + np.outer(rest, (V ** 2) @ (f ** 2 / s ** 2))


def _expected_tall(U, s, V, quintic, cubic, m, n):
    """Shared by the full and the sampled-rows forms: U holds the requested
    rows of the left factor."""
    r = s.size
    norm_f = float(np.sqrt(np.sum(s ** 2)))
    f = opolar.iteration_map(s / norm_f, quintic, cubic)
    rms_a = norm_f / np.sqrt(m * n)
    rms_p = np.sqrt(r / (m * n))
    s_b = C_S * U32 * np.sqrt(r) * rms_a
    s_f = C_ETA * U32 * np.sqrt(r) * rms_p
    it = (U * f) @ V.T
    var = (2.0 * s_b ** 2 * backward_variance(U, s, V, quintic, cubic) + s_f ** 2
           + (U32 * it) ** 2 / 12.0)
    return Expected(svd=U @ V.T, iterated=it, std=np.sqrt(var), sigma=s)


def expected(a, quintic: int = 12, cubic: int = 6) -> Expected:
    """Every element of the factor of a (rows x cols), from its fp64 SVD."""
    a = np.asarray(a, dtype=np.float64)
    m, n = a.shape
    wide = m < n
    t = a.T if wide else a
    U, s, vt = np.linalg.svd(t, full_matrices=False)
    e = _expected_tall(U, s, vt.T, quintic, cubic, m, n)
    if wide:
        e = Expected(svd=e.svd.T, iterated=e.iterated.T, std=e.std.T, sigma=e.sigma)
    return e


def expected_rows(a, rows, quintic: int = 12, cubic: int = 6) -> Expected:
    """Selected rows of a tall full-column-rank matrix's factor, through the
    eigendecomposition of A^T A (for matrices too large for a full SVD)."""
    a = np.asarray(a, dtype=np.float64)
    m, n = a.shape
    if m < n:
        raise ValueError("tall matrices only")
    lam, v = np.linalg.eigh(a.T @ a)
    lam, v = lam[::-1], v[:, ::-1]
    if lam[-1] <= 0:
        raise ValueError("rank deficient")
    s = np.sqrt(lam)
    U = (a[np.asarray(rows)] @ v) / s
    return _expected_tall(U, s, v, quintic, cubic, m, n)


def step_tolerance(theta, got_theta, e: Expected, scale: float) -> np.ndarray:
    """Per-element tolerance of theta' = theta - scale * P in binary32 (one
    rounding of scale * P, one of the subtraction) about theta - scale *
    iterated: |scale| times the factor's tolerance plus the two roundings."""
    sp = np.abs(scale) * (np.abs(e.iterated) + e.tol)
    return np.abs(scale) * e.tol + U32 * sp + U32 * (1 + U32) * np.abs(got_theta)


def report(got, e: Expected, what: str) -> float:
    """Largest |got - iterated| / std over the elements; prints the figures
    the parity claim rests on."""
    d = np.abs(got - e.iterated)
    zmax = float(np.max(d / e.std))
    scale = float(np.max(np.abs(e.svd)))
    print(f"{what}: max z = {zmax:.2f} (limit {Z:g}), max|err| = {np.max(d):.3e}"
          f" = {np.max(d) / scale:.2e} of max|P|, vs U V^T {np.max(np.abs(got - e.svd)):.3e}",
          flush=True)
    return zmax
