"""The orthogonalisation oracle (fp64 SVD polar factor) against what the
mathematics fixes: a closed form for matrices built from known orthonormal
factors, the defining properties of the polar decomposition, the closed form
of the outer step, and the Newton-Schulz schedule's fixed point.  The pins
are written as checks over an implementation, so that plausible mistakes
planted in copies of the oracle can be shown to fail at least one of them."""
import types

import numpy as np
import pytest

from oracle import polar


def orthonormal(rng, m, r):
    q, _ = np.linalg.qr(rng.standard_normal((m, r)))
    return q


def constructed(rng, m, n, kappa):
    """A = Q1 diag(s) Q2^T with singular values log-spaced in [1/kappa, 1];
    its polar factor is exactly Q1 Q2^T."""
    r = min(m, n)
    q1, q2 = orthonormal(rng, m, r), orthonormal(rng, n, r)
    s = np.logspace(0, -np.log10(kappa), r)
    return (q1 * s) @ q2.T, q1 @ q2.T


# -- checks over an implementation (module-like: polar_factor,
#    outer_orthogonal_step, polar_factor_rows) ---------------------------------

CLOSED_FORM_CASES = [(64, 64, 10), (200, 50, 1e3), (50, 200, 1e3), (300, 300, 1e6), (1, 7, 1),
                     (9, 1, 1)]


def check_closed_form(impl, m, n, kappa):
    rng = np.random.default_rng(m * 1000 + n)
    a, want = constructed(rng, m, n, kappa)
    got = impl.polar_factor(a)
    assert got.shape == want.shape
    assert np.max(np.abs(got - want)) <= 1e-9


def check_defining_properties(impl, m, n):
    """P has orthonormal columns (tall) or rows (wide), and H = P^T A (tall)
    or A P^T (wide) is symmetric positive semi-definite; the factor does not
    change under positive scaling and transposes with A; an orthogonal
    matrix is its own factor."""
    rng = np.random.default_rng(m + 7 * n)
    a = rng.standard_normal((m, n))
    p = impl.polar_factor(a)
    r = min(m, n)
    gram = p.T @ p if m >= n else p @ p.T
    assert np.max(np.abs(gram - np.eye(r))) <= 1e-12
    h = p.T @ a if m >= n else a @ p.T
    assert np.max(np.abs(h - h.T)) <= 1e-12 * np.max(np.abs(h))
    assert np.min(np.linalg.eigvalsh((h + h.T) / 2)) >= -1e-12 * np.max(np.abs(h))
    assert np.max(np.abs(impl.polar_factor(3.7 * a) - p)) <= 1e-12
    assert np.max(np.abs(impl.polar_factor(a.T) - p.T)) <= 1e-12
    q = orthonormal(rng, m, r) if m >= n else orthonormal(rng, n, r).T
    assert np.max(np.abs(impl.polar_factor(q) - q)) <= 1e-12


def check_outer_step_closed_form(impl, m, n):
    """theta - s P(theta - averaged) with theta - averaged = Q1 S Q2^T built
    from known factors is theta - s Q1 Q2^T."""
    rng = np.random.default_rng(5 + m)
    upd, p = constructed(rng, m, n, 30)
    theta = rng.standard_normal((m, n))
    got = impl.outer_orthogonal_step(theta, theta - upd, 0.25)
    assert np.max(np.abs(got - (theta - 0.25 * p))) <= 1e-9


def check_zero_update(impl):
    z = np.zeros((5, 3))
    assert not np.any(impl.polar_factor(z))
    theta = np.arange(15.0).reshape(5, 3)
    assert np.array_equal(impl.outer_orthogonal_step(theta, theta, 0.5), theta)


def check_rows_closed_form(impl, m, n, kappa):
    rng = np.random.default_rng(3 * m + n)
    a, want = constructed(rng, m, n, kappa)
    rows = [0, 7, m // 2, m - 1]
    assert np.max(np.abs(impl.polar_factor_rows(a, rows) - want[rows])) <= 1e-9


def all_checks(impl):
    """Runs every pin on impl; the first failure propagates."""
    for c in CLOSED_FORM_CASES:
        check_closed_form(impl, *c)
    for c in ((120, 40), (40, 120), (77, 77)):
        check_defining_properties(impl, *c)
    for c in ((60, 30), (30, 60), (40, 40)):
        check_outer_step_closed_form(impl, *c)
    check_zero_update(impl)
    for c in ((300, 40, 10), (500, 120, 1e3)):
        check_rows_closed_form(impl, *c)


# -- the oracle against its pins ---------------------------------------------------

@pytest.mark.parametrize("m,n,kappa", CLOSED_FORM_CASES)
def test_closed_form_from_known_factors(m, n, kappa):
    check_closed_form(polar, m, n, kappa)


@pytest.mark.parametrize("m,n", [(120, 40), (40, 120), (77, 77)])
def test_defining_properties(m, n):
    check_defining_properties(polar, m, n)


@pytest.mark.parametrize("m,n", [(60, 30), (30, 60), (40, 40)])
def test_outer_step(m, n):
    check_outer_step_closed_form(polar, m, n)


def test_zero_update_is_a_no_op():
    check_zero_update(polar)


@pytest.mark.parametrize("m,n,kappa", [(300, 40, 10), (500, 120, 1e3)])
def test_rows_from_the_gram_closed_form(m, n, kappa):
    check_rows_closed_form(polar, m, n, kappa)
    with pytest.raises(ValueError):
        polar.polar_factor_rows(np.ones((3, 5)), [0])


def newton_schulz(a, quintic=12, cubic=6):
    """The iteration the GPU runs, written plainly in fp64 (not the GPU code):
    X0 = A/||A||_F; X <- X (a I + b G + c G^2) then X <- X (1.5 I - 0.5 G)."""
    x = a / np.linalg.norm(a)
    tall = a.shape[0] >= a.shape[1]
    for step in range(quintic + cubic):
        g = x.T @ x if tall else x @ x.T
        if step < quintic:
            mm = 3.4445 * np.eye(len(g)) - 4.7750 * g + 2.0315 * g @ g
        else:
            mm = 1.5 * np.eye(len(g)) - 0.5 * g
        x = x @ mm if tall else mm @ x
    return x


@pytest.mark.parametrize("m,n,kappa", [(256, 64, 1e3), (64, 256, 1e3), (128, 128, 1e4)])
def test_iteration_schedule_reaches_the_polar_factor(m, n, kappa):
    """12 quintic + 6 cubic steps reach the SVD polar factor (to 1e-9 in fp64)
    for singular values down to 1/kappa of the largest (s >= 1.4e-7 ||A||_F)."""
    rng = np.random.default_rng(int(kappa) + m)
    a, want = constructed(rng, m, n, kappa)
    assert np.max(np.abs(newton_schulz(a) - want)) <= 1e-9
    assert np.max(np.abs(newton_schulz(a) - polar.polar_factor(a))) <= 1e-9


# -- planted mistakes --------------------------------------------------------------

def _svd(a):
    return np.linalg.svd(np.asarray(a, dtype=np.float64), full_matrices=False)


def _mutant_impl(**over):
    impl = types.SimpleNamespace(polar_factor=polar.polar_factor,
                                 outer_orthogonal_step=polar.outer_orthogonal_step,
                                 polar_factor_rows=polar.polar_factor_rows)
    for k, v in over.items():
        setattr(impl, k, v)
    if "polar_factor" in over and "outer_orthogonal_step" not in over:
        pf = over["polar_factor"]
        impl.outer_orthogonal_step = lambda t, av, s: t - s * pf(t - av)
    return impl


def _pf_transposed_square(a):
    u, _, vt = _svd(a)
    p = u @ vt
    # on square inputs the factors come out in the wrong order: V U^T
    return vt.T @ u.T if a.shape[0] == a.shape[1] else p


def _pf_normalised_update(a):
    a = np.asarray(a, dtype=np.float64)
    n = np.linalg.norm(a)
    return a / n * np.sqrt(min(a.shape)) if n else a


def _pf_singular_vectors_misaligned(a):
    u, _, vt = _svd(a)
    return u[:, ::-1] @ vt


def _pf_negated(a):
    u, _, vt = _svd(a)
    return -(u @ vt)


def _pf_no_zero_case(a):
    u, _, vt = _svd(a)
    return u @ vt


def _pf_full_matrices(a):
    u, _, vt = np.linalg.svd(np.asarray(a, dtype=np.float64), full_matrices=True)
    r = min(a.shape)
    return u[:, :r] @ vt[:r] if a.shape[0] >= a.shape[1] else u @ vt[:r]


def _pf_one_newton_schulz(a):
    a = np.asarray(a, dtype=np.float64)
    return newton_schulz(a, quintic=5, cubic=0) if np.any(a) else np.zeros_like(a)


def _step_sign(t, av, s):
    return t + s * polar.polar_factor(t - av)


def _step_swapped_difference(t, av, s):
    return t - s * polar.polar_factor(av - t)


def _rows_unsquared_root(a, rows):
    a = np.asarray(a, dtype=np.float64)
    lam, v = np.linalg.eigh(a.T @ a)
    return a[np.asarray(rows)] @ ((v / lam) @ v.T)


PLANTED = {
    "factors_in_wrong_order": dict(polar_factor=_pf_transposed_square),
    "normalised_update_not_factor": dict(polar_factor=_pf_normalised_update),
    "singular_vectors_misaligned": dict(polar_factor=_pf_singular_vectors_misaligned),
    "factor_negated": dict(polar_factor=_pf_negated),
    "zero_update_not_zero": dict(polar_factor=_pf_no_zero_case),
    "too_few_newton_schulz_steps": dict(polar_factor=_pf_one_newton_schulz),
    "step_sign_flipped": dict(outer_orthogonal_step=_step_sign),
    "step_difference_swapped": dict(outer_orthogonal_step=_step_swapped_difference),
    "rows_inverse_not_inverse_root": dict(polar_factor_rows=_rows_unsquared_root),
}


def test_correct_full_svd_variant_passes():
    """Control: a different but correct computation (full SVD, truncated)
    passes every check, so the checks do not just pin one code path."""
    impl = _mutant_impl(polar_factor=lambda a: (_pf_full_matrices(a) if np.any(a)
                                                 else np.zeros_like(np.asarray(a, float))))
    all_checks(impl)


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_mistake_is_caught(name):
    impl = _mutant_impl(**PLANTED[name])
    with pytest.raises((AssertionError, ValueError, np.linalg.LinAlgError)):
        all_checks(impl)


def test_unplanted_oracle_passes_all_checks():
    all_checks(polar)
