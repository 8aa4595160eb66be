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


# -- the iteration's exact-arithmetic result (iterated_factor) ---------------------

def spectrum_matrix(rng, m, n, svals):
    r = min(m, n)
    q1, q2 = orthonormal(rng, m, r), orthonormal(rng, n, r)
    return (q1 * np.asarray(svals, dtype=np.float64)) @ q2.T


ITERATED_CASES = [
    # (m, n, smallest s / ||A||_F, quintic, cubic)
    (60, 20, 1e-3, 12, 6), (20, 60, 1e-3, 12, 6), (30, 30, 1e-4, 12, 6),
    (60, 20, 2e-8, 12, 6), (30, 30, 3e-8, 12, 6),     # directions left unconverged
    (40, 16, 1e-2, 1, 0), (16, 40, 1e-2, 3, 2), (25, 25, 1e-3, 12, 0),
]


def check_iterated_matches_newton_schulz(impl, m, n, xmin, q, c):
    """The plain fp64 matrix iteration (newton_schulz above) and U phi(S) V^T
    agree: the polynomial steps keep the singular vectors."""
    rng = np.random.default_rng(m * 13 + n + q)
    r = min(m, n)
    x = np.logspace(0, np.log10(xmin), r)
    s = x * 1.0
    a = spectrum_matrix(rng, m, n, s)
    a = a * (1.0 / np.linalg.norm(a))          # ||A||_F = 1, so s/||A||_F = x (approx.)
    got = impl.iterated_factor(a, q, c)
    want = newton_schulz(a, q, c)
    assert np.max(np.abs(got - want)) <= 1e-7, np.max(np.abs(got - want))
    if xmin >= 2e-7 and q == 12 and c == 6:
        assert np.max(np.abs(got - impl.polar_factor(a))) <= 1e-11


def check_iterated_diagonal(impl):
    """A diagonal matrix: the factor is diag(phi(d / ||d||)), and phi pins the
    first steps by hand: one quintic step of x is a x + b x^3 + c x^5."""
    d = np.array([3.0, 1.0, 0.5, 1e-6, 3e-8])
    a = np.diag(d)
    nrm = np.linalg.norm(d)
    for q, c in ((12, 6), (1, 0), (0, 1), (2, 3)):
        got = impl.iterated_factor(a, q, c)
        want = np.diag(polar.iteration_map(d / nrm, q, c))
        assert np.max(np.abs(got - want)) <= 1e-14
    x = 0.3
    assert abs(float(polar.iteration_map(x, 1, 0)) - (3.4445 * x - 4.7750 * x ** 3
                                                      + 2.0315 * x ** 5)) <= 1e-15
    assert abs(float(polar.iteration_map(x, 0, 1)) - (1.5 * x - 0.5 * x ** 3)) <= 1e-15
    assert abs(float(polar.iteration_map(x, 1, 1))
               - float(polar.iteration_map(polar.iteration_map(x, 1, 0), 0, 1))) <= 1e-15


def check_iterated_rows(impl):
    rng = np.random.default_rng(44)
    a = spectrum_matrix(rng, 300, 40, np.logspace(0, -2, 40))
    rows = [0, 3, 150, 299]
    for q, c in ((12, 6), (2, 1)):
        got = impl.iterated_factor_rows(a, rows, q, c)
        want = impl.iterated_factor(a, q, c)[rows]
        assert np.max(np.abs(got - want)) <= 1e-10


def iterated_checks(impl):
    for case in ITERATED_CASES:
        check_iterated_matches_newton_schulz(impl, *case)
    check_iterated_diagonal(impl)
    check_iterated_rows(impl)


def test_iterated_factor_pins():
    iterated_checks(polar)


def _it_spectral_norm(a, q=12, c=6):
    a = np.asarray(a, dtype=np.float64)
    u, s, vt = np.linalg.svd(a, full_matrices=False)
    return (u * polar.iteration_map(s / s[0], q, c)) @ vt


def _it_steps_swapped(a, q=12, c=6):
    a = np.asarray(a, dtype=np.float64)
    u, s, vt = np.linalg.svd(a, full_matrices=False)
    x = s / np.linalg.norm(a)
    x = polar.iteration_map(polar.iteration_map(x, 0, c), q, 0)
    return (u * x) @ vt


def _it_coefficients_swapped(a, q=12, c=6):
    a = np.asarray(a, dtype=np.float64)
    u, s, vt = np.linalg.svd(a, full_matrices=False)
    x = s / np.linalg.norm(a)
    for _ in range(q):
        x = 3.4445 * x + 2.0315 * x ** 3 - 4.7750 * x ** 5
    x = polar.iteration_map(x, 0, c)
    return (u * x) @ vt


def _it_rows_times_s(a, rows, q=12, c=6):
    a = np.asarray(a, dtype=np.float64)
    lam, v = np.linalg.eigh(a.T @ a)
    s = np.sqrt(lam)
    f = polar.iteration_map(s / np.linalg.norm(a), q, c)
    return a[np.asarray(rows)] @ ((v * (f * s)) @ v.T)


ITERATED_PLANTED = {
    "normalised_by_largest_singular_value": dict(iterated_factor=_it_spectral_norm),
    "cubic_steps_first": dict(iterated_factor=_it_steps_swapped),
    "quintic_coefficients_swapped": dict(iterated_factor=_it_coefficients_swapped),
    "rows_scaled_by_s_not_one_over_s": dict(iterated_factor_rows=_it_rows_times_s),
}


@pytest.mark.parametrize("name", sorted(ITERATED_PLANTED))
def test_iterated_planted_mistake_is_caught(name):
    impl = types.SimpleNamespace(iterated_factor=polar.iterated_factor,
                                 iterated_factor_rows=polar.iterated_factor_rows,
                                 polar_factor=polar.polar_factor)
    for k, v in ITERATED_PLANTED[name].items():
        setattr(impl, k, v)
    with pytest.raises(AssertionError):
        iterated_checks(impl)


# -- the per-element tolerance's first-order formula ------------------------------

def check_variance_formula(var_fn, m, n, q, c, samples=600, seed=0):
    """Monte Carlo of the fp64 oracle: perturb a tall A by eps G (G with
    independent N(0, 1) entries, so its coefficients in A's singular bases are
    independent N(0, 1) too) and collect iterated_factor(A + eps G) -
    iterated_factor(A).  The formula, cross terms dropped, must give the
    total variance over all elements exactly (the cross terms cancel in the
    sum because U and V have orthonormal columns), and bound every element's
    variance within a factor 2 (each pair's cross term is at most its share),
    up to the Monte Carlo's own scatter."""
    from tests import polar_tolerance as pt
    rng = np.random.default_rng(seed + 100 * m + n)
    a = spectrum_matrix(rng, m, n, np.logspace(0, -1.3, min(m, n)))
    u, s, vt = np.linalg.svd(a, full_matrices=False)
    model = var_fn(u, s, vt.T, q, c)
    base = polar.iterated_factor(a, q, c)
    eps = 1e-7
    acc = np.zeros_like(a)
    for _ in range(samples):
        d = polar.iterated_factor(a + eps * rng.standard_normal(a.shape), q, c) - base
        acc += d * d
    emp = acc / samples / eps ** 2
    ratio_total = emp.sum() / model.sum()
    assert abs(ratio_total - 1.0) <= 0.06, ratio_total
    assert np.all(emp <= 2.0 * model * 1.35), float(np.max(emp / model))


VARIANCE_CASES = [(36, 14, 2, 1), (20, 20, 3, 0), (6, 6, 1, 0), (40, 8, 12, 6)]


@pytest.mark.parametrize("m,n,q,c", VARIANCE_CASES)
def test_variance_formula_matches_monte_carlo(m, n, q, c):
    from tests import polar_tolerance as pt
    check_variance_formula(pt.backward_variance, m, n, q, c)


def _var_mutant(drop):
    from tests import polar_tolerance as pt

    def fn(U, s, V, q, c):
        nf = float(np.sqrt(np.sum(s ** 2)))
        f = polar.iteration_map(s / nf, q, c)
        fp = pt.iteration_map_derivative(s / nf, q, c) / nf
        ds = s[:, None] - s[None, :]
        with np.errstate(divide="ignore", invalid="ignore"):
            sym = np.where(ds == 0, fp[:, None], (f[:, None] - f[None, :]) / np.where(ds == 0, 1, ds))
        skw = (f[:, None] + f[None, :]) / (s[:, None] + s[None, :])
        if drop == "skew_over_difference":
            skw = (f[:, None] + f[None, :]) / np.where(ds == 0, 1, np.abs(ds))
        if drop == "symmetric_term":
            sym = 0 * sym
        w = 0.5 * (sym ** 2 + skw ** 2)
        np.fill_diagonal(w, 0 if drop == "diagonal_derivative" else fp ** 2)
        out = (U ** 2) @ w @ (V ** 2).T
        if drop != "complement":
            rest = np.maximum(0.0, 1.0 - np.sum(U ** 2, axis=1))
            out = out + np.outer(rest, (V ** 2) @ (f ** 2 / s ** 2))
        return out
    return fn


@pytest.mark.parametrize("drop", ["complement", "diagonal_derivative", "symmetric_term",
                                  "skew_over_difference"])
def test_variance_formula_planted_mistake_is_caught(drop):
    with pytest.raises(AssertionError):
        for case in VARIANCE_CASES:
            check_variance_formula(_var_mutant(drop), *case, samples=300)
