"""The orthogonalisation oracle (fp64 SVD polar factor) against what the
mathematics fixes: a closed form for matrices built from known orthonormal
factors, the defining properties of the polar decomposition, and the
Newton-Schulz schedule's fixed point."""
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


@pytest.mark.parametrize("m,n,kappa", [(64, 64, 10), (200, 50, 1e3), (50, 200, 1e3),
                                       (300, 300, 1e6), (1, 7, 1), (9, 1, 1)])
def test_closed_form_from_known_factors(m, n, kappa):
    rng = np.random.default_rng(m * 1000 + n)
    a, want = constructed(rng, m, n, kappa)
    assert np.max(np.abs(polar.polar_factor(a) - want)) <= 1e-9


@pytest.mark.parametrize("m,n", [(120, 40), (40, 120), (77, 77)])
def test_defining_properties(m, n):
    """P has orthonormal columns (tall) or rows (wide), and H = P^T A (tall)
    or A P^T (wide) is symmetric positive semi-definite; the factor does not
    change under positive scaling and transposes with A; an orthogonal
    matrix is its own factor."""
    rng = np.random.default_rng(m + 7 * n)
    a = rng.standard_normal((m, n))
    p = polar.polar_factor(a)
    r = min(m, n)
    gram = p.T @ p if m >= n else p @ p.T
    assert np.max(np.abs(gram - np.eye(r))) <= 1e-12
    h = p.T @ a if m >= n else a @ p.T
    assert np.max(np.abs(h - h.T)) <= 1e-12 * np.max(np.abs(h))
    assert np.min(np.linalg.eigvalsh((h + h.T) / 2)) >= -1e-12 * np.max(np.abs(h))
    assert np.max(np.abs(polar.polar_factor(3.7 * a) - p)) <= 1e-12
    assert np.max(np.abs(polar.polar_factor(a.T) - p.T)) <= 1e-12
    q = orthonormal(rng, m, r) if m >= n else orthonormal(rng, n, r).T
    assert np.max(np.abs(polar.polar_factor(q) - q)) <= 1e-12


def test_outer_step():
    rng = np.random.default_rng(5)
    theta = rng.standard_normal((60, 30))
    avg = theta - 1e-3 * rng.standard_normal((60, 30))
    got = polar.outer_orthogonal_step(theta, avg, 0.25)
    assert np.allclose(got, theta - 0.25 * polar.polar_factor(theta - avg), atol=0, rtol=0)


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


def test_zero_update_is_a_no_op():
    z = np.zeros((5, 3))
    assert not np.any(polar.polar_factor(z))
    theta = np.arange(15.0).reshape(5, 3)
    assert np.array_equal(polar.outer_orthogonal_step(theta, theta, 0.5), theta)


@pytest.mark.parametrize("m,n,kappa", [(300, 40, 10), (500, 120, 1e3)])
def test_rows_from_the_gram_closed_form(m, n, kappa):
    """The Gram-based rows agree with the known factors Q1 Q2^T."""
    rng = np.random.default_rng(3 * m + n)
    a, want = constructed(rng, m, n, kappa)
    rows = [0, 7, m // 2, m - 1]
    assert np.max(np.abs(polar.polar_factor_rows(a, rows) - want[rows])) <= 1e-9
    with pytest.raises(ValueError):
        polar.polar_factor_rows(a.T, rows[:1])
