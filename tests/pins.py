"""Checks that pin the CPU oracle to mathematics, not to itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with:
* exact rational arithmetic (fractions.Fraction) on inputs where every binary32
  operation of the merge is exact or has a known correctly rounded result;
* closed forms of the EMA and of the outer Nesterov recursion;
* library routines in fp64 (numpy.mean, numpy.average with weights, torch's
  bfloat16 widening) within error bounds derived from the operation count;
* invariants the pages imply (identity on identical checkpoints, momentum 0
  and learning rate 1 reducing to the token-weighted mean);
* hand-derived binary32 examples in which the arrival order changes the sum.

The same pins are run against deliberately broken builds of the oracle
(tests/test_oracle_mutants.py) to show that each plausible mistake fails one.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

U = 2.0 ** -24          # unit roundoff of binary32
F32_BETA = float(np.float32(0.9))
F32_OMEGA = float(np.float32(1.0) - np.float32(0.9))


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def f32_rne(x: Fraction) -> np.float32:
    """Nearest binary32 to the rational x, ties to even (exact, no double
    rounding: the three binary32 neighbours of a first guess are compared)."""
    guess = np.float32(float(x))
    cands = [np.nextafter(guess, np.float32(-np.inf)), guess,
             np.nextafter(guess, np.float32(np.inf))]
    best = None
    for c in cands:
        err = abs(Fraction(float(c)) - x)
        key = (err, int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


def assert_bits_equal(got, want, what: str):
    g, w = bits(got), bits(want)
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, (f"{what}: {bad.size} elements differ; first at {bad[0]}: "
                           f"got {np.asarray(got).flat[bad[0]]!r} want {np.asarray(want).flat[bad[0]]!r}")


def dyadic(rng, n: int, frac_bits: int = 16, mag: int = 2) -> np.ndarray:
    """Random multiples of 2^-frac_bits in (-mag, mag): exact in binary32 and
    with room for exact sums of a few of them."""
    lim = mag << frac_bits
    ints = rng.integers(-lim + 1, lim, size=n)
    return (ints.astype(np.float64) * 2.0 ** -frac_bits).astype(np.float32)


def workload_like(rng, n: int, workers: int):
    """Global ~ 0.02 * N(0,1) and workers = global + 1e-3 * N(0,1), in fp32."""
    theta = (0.02 * rng.standard_normal(n)).astype(np.float32)
    cks = [(theta.astype(np.float64) + 1e-3 * rng.standard_normal(n)).astype(np.float32)
           for _ in range(workers)]
    return theta, cks


# ---------------------------------------------------------------------------
# plain replacement averaging
# ---------------------------------------------------------------------------

def pin_mean_exact_rational(orc):
    """Mean of N dyadic checkpoints: the fp32 running sum is exact here, so
    the result must be the correctly rounded rational mean for every N
    (division exact for N = 1, 2, 4, 8; correctly rounded for the others)."""
    rng = np.random.default_rng(101)
    n = 1024
    for N in range(1, 9):
        cks = [dyadic(rng, n) for _ in range(N)]
        got = orc.mean_round(cks)
        want = np.array([f32_rne(sum(Fraction(float(c[j])) for c in cks) / N) for j in range(n)],
                        dtype=np.float32)
        assert_bits_equal(got, want, f"exact rational mean, N={N}")


def pin_mean_division_correctly_rounded(orc):
    """A single arrival of S folded then divided by N=1 is S; the division of
    a known sum by N must be the correctly rounded quotient, which a
    reciprocal-multiply or a wrong divisor misses on some inputs."""
    rng = np.random.default_rng(102)
    n = 4096
    s = dyadic(rng, n, frac_bits=20, mag=4)
    for N in (3, 5, 6, 7):
        acc = s.copy()
        out = np.empty_like(acc)
        orc.finalize_mean(out, acc, N)
        want = np.array([f32_rne(Fraction(float(s[j])) / N) for j in range(n)], dtype=np.float32)
        assert_bits_equal(out, want, f"S/N correctly rounded, N={N}")


def pin_mean_arrival_order(orc):
    """Hand-derived binary32 example in which the fold order decides the sum.

    a = 1, b = c = 2^-24.  In order (a, b, c): 1 + 2^-24 is a tie between 1
    and 1 + 2^-23 and rounds to the even significand, 1; adding c again gives
    1.  In order (b, c, a): 2^-24 + 2^-24 = 2^-23 exactly, and 1 + 2^-23 is
    representable.  An fp64 accumulator would give 1 + 2^-23 both ways.  The
    means are then the correctly rounded 1/3 and (1 + 2^-23)/3."""
    a = np.array([1.0], dtype=np.float32)
    b = np.array([2.0 ** -24], dtype=np.float32)
    c = np.array([2.0 ** -24], dtype=np.float32)
    g1 = orc.mean_round([a, b, c])
    g2 = orc.mean_round([b, c, a])
    assert_bits_equal(g1, [f32_rne(Fraction(1, 3))], "order (a,b,c)")
    assert_bits_equal(g2, [f32_rne((1 + Fraction(1, 2 ** 23)) / 3)], "order (b,c,a)")
    assert bits(g1)[0] != bits(g2)[0]


def pin_mean_fp64_bound(orc):
    """Against numpy's fp64 mean on workload-like data: a sequential binary32
    sum of N terms followed by one division is within (N+1) u max_i |c_i|."""
    rng = np.random.default_rng(103)
    n = 1 << 16
    for N in (1, 2, 3, 5, 8):
        _, cks = workload_like(rng, n, N)
        got = orc.mean_round(cks).astype(np.float64)
        stack = np.stack([c.astype(np.float64) for c in cks])
        ref = np.mean(stack, axis=0)
        bound = (N + 1) * U * np.max(np.abs(stack), axis=0)
        err = np.abs(got - ref)
        assert np.all(err <= bound), f"N={N}: max err/bound {np.max(err / bound)}"


def pin_mean_identical(orc):
    """The mean of N copies of one checkpoint is that checkpoint: exactly for
    N = 1, 2, 4 (every sum is exact or rounds back), within N u |c| else."""
    rng = np.random.default_rng(104)
    c = (0.02 * rng.standard_normal(1 << 16)).astype(np.float32)
    for N in range(1, 9):
        g = orc.mean_round([c] * N)
        if N in (1, 2, 4):
            assert_bits_equal(g, c, f"identical mean N={N}")
        else:
            err = np.abs(g.astype(np.float64) - c.astype(np.float64))
            assert np.all(err <= N * U * np.abs(c.astype(np.float64))), f"N={N}"


def pin_first_fold_is_copy(orc):
    """The first arrival of a round is copied into the sum (whatever the
    buffer held before, NaN included), and a lone -0.0 stays -0.0 (a sum
    started from +0 would turn it into +0)."""
    c = np.array([-0.0, 1.5, -2.25, 3e-41], dtype=np.float32)
    acc = np.full(4, np.nan, dtype=np.float32)
    orc.fold_mean(acc, c, first=True)
    assert_bits_equal(acc, c, "first fold copies")
    g = orc.mean_round([c])
    assert_bits_equal(g, c, "mean of one checkpoint")
    acc = np.full(4, np.nan, dtype=np.float32)
    orc.fold_delta(acc, np.zeros(4, np.float32), c, 1, first=True)
    assert_bits_equal(acc, -c, "first delta fold copies")


def pin_bf16_widening(orc):
    """bf16 checkpoints are widened exactly: compare every one of the 65,536
    bit patterns with torch's bfloat16 -> float32 conversion."""
    import torch
    pat = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    acc = np.empty(pat.size, dtype=np.float32)
    orc.fold_mean(acc, pat, first=True)
    ref = torch.from_numpy(pat.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert_bits_equal(acc, ref, "bf16 widening")
    # and a bf16 arrival folds like its widened fp32 value
    rng = np.random.default_rng(105)
    a = dyadic(rng, 512, frac_bits=6)
    bf = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    g_bf = orc.mean_round([bf, bf, bf, bf])
    widened = torch.from_numpy(bf.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert_bits_equal(g_bf, widened, "bf16 mean of identical")


def pin_denormals_kept(orc):
    """Subnormal inputs are neither flushed nor lost: exact dyadic subnormal
    sums and power-of-two divisions stay exact."""
    t = 2.0 ** -140
    a = np.array([t, 3 * t, -5 * t, 2.0 ** -149], dtype=np.float32)
    b = np.array([t, t, 7 * t, 2.0 ** -149], dtype=np.float32)
    g = orc.mean_round([a, b])
    want = [f32_rne((Fraction(float(x)) + Fraction(float(y))) / 2) for x, y in zip(a, b)]
    assert_bits_equal(g, want, "subnormal mean")
    assert bits(g)[0] != 0


def pin_nan_inf_propagate(orc):
    """IEEE propagation: a NaN in any arrival gives NaN at that element, and
    +inf and -inf arriving at one element give NaN; other elements finite."""
    a = np.array([1.0, np.nan, np.inf, 2.0], dtype=np.float32)
    b = np.array([1.0, 2.0, -np.inf, 2.0], dtype=np.float32)
    g = orc.mean_round([a, b])
    assert g[0] == 1.0 and np.isnan(g[1]) and np.isnan(g[2]) and g[3] == 2.0
    theta = np.array([0.5, 0.5, 0.5, 0.5], dtype=np.float32)
    m = np.zeros(4, np.float32)
    orc.nesterov_fragment_round(theta, m, [a, b], [3, 5], 0.7, 0.9)
    assert np.isfinite(theta[0]) and np.isnan(theta[1]) and np.isnan(theta[2])
    assert np.isnan(m[1]) and np.isfinite(m[3])


def pin_finalize_in_place(orc):
    """Dividing in place (output is the sum buffer) gives the same bits as
    dividing into a separate buffer."""
    rng = np.random.default_rng(106)
    _, cks = workload_like(rng, 4099, 3)
    acc = np.empty(4099, np.float32)
    for k, c in enumerate(cks):
        orc.fold_mean(acc, c, first=(k == 0))
    out = np.empty_like(acc)
    orc.finalize_mean(out, acc, 3)
    orc.finalize_mean(acc, acc, 3)
    assert_bits_equal(acc, out, "in-place finalize")


# ---------------------------------------------------------------------------
# EMA of globals
# ---------------------------------------------------------------------------

def _ema_closed(e0, gs, beta: Fraction, omega: Fraction):
    """e_k = beta^k e0 + omega * sum_j beta^(k-j) g_j, exactly."""
    k = len(gs)
    out = []
    for j in range(e0.size):
        v = beta ** k * Fraction(float(e0[j]))
        for i, g in enumerate(gs, start=1):
            v += omega * beta ** (k - i) * Fraction(float(g[j]))
        out.append(v)
    return out


def pin_ema_closed_form_exact(orc):
    """beta = 3/4 on dyadic globals (1 - beta = 1/4 is exact too, and beta
    differs from 1 - beta so swapped weights show): every EMA step is exact,
    so after k rounds the EMA equals its geometric-sum closed form exactly;
    both the stand-alone EMA and the EMA fused into the mean's close are
    checked."""
    rng = np.random.default_rng(107)
    n, k = 256, 6
    e0 = dyadic(rng, n, frac_bits=8)
    gs = [dyadic(rng, n, frac_bits=8) for _ in range(k)]
    want = [f32_rne(v) for v in _ema_closed(e0, gs, Fraction(3, 4), Fraction(1, 4))]
    e = e0.copy()
    for g in gs:
        orc.ema_update(e, g, 0.75)
    assert_bits_equal(e, want, "EMA closed form (stand-alone)")
    e = e0.copy()
    for g in gs:
        out = np.empty_like(g)
        orc.finalize_mean(out, g.copy(), 1, e, 0.75)      # global = g / 1 = g
        assert_bits_equal(out, g, "g/1")
    assert_bits_equal(e, want, "EMA closed form (fused with mean)")


def pin_ema_closed_form_bound(orc):
    """beta = fp32(0.9) over 50 rounds of workload-like globals: the binary32
    iterate stays within 24 u max|g| of the exact closed form (each step adds
    at most 2 u max|g| of rounding, damped by beta afterwards).  Checked for
    the stand-alone EMA, the EMA fused into the mean's close and the EMA
    fused into the outer Nesterov step (momentum 0, lr 1, one participant
    pushing g: the new global is g up to the delta's rounding)."""
    rng = np.random.default_rng(108)
    n, k = 512, 50
    e0 = (0.02 * rng.standard_normal(n)).astype(np.float32)
    gs = [(0.02 * rng.standard_normal(n)).astype(np.float32) for _ in range(k)]
    beta = Fraction(F32_BETA)
    omega = Fraction(F32_OMEGA)
    assert beta + omega == 1
    exact = np.array([float(v) for v in _ema_closed(e0, gs, beta, omega)])
    M = max(np.max(np.abs(e0)), max(np.max(np.abs(g)) for g in gs))
    e = e0.copy()
    for g in gs:
        orc.ema_update(e, g, 0.9)
    err = np.abs(e.astype(np.float64) - exact)
    assert np.all(err <= 24 * U * M), f"stand-alone: max err {err.max()} vs {24 * U * M}"
    e = e0.copy()
    for g in gs:
        orc.finalize_mean(np.empty_like(g), g.copy(), 1, e, 0.9)
    err = np.abs(e.astype(np.float64) - exact)
    assert np.all(err <= 24 * U * M), f"fused mean: max err {err.max()} vs {24 * U * M}"
    e = e0.copy()
    theta = e0.copy()
    for g in gs:
        orc.nesterov_fragment_round(theta, np.zeros_like(theta), [g.copy()], [1], 1.0, 0.0, e, 0.9)
    err = np.abs(e.astype(np.float64) - exact)
    assert np.all(err <= 40 * U * M), f"fused nesterov: max err {err.max()} vs {40 * U * M}"


# ---------------------------------------------------------------------------
# token-weighted delta merge + outer Nesterov
# ---------------------------------------------------------------------------

def pin_nesterov_identical_snapshots(orc):
    """All participants pushed the global unchanged: the deltas are 0, so with
    zero momentum the global is bit-for-bit unchanged and the momentum stays
    0; the EMA still takes its step towards the (unchanged) global."""
    rng = np.random.default_rng(109)
    theta = (0.02 * rng.standard_normal(3001)).astype(np.float32)
    theta0 = theta.copy()
    m = np.zeros_like(theta)
    e = dyadic(rng, 3001)
    e0 = e.copy()
    orc.nesterov_fragment_round(theta, m, [theta0.copy()] * 3, [250_000, 210_000, 266_000],
                                0.7, 0.9, e, 0.9)
    assert_bits_equal(theta, theta0, "theta unchanged")
    assert_bits_equal(m, np.zeros_like(m), "momentum zero")
    want = (np.float32(0.9) * e0 + np.float32(F32_OMEGA) * theta0).astype(np.float32)
    assert_bits_equal(e, want, "EMA step")


def pin_nesterov_reduces_to_weighted_mean_exact(orc):
    """Momentum 0 and learning rate 1 make the outer step plain parameter
    averaging (GradientMail post, second follow-up run): the new global is
    sum_i t_i c_i / sum_i t_i.  Dyadic values and tokens summing to a power
    of two keep every operation exact, so the match is bit-for-bit."""
    rng = np.random.default_rng(110)
    n = 1024
    tokens = [1, 3, 2, 2]
    theta = dyadic(rng, n, frac_bits=12)
    cks = [dyadic(rng, n, frac_bits=12) for _ in tokens]
    th = theta.copy()
    m = dyadic(rng, n, frac_bits=12)      # any momentum: mu = 0 ignores it
    orc.nesterov_fragment_round(th, m, cks, tokens, 1.0, 0.0)
    W = sum(tokens)
    want = [f32_rne(sum(t * Fraction(float(c[j])) for t, c in zip(tokens, cks)) / W)
            for j in range(n)]
    assert_bits_equal(th, want, "weighted mean (exact)")
    dbar = [f32_rne(sum(t * (Fraction(float(theta[j])) - Fraction(float(c[j])))
                        for t, c in zip(tokens, cks)) / W) for j in range(n)]
    assert_bits_equal(m, dbar, "momentum = mean delta when mu = 0")


def pin_nesterov_reduces_to_weighted_mean_bound(orc):
    """Same reduction on workload-like data with token counts in
    [200k, 270k], against numpy.average(weights=tokens) in fp64.  Bound:
    (k + 3) u (sum_i t_i |theta - c_i| / W + |theta'|) for k participants."""
    rng = np.random.default_rng(111)
    n = 1 << 15
    for k in (1, 3, 4, 5):
        theta, cks = workload_like(rng, n, k)
        tokens = [int(t) for t in rng.integers(200_000, 270_001, size=k)]
        th = theta.copy()
        m = np.zeros_like(theta)
        orc.nesterov_fragment_round(th, m, cks, tokens, 1.0, 0.0)
        stack = np.stack([c.astype(np.float64) for c in cks])
        ref = np.average(stack, axis=0, weights=np.array(tokens, dtype=np.float64))
        W = float(sum(tokens))
        spread = np.sum(np.array(tokens, dtype=np.float64)[:, None]
                        * np.abs(theta.astype(np.float64)[None, :] - stack), axis=0) / W
        bound = (k + 3) * U * (spread + np.abs(ref))
        err = np.abs(th.astype(np.float64) - ref)
        assert np.all(err <= bound), f"k={k}: max err/bound {np.max(err / bound)}"


def pin_nesterov_equal_tokens_is_plain_mean(orc):
    """With equal token counts the token-weighted mean is the plain mean
    (numpy.mean in fp64), within the same bound."""
    rng = np.random.default_rng(112)
    theta, cks = workload_like(rng, 1 << 14, 4)
    th = theta.copy()
    orc.nesterov_fragment_round(th, np.zeros_like(th), cks, [131072] * 4, 1.0, 0.0)
    ref = np.mean(np.stack([c.astype(np.float64) for c in cks]), axis=0)
    spread = np.mean(np.abs(theta.astype(np.float64) - np.stack(cks).astype(np.float64)), axis=0)
    assert np.all(np.abs(th - ref) <= 7 * U * (spread + np.abs(ref)))


def _nesterov_closed(theta0: Fraction, d: Fraction, K: int, lr: Fraction, mu: Fraction):
    """Constant outer gradient d from zero momentum:
       m_K     = d (1 - mu^K) / (1 - mu)
       theta_K = theta0 - lr d [K + mu/(1-mu) (K - mu (1 - mu^K)/(1 - mu))]"""
    mK = d * (1 - mu ** K) / (1 - mu)
    s = K + mu / (1 - mu) * (K - mu * (1 - mu ** K) / (1 - mu))
    return theta0 - lr * d * s, mK


def pin_nesterov_closed_form_exact(orc):
    """Every round's participants push theta - d (a constant outer gradient
    d).  With mu = 1/2, lr = 1/2 and dyadic values every binary32 operation
    is exact, so after K rounds theta and m equal the closed form exactly."""
    rng = np.random.default_rng(113)
    n, K = 257, 6
    theta = dyadic(rng, n, frac_bits=10)
    d = dyadic(rng, n, frac_bits=4, mag=1)
    theta0 = theta.copy()
    m = np.zeros_like(theta)
    for r in range(K):
        cks = [(theta - d).astype(np.float32) for _ in range(3)]
        orc.nesterov_fragment_round(theta, m, cks, [4, 8, 4], 0.5, 0.5)
    for j in range(n):
        th, mk = _nesterov_closed(Fraction(float(theta0[j])), Fraction(float(d[j])), K,
                                  Fraction(1, 2), Fraction(1, 2))
        assert Fraction(float(theta[j])) == th, (j, float(theta[j]), float(th))
        assert Fraction(float(m[j])) == mk, (j, float(m[j]), float(mk))


def pin_nesterov_closed_form_bound(orc):
    """Same constant-gradient test at lr = fp32(0.7), mu = fp32(0.9) over 8
    rounds, against the closed form in exact arithmetic.  Error budget per
    round: forming the pushed snapshot theta - d rounds by u |theta - d|, and
    an error in the mean delta reaches theta with weight at most
    lr (1 + mu) / (1 - mu) < 14; the step itself adds a few u of |lr u_k|.
    Over K rounds: |theta_K - closed| <= 20 K u (max|theta| + |d| / (1 - mu)),
    |m_K - closed| <= 20 u (max|theta| + |d|) / (1 - mu)."""
    rng = np.random.default_rng(114)
    n, K = 512, 8
    theta = (0.02 * rng.standard_normal(n)).astype(np.float32)
    d = (1e-3 * rng.standard_normal(n)).astype(np.float32)
    theta0 = theta.copy()
    m = np.zeros_like(theta)
    tmax = np.abs(theta0).astype(np.float64)
    for r in range(K):
        cks = [(theta - d).astype(np.float32) for _ in range(5)]
        orc.nesterov_fragment_round(theta, m, cks, [1 << 20] * 5, 0.7, 0.9)
        tmax = np.maximum(tmax, np.abs(theta))
    lr, mu = Fraction(float(np.float32(0.7))), Fraction(float(np.float32(0.9)))
    for j in range(n):
        th, mk = _nesterov_closed(Fraction(float(theta0[j])), Fraction(float(d[j])), K, lr, mu)
        ad = abs(float(d[j]))
        assert abs(float(theta[j]) - float(th)) <= 20 * K * U * (tmax[j] + ad / 0.1), j
        assert abs(float(m[j]) - float(mk)) <= 20 * U * (tmax[j] + ad) / 0.1, j


def pin_nesterov_first_steps(orc):
    """The first rounds of the constant-gradient test at lr 0.7, mu 0.9 and
    d = 1 give theta_K - theta_0 = -1.33, -3.227, -5.6343 (the closed form;
    checked to 1e-6 relative with theta0 = 0 and exact-ish binary32 data)."""
    theta = np.zeros(1, np.float32)
    m = np.zeros(1, np.float32)
    got = []
    for r in range(3):
        orc.nesterov_fragment_round(theta, m, [(theta - 1).astype(np.float32)], [1], 0.7, 0.9)
        got.append(float(theta[0]))
    for g, w in zip(got, [-1.33, -3.227, -5.6343]):
        assert abs(g - w) <= 1e-6 * abs(w), (got)


def pin_token_weights_rounded_once(orc):
    """Token counts above 2^24 are rounded to binary32 once (nearest-even);
    the total is summed exactly as an integer and rounded once.  Two
    participants of 2^24 + 1 tokens each weigh 2^24 against a total of
    fp32(2^25 + 2) = 2^25, so the mean delta is (d1 + d2) / 2 exactly."""
    rng = np.random.default_rng(115)
    theta = dyadic(rng, 64, frac_bits=10)
    c1, c2 = dyadic(rng, 64, frac_bits=10), dyadic(rng, 64, frac_bits=10)
    th = theta.copy()
    m = np.zeros_like(th)
    t = (1 << 24) + 1
    orc.nesterov_fragment_round(th, m, [c1, c2], [t, t], 1.0, 0.0)
    want = [f32_rne((Fraction(float(a)) + Fraction(float(b))) / 2) for a, b in zip(c1, c2)]
    assert_bits_equal(th, want, "weights rounded once")


def pin_delta_sign_and_weights(orc):
    """One participant with t tokens: the accumulated value is t (theta - c),
    exactly, for dyadic data (the delta points from the snapshot to the
    global)."""
    theta = np.array([1.0, -0.5, 0.25, 0.0], np.float32)
    c = np.array([0.75, -0.25, 0.25, 2.0 ** -10], np.float32)
    acc = np.empty(4, np.float32)
    orc.fold_delta(acc, theta, c, 6, first=True)
    assert_bits_equal(acc, [1.5, -1.5, 0.0, -6 * 2.0 ** -10], "t (theta - c)")
    orc.fold_delta(acc, theta, c, 2, first=False)
    assert_bits_equal(acc, [2.0, -2.0, 0.0, -8 * 2.0 ** -10], "second arrival adds")


def pin_uniform_average_of_130_globals(orc):
    """The published model averages 130 globals with equal weights (technical
    report, "Data and schedule").  Dyadic globals with 14 fraction bits keep
    every partial sum of 130 of them exact in binary32, so the average must be
    the correctly rounded rational mean; the last-3 and last-5 snapshot
    averages (Table 5) likewise."""
    rng = np.random.default_rng(116)
    n = 128
    gs = [dyadic(rng, n, frac_bits=14) for _ in range(130)]
    got = orc.swa_average(gs)
    want = [f32_rne(sum(Fraction(float(g[j])) for g in gs) / 130) for j in range(n)]
    assert_bits_equal(got, want, "uniform average of 130 globals")
    for k in (3, 5):
        got = orc.snapshot_average(gs[-k:])
        want = [f32_rne(sum(Fraction(float(g[j])) for g in gs[-k:]) / k) for j in range(n)]
        assert_bits_equal(got, want, f"average of the last {k} snapshots")


def pin_adopt_keep_drift(orc):
    """Keep-local-drift adoption theta + (g - pushed) (technical report,
    "Distributed optimisation"): exact on dyadic data; a worker that made no
    progress since its push (theta == pushed) lands exactly on the global
    when the difference is exact (Sterbenz range); plain replacement is the
    other policy and is not this function."""
    rng = np.random.default_rng(117)
    n = 2048
    theta, g, pushed = (dyadic(rng, n, frac_bits=12) for _ in range(3))
    th = theta.copy()
    orc.adopt_keep_drift(th, g, pushed)
    want = [f32_rne(Fraction(float(t)) + (Fraction(float(a)) - Fraction(float(b))))
            for t, a, b in zip(theta, g, pushed)]
    assert_bits_equal(th, want, "theta + (g - pushed)")
    # no progress since the push: the worker takes the global
    x = (1.0 + rng.random(n)).astype(np.float32)
    gg = (x * np.float32(1.5)).astype(np.float32)        # within a factor 2: exact difference
    th = x.copy()
    orc.adopt_keep_drift(th, gg, x.copy())
    assert_bits_equal(th, gg, "no progress -> global")
    # bf16 pushed checkpoints are widened exactly
    import torch
    pb = torch.from_numpy(pushed).to(torch.bfloat16)
    pbits = pb.view(torch.int16).numpy().view(np.uint16).copy()
    th = theta.copy()
    orc.adopt_keep_drift(th, g, pbits)
    wid = pb.float().numpy()
    want = [f32_rne(Fraction(float(t)) + (Fraction(float(a)) - Fraction(float(b))))
            for t, a, b in zip(theta, g, wid)]
    assert_bits_equal(th, want, "bf16 pushed")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
