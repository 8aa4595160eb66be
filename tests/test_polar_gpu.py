"""Outer orthogonalisation on the GPU against the fp64 oracle (DiffuRefill-1B
technical report, "What we measured", "Optimisers": the averaged outer
update is replaced by its polar factor).

Every element of every polar factor and outer step below is compared with
the oracle's exact-arithmetic iteration result U phi(S/||A||_F) V^T.  That
result is U V^T wherever the iteration has converged.  The per-element
tolerance is the first-order propagation of the fp32 iteration's rounding
errors through the singular bases of A (tests/polar_tolerance.py).

The Frobenius-norm checks stay as a second line.  Their tolerances come
from the arithmetic:
  * the fp32 MFMA product: any summation order of k products in binary32
    stays within gamma_(k+1) = (k+1) u / (1 - (k+1) u) of the exact sum
    times the sum of magnitudes, plus one rounding per epilogue operation;
  * the polar factor: the iteration's rounding errors act as a perturbation
    of relative size ~ sqrt(r) u on each iterate, and the polar factor moves
    by at most ~ 2 ||dX|| / sigma_min(X) under a perturbation dX, so the
    error relative to ||P||_F is bounded by C sqrt(r) u kappa_F with
    kappa_F = ||A||_F / sigma_min(A) (the iteration starts from A / ||A||_F)
    and C = 16 covering the three products per step and the geometric sum
    over steps while sigma_min grows.
"""
import math

import numpy as np
import pytest
import torch

from checkpoint_averaging_amd import dlmerge as dl
from checkpoint_averaging_amd import synth
from oracle import polar as opolar
from tests import polar_tolerance as pt

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24           # unit roundoff of binary32
C_POLAR = 16.0
DEV = torch.device("cuda")


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.float64)


def workspace(rows, cols):
    nbytes = dl.dl_polar_workspace_bytes(rows, cols)
    return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=DEV)


def orthonormal(rng, m, r):
    q, _ = np.linalg.qr(rng.standard_normal((m, r)))
    return q


def constructed(rng, m, n, kappa):
    r = min(m, n)
    q1, q2 = orthonormal(rng, m, r), orthonormal(rng, n, r)
    s = np.logspace(0, -np.log10(kappa), r)
    return ((q1 * s) @ q2.T).astype(np.float32)


def polar_bound(a64):
    s = np.linalg.svd(a64, compute_uv=False)
    r = min(a64.shape)
    kappa_f = np.linalg.norm(a64) / s[-1]
    return C_POLAR * math.sqrt(r) * U32 * kappa_f


def polar_estimate(a64):
    """Random-rounding estimate of the same error.  Early steps: a few
    roundings per step (relative u each, independent across elements)
    perturb X by ~u in norm, which moves P by ~2u/sigma_min(X); summed
    geometrically over the steps while sigma_min grows, ~8u kappa_2.  Late
    steps, with X already orthonormal: each element of a product is a sum of
    r terms whose rounding errors add like a random walk, ~sqrt(r) u per
    element and step.  Together, with margin: 16 u (kappa_2 + sqrt(r))."""
    s = np.linalg.svd(a64, compute_uv=False)
    return estimate_from(s[0] / s[-1], min(a64.shape))


def estimate_from(kappa_2, r):
    return 16.0 * U32 * (kappa_2 + math.sqrt(r))


# -- the MFMA product ---------------------------------------------------------

@pytest.mark.parametrize("form", [dl.DL_TN, dl.DL_NT], ids=["TN", "NT"])
@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (130, 257, 33), (300, 129, 500), (128, 128, 16),
                                   (5, 700, 3), (640, 256, 1)])
@pytest.mark.parametrize("epi", ["plain", "y_separate", "y_in_place"])
def test_matmul_against_fp64(form, m, n, k, epi):
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    pad = 3
    if form == dl.DL_TN:
        a = rng.standard_normal((k, m + pad)).astype(np.float32)
        b = rng.standard_normal((k, n + pad)).astype(np.float32)
        opa, opb = a[:, :m].astype(np.float64).T, b[:, :n].astype(np.float64)
    else:
        a = rng.standard_normal((m, k + pad)).astype(np.float32)
        b = rng.standard_normal((n, k + pad)).astype(np.float32)
        opa, opb = a[:, :k].astype(np.float64), b[:, :k].astype(np.float64).T
    ldc = n + 5
    c0 = rng.standard_normal((m, ldc)).astype(np.float32)
    y0 = rng.standard_normal((m, ldc)).astype(np.float32)
    alpha, beta, diag = (1.0, 0.0, 0.0) if epi == "plain" else (-0.5, 2.0315, 3.4445)
    a_d, b_d, c_d = gpu(a), gpu(b), gpu(c0)
    y_d = None if epi == "plain" else (c_d if epi == "y_in_place" else gpu(y0))
    y_h = None if epi == "plain" else (c0 if epi == "y_in_place" else y0)[:, :n].astype(np.float64)
    dl.dl_matmul_f32(form, a_d, a.shape[1], b_d, b.shape[1], m, n, k, c_d, ldc, y_d,
                     alpha, beta, diag)
    got = host(c_d)
    want = alpha * (opa @ opb)
    mag = abs(alpha) * (np.abs(opa) @ np.abs(opb))
    if y_h is not None:
        want = want + beta * y_h
        mag = mag + abs(beta) * np.abs(y_h)
    eye = np.eye(m, n) * diag
    want, mag = want + eye, mag + np.abs(eye)
    g = (k + 4) * U32 / (1 - (k + 4) * U32)
    err = np.abs(got[:, :n] - want)
    assert np.all(err <= g * mag + 1e-30), (float(np.max(err / (mag + 1e-30))), g)
    # columns past n are untouched
    assert np.array_equal(got[:, n:], c0[:, n:].astype(np.float64))


def _bound_check(got, want, mag, k):
    g = (k + 4) * U32 / (1 - (k + 4) * U32)
    err = np.abs(got - want)
    assert np.all(err <= g * mag + 1e-30), (float(np.max(err / (mag + 1e-30))), g)


@pytest.mark.parametrize("form,m,n,k,lda_pad", [
    # k-major operands with row counts divisible by 4 and aligned pitches:
    # the edge tiles take the plain loads with clamped rows
    (dl.DL_TN, 132, 260, 96, 0), (dl.DL_TN, 1100, 1000, 64, 4), (dl.DL_TN, 4, 388, 32, 0),
    # aligned pitches but row counts not divisible by 4: guarded edge tiles
    (dl.DL_TN, 130, 258, 96, 2), (dl.DL_TN, 7, 129, 64, 1),
    # row-major operands with aligned pitches: any row count clamps
    (dl.DL_NT, 129, 131, 96, 0), (dl.DL_NT, 1, 300, 64, 4), (dl.DL_NT, 257, 3, 160, 0),
    # and with a partial last K-tile
    (dl.DL_NT, 200, 130, 100, 0), (dl.DL_TN, 200, 132, 100, 0),
])
@pytest.mark.parametrize("ws_mode", ["stream", "none"])
def test_matmul_edge_tiles(form, m, n, k, lda_pad, ws_mode):
    """Edge tiles (rows past the last output row or column) against fp64,
    for the pitch and row-count combinations that pick the clamped plain
    loads or the guarded ones, with and without the stream-K split."""
    rng = np.random.default_rng(m * 5 + n * 11 + k + lda_pad)
    if form == dl.DL_TN:
        lda, ldb = m + lda_pad, n + lda_pad
        a = rng.standard_normal((k, lda)).astype(np.float32)
        b = rng.standard_normal((k, ldb)).astype(np.float32)
        opa, opb = a[:, :m].astype(np.float64).T, b[:, :n].astype(np.float64)
    else:
        lda = ldb = k + lda_pad
        a = rng.standard_normal((m, lda)).astype(np.float32)
        b = rng.standard_normal((n, ldb)).astype(np.float32)
        opa, opb = a[:, :k].astype(np.float64), b[:, :k].astype(np.float64).T
    want, mag = opa @ opb, np.abs(opa) @ np.abs(opb)
    ldc = n + 3
    c0 = rng.standard_normal((m, ldc)).astype(np.float32)
    c_d = gpu(c0)
    ws = None
    if ws_mode == "stream":
        wsb = dl.dl_matmul_workspace_bytes(m, n, k, False)
        ws = torch.empty(max(wsb, 256) // 4, dtype=torch.float32, device=DEV)
    dl.dl_matmul_f32(form, gpu(a), lda, gpu(b), ldb, m, n, k, c_d, ldc, workspace=ws)
    got = host(c_d)
    _bound_check(got[:, :n], want, mag, k)
    assert np.array_equal(got[:, n:], c0[:, n:].astype(np.float64))


@pytest.mark.parametrize("form", [dl.DL_TN, dl.DL_NT], ids=["TN", "NT"])
@pytest.mark.parametrize("n,k", [(1, 5), (130, 33), (300, 700), (257, 2000), (128, 4096),
                                 (384, 300), (5760, 100)])
@pytest.mark.parametrize("ws_mode", ["stream", "none"])
@pytest.mark.parametrize("y_mode", ["none", "separate", "in_place"])
def test_matmul_symmetric(form, n, k, ws_mode, y_mode):
    """A Gram product (X^T X as TN, X X^T as NT) declared symmetric: the upper
    triangle within the product bound, the lower one its exact mirror."""
    rng = np.random.default_rng(n * 13 + k)
    x = rng.standard_normal((k, n + 2) if form == dl.DL_TN else (n, k + 2)).astype(np.float32)
    x64 = x.astype(np.float64)
    gram = x64[:, :n].T @ x64[:, :n] if form == dl.DL_TN else x64[:, :k] @ x64[:, :k].T
    mag = np.abs(x64[:, :n]).T @ np.abs(x64[:, :n]) if form == dl.DL_TN else \
        np.abs(x64[:, :k]) @ np.abs(x64[:, :k]).T
    ldc = n + 3
    r = rng.standard_normal((n, n)).astype(np.float32)
    ysym = np.zeros((n, ldc), np.float32)
    ysym[:, :n] = (r + r.T) * np.float32(0.5)
    c0 = ysym.copy() if y_mode == "in_place" else rng.standard_normal((n, ldc)).astype(np.float32)
    alpha, beta, diag = (1.0, 0.0, 0.0) if y_mode == "none" else (2.0315, -4.775, 3.4445)
    x_d, c_d = gpu(x), gpu(c0)
    y_d = None if y_mode == "none" else (c_d if y_mode == "in_place" else gpu(ysym))
    ws = None
    if ws_mode == "stream":
        ws = torch.empty(dl.dl_matmul_workspace_bytes(n, n, k, True) // 4, dtype=torch.float32,
                         device=DEV)
    dl.dl_matmul_f32(form, x_d, x.shape[1], x_d, x.shape[1], n, n, k, c_d, ldc, y_d, alpha, beta,
                     diag, symmetric=True, workspace=ws)
    got = host(c_d)
    want = alpha * gram + np.eye(n) * diag
    mg = abs(alpha) * mag + np.abs(np.eye(n) * diag)
    if y_mode != "none":
        want = want + beta * ysym[:, :n].astype(np.float64)
        mg = mg + abs(beta) * np.abs(ysym[:, :n].astype(np.float64))
    _bound_check(got[:, :n], want, mg, k)
    assert np.array_equal(got[:, :n], got[:, :n].T)
    assert np.array_equal(got[:, n:], c0[:, n:].astype(np.float64))


@pytest.mark.parametrize("form", [dl.DL_TN, dl.DL_NT], ids=["TN", "NT"])
@pytest.mark.parametrize("m,n,k", [(100, 100, 5000), (256, 256, 2048), (129, 300, 1000),
                                   (640, 384, 777), (1100, 1000, 96), (3000, 200, 4100),
                                   (4224, 4000, 300)])
def test_matmul_stream_k(form, m, n, k):
    """With a workspace the work is spread over the resident workgroups
    (whole-tile rounds while at least two rounds' worth remain, then
    stream-K runs) and tiles cut between them are summed in K order: within
    the product bound, the same bits on a second call; without one, one
    workgroup per tile, also within the bound.  4224 x 4000 x 300 has 1056
    tiles: one whole-tile round of 512, then 544 tiles in runs of ~10.6
    K-tiles."""
    rng = np.random.default_rng(m + n + k)
    if form == dl.DL_TN:
        a = rng.standard_normal((k, m)).astype(np.float32)
        b = rng.standard_normal((k, n)).astype(np.float32)
        opa, opb = a.astype(np.float64).T, b.astype(np.float64)
        lda, ldb = m, n
    else:
        a = rng.standard_normal((m, k)).astype(np.float32)
        b = rng.standard_normal((n, k)).astype(np.float32)
        opa, opb = a.astype(np.float64), b.astype(np.float64).T
        lda, ldb = k, k
    want, mag = opa @ opb, np.abs(opa) @ np.abs(opb)
    a_d, b_d = gpu(a), gpu(b)
    wsb = dl.dl_matmul_workspace_bytes(m, n, k, False)
    assert wsb > 0
    outs = []
    for use_ws in (True, True, False):
        ws = torch.empty(wsb // 4, dtype=torch.float32, device=DEV) if use_ws else None
        c_d = torch.empty((m, n), device=DEV)
        dl.dl_matmul_f32(form, a_d, lda, b_d, ldb, m, n, k, c_d, n, workspace=ws)
        outs.append(host(c_d))
        _bound_check(outs[-1], want, mag, k)
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("form", [dl.DL_TN, dl.DL_NT], ids=["TN", "NT"])
@pytest.mark.parametrize("m,k,sym,epi", [(1000, 30000, True, False), (1024, 28672, True, True),
                                         (512, 65536, False, True)])
def test_matmul_split_k(form, m, k, sym, epi):
    """Few output tiles over a long K (the Gram product of a tall matrix): K
    is cut into ranges dealt out range by range over the tiles, and each
    tile's pieces are summed in K order by a second kernel.  Within the
    product bound of fp64, the same bits on a second call, an exactly
    symmetric result; without a workspace (one workgroup per tile, the
    whole K in order) also within the bound."""
    n = m
    rng = np.random.default_rng(m + k)
    if form == dl.DL_TN:
        a = rng.standard_normal((k, m)).astype(np.float32)
        b = a if sym else rng.standard_normal((k, n)).astype(np.float32)
        opa, opb = a.astype(np.float64).T, b.astype(np.float64)
        lda = ldb = m
    else:
        a = rng.standard_normal((m, k)).astype(np.float32)
        b = a if sym else rng.standard_normal((n, k)).astype(np.float32)
        opa, opb = a.astype(np.float64), b.astype(np.float64).T
        lda = ldb = k
    alpha, beta, diag = (-0.5, 2.0, 1.5) if epi else (1.0, 0.0, 0.0)
    y0 = rng.standard_normal((m, n)).astype(np.float32)
    if sym:
        y0 = (y0 + y0.T) / 2
    want = alpha * (opa @ opb) + (beta * y0.astype(np.float64) if epi else 0) + diag * np.eye(m)
    mag = abs(alpha) * (np.abs(opa) @ np.abs(opb)) + (abs(beta) * np.abs(y0) if epi else 0) + \
        abs(diag) * np.eye(m)
    a_d = gpu(a)
    b_d = a_d if sym else gpu(b)
    y_d = gpu(y0) if epi else None
    wsb = dl.dl_matmul_workspace_bytes(m, n, k, sym)
    assert wsb > 0
    outs = []
    for ws_bytes in (wsb, wsb, 0):
        ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=DEV) if ws_bytes else None
        c_d = torch.empty((m, n), device=DEV)
        dl.dl_matmul_f32(form, a_d, lda, b_d, ldb, m, n, k, c_d, n, y_d, alpha, beta, diag,
                         symmetric=sym, workspace=ws)
        outs.append(host(c_d))
        _bound_check(outs[-1], want, mag, k)
        if sym:
            assert np.array_equal(outs[-1], outs[-1].T)
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("m,n,k,batch,epi", [
    (4096 + 37, 4096 + 64, 80, 1, "plain"),       # main block + both strips
    (4096 + 37, 4096 + 64, 80, 1, "y_in_place"),  # theta - s P style epilogue
    (2048, 2048, 512, 4, "plain"),                # a batch filling one round exactly
    (2048, 2048 + 200, 96, 4, "y_separate"),      # batch, right strip, separate Y
])
def test_matmul_large_tiles(m, n, k, batch, epi):
    """Plain row-major (NT) products with at least 256 tiles of 256 x 256
    run their main block on the large-tile kernel (one wave per SIMD) and
    the ragged strips on the general one: every element within the product
    bound of fp64, the same bits on a second call."""
    assert dl.dl_matmul_large_tiles(m, n, k, False, batch,
                                    dl.dl_matmul_workspace_bytes_batch(m, n, k, False, batch))
    rng = np.random.default_rng(m + n + k + batch)
    a = rng.standard_normal((batch, m, k)).astype(np.float32)
    b = rng.standard_normal((batch, n, k)).astype(np.float32)
    c0 = rng.standard_normal((batch, m, n)).astype(np.float32)
    y0 = rng.standard_normal((batch, m, n)).astype(np.float32)
    alpha, beta = (1.0, 0.0) if epi == "plain" else (-0.25, 1.0)
    a_d, b_d = gpu(a), gpu(b)
    y_h = None if epi == "plain" else (c0 if epi == "y_in_place" else y0)
    wsb = dl.dl_matmul_workspace_bytes_batch(m, n, k, False, batch)
    ws = torch.empty(max(wsb, 256) // 4, dtype=torch.float32, device=DEV)
    outs = []
    for _ in range(2):
        c_d = gpu(c0)
        y_d = None if epi == "plain" else (c_d if epi == "y_in_place" else gpu(y0))
        dl.dl_matmul_f32_batch(dl.DL_NT, a_d, k, m * k, b_d, k, n * k, m, n, k, c_d, n, m * n,
                               batch, y=y_d, stride_y=m * n if y_d is not None else 0,
                               alpha=alpha, beta=beta, workspace=ws)
        outs.append(host(c_d))
    assert np.array_equal(outs[0], outs[1])
    for i in range(batch):
        a64, b64 = a[i].astype(np.float64), b[i].astype(np.float64)
        want = alpha * (a64 @ b64.T)
        mag = abs(alpha) * (np.abs(a64) @ np.abs(b64).T)
        if y_h is not None:
            want = want + beta * y_h[i].astype(np.float64)
            mag = mag + abs(beta) * np.abs(y_h[i].astype(np.float64))
        _bound_check(outs[0][i], want, mag, k)


@pytest.mark.parametrize("form,m,n,k,batch,sym,epi", [
    (dl.DL_TN, 2048 + 40, 2048, 96, 4, False, "plain"),        # k-major operands, bottom strip
    (dl.DL_TN, 2048, 2048 + 72, 128, 4, False, "y_in_place"),  # right strip, theta - s P style
    (dl.DL_TN, 2048, 2048, 2048, 8, True, "plain"),    # Gram: upper tiles, last round's split
    (dl.DL_TN, 2048, 2048, 2048, 8, True, "cubic"),    # -0.5 G + 1.5 I
    (dl.DL_NT, 2048, 2048, 2048, 8, True, "square"),   # c G G + b G + a I, G symmetric
    (dl.DL_TN, 2048, 2048, 16384, 1, True, "plain"),   # few tiles over a long K: all in pieces
], ids=["TN-strip-rows", "TN-strip-cols-y", "TN-gram", "TN-gram-cubic", "NT-square",
        "TN-gram-longK"])
def test_matmul_large_tiles_forms(form, m, n, k, batch, sym, epi):
    """The large-tile kernel with k-major operands (transposed on their way to
    LDS) and with symmetric results (upper tiles only, mirrored; the last
    round's tiles cut along K and summed in K order by a second kernel):
    every element within the product bound of fp64 (computed on the GPU in
    fp64), symmetric results exactly symmetric, the same bits on a second
    call."""
    wsb = dl.dl_matmul_workspace_bytes_batch(m, n, k, sym, batch)
    assert dl.dl_matmul_large_tiles(m, n, k, sym, batch, wsb)
    rng = np.random.default_rng(m + 3 * n + 7 * k + batch + len(epi))
    if form == dl.DL_TN:
        a = rng.standard_normal((batch, k, m)).astype(np.float32)
        b = a if sym else rng.standard_normal((batch, k, n)).astype(np.float32)
        lda, ldb = m, n
    else:
        a = rng.standard_normal((batch, m, k)).astype(np.float32)
        if epi == "square":   # a symmetric G (m == k), exactly
            a = ((a + np.transpose(a, (0, 2, 1))) * np.float32(0.5)).astype(np.float32)
        b = a if sym else rng.standard_normal((batch, n, k)).astype(np.float32)
        lda, ldb = k, k
    c0 = rng.standard_normal((batch, m, n)).astype(np.float32)
    alpha, beta, diag = {"plain": (1.0, 0.0, 0.0), "y_in_place": (-0.25, 1.0, 0.0),
                         "cubic": (-0.5, 0.0, 1.5),
                         "square": (2.0315, -4.7750, 3.4445)}[epi]
    a_d = gpu(a)
    b_d = a_d if b is a else gpu(b)
    ws = torch.empty(max(wsb, 256) // 4, dtype=torch.float32, device=DEV)
    outs = []
    for _ in range(2):
        c_d = gpu(c0)
        y_d = {"y_in_place": c_d, "square": a_d}.get(epi)
        dl.dl_matmul_f32_batch(form, a_d, lda, a[0].size, b_d, ldb, b[0].size, m, n, k, c_d, n,
                               m * n, batch, y=y_d, stride_y=m * n if y_d is not None else 0,
                               alpha=alpha, beta=beta, diag=diag, symmetric=sym, workspace=ws)
        outs.append(host(c_d))
    assert np.array_equal(outs[0], outs[1])
    a64, b64 = a_d.double(), b_d.double()
    for i in range(batch):
        ai, bi = (a64[i].T, b64[i]) if form == dl.DL_TN else (a64[i], b64[i].T)
        want = alpha * (ai @ bi)
        mag = abs(alpha) * (ai.abs() @ bi.abs())
        if epi == "y_in_place":
            y64 = torch.from_numpy(c0[i]).to(DEV, torch.float64)
        elif epi == "square":
            y64 = a64[i]
        else:
            y64 = None
        if y64 is not None:
            want = want + beta * y64
            mag = mag + abs(beta) * y64.abs()
        if diag:
            want = want + diag * torch.eye(m, dtype=torch.float64, device=DEV)
            mag = mag + abs(diag) * torch.eye(m, dtype=torch.float64, device=DEV)
        _bound_check(outs[0][i], host(want), host(mag), k)
        if sym:
            assert np.array_equal(outs[0][i], outs[0][i].T)


# shapes drawn once from a seeded generator (ragged M and N, K from 112 to
# 2800, batches from 12 to 38) and kept where the library takes the
# large-tile path: whole rounds, last rounds cut along K into pieces of
# unequal length, strips on both sides
SEEDED_BIG = [
    (dl.DL_TN, 1316, 1124, 2528, 28, False), (dl.DL_TN, 1540, 1024, 2112, 12, False),
    (dl.DL_TN, 2048, 2048, 2800, 38, True), (dl.DL_NT, 2308, 1792, 1344, 36, False),
    (dl.DL_NT, 1280, 1536, 1520, 23, False), (dl.DL_TN, 2308, 2560, 112, 27, False),
    (dl.DL_NT, 2048, 2048, 1328, 32, True), (dl.DL_TN, 2432, 1636, 1040, 29, False),
]


@pytest.mark.parametrize("form,m,n,k,batch,sym", SEEDED_BIG)
def test_matmul_large_tiles_seeded_shapes(form, m, n, k, batch, sym):
    """Seeded shapes on the large-tile path, with Y, and a diagonal term
    where the result's diagonal lies in the main block: every element
    within the product bound of fp64 (checked on the GPU), symmetric
    results exactly symmetric."""
    _check_big_product(form, m, n, k, batch, sym,
                       0.75 if sym or (m % 256 == 0 and n % 256 == 0) else 0.0)


@pytest.mark.parametrize("form", [dl.DL_TN, dl.DL_NT], ids=["TN", "NT"])
def test_matmul_diagonal_term_with_ragged_edges(form):
    """A non-symmetric product with a diagonal term and ragged edges: the
    diagonal crosses into the strips past the last whole 256 rows and
    columns, so the whole product runs on the general kernel (a strip's own
    diagonal is not the result's; adding the term there once put it on the
    wrong elements)."""
    _check_big_product(form, 1316, 1124, 2528, 28, False, 0.75, shape_takes_large_tiles=None)


def _check_big_product(form, m, n, k, batch, sym, diag, shape_takes_large_tiles=True):
    wsb = dl.dl_matmul_workspace_bytes_batch(m, n, k, sym, batch)
    if shape_takes_large_tiles is not None:
        assert dl.dl_matmul_large_tiles(m, n, k, sym, batch, wsb) == shape_takes_large_tiles
    g = torch.Generator(device=DEV).manual_seed(m * 7 + n * 3 + k + batch)
    rows_a, rows_b = (k, k) if form == dl.DL_TN else (m, n)
    cols_a, cols_b = (m, n) if form == dl.DL_TN else (k, k)
    a_d = torch.randn(batch, rows_a, cols_a, generator=g, device=DEV)
    b_d = a_d if sym else torch.randn(batch, rows_b, cols_b, generator=g, device=DEV)
    y_d = torch.randn(batch, m, n, generator=g, device=DEV)
    if sym:
        y_d = (y_d + y_d.transpose(1, 2).contiguous()) * 0.5
    c_d = torch.full((batch, m, n), float("nan"), device=DEV)
    alpha, beta = 0.625, -1.5
    ws = torch.empty(max(wsb, 256) // 4, dtype=torch.float32, device=DEV)
    dl.dl_matmul_f32_batch(form, a_d, cols_a, rows_a * cols_a, b_d, cols_b, rows_b * cols_b, m,
                           n, k, c_d, n, m * n, batch, y=y_d, stride_y=m * n, alpha=alpha,
                           beta=beta, diag=diag, symmetric=sym, workspace=ws)
    torch.cuda.synchronize()
    gam = (k + 4) * U32 / (1 - (k + 4) * U32)
    eye = torch.eye(m, n, dtype=torch.float64, device=DEV)
    for i in range(batch):
        a64, b64 = a_d[i].double(), b_d[i].double()
        ai, bi = (a64.T, b64) if form == dl.DL_TN else (a64, b64.T)
        y64 = y_d[i].double()
        want = alpha * (ai @ bi) + beta * y64 + diag * eye
        mag = abs(alpha) * (ai.abs() @ bi.abs()) + abs(beta) * y64.abs() + abs(diag) * eye
        err = (c_d[i].double() - want).abs()
        assert bool((err <= gam * mag + 1e-30).all()), (i, float((err / (mag + 1e-30)).max()))
        if sym:
            assert torch.equal(c_d[i], c_d[i].T)


@pytest.mark.parametrize("form,sym", [(dl.DL_TN, False), (dl.DL_NT, True), (dl.DL_TN, True)],
                         ids=["TN-general", "NT-symmetric", "TN-symmetric"])
def test_matmul_large_tiles_strided(form, sym):
    """The large-tile kernel on a strided batch: padded leading dimensions
    (still 16-byte aligned), batch strides with gaps, Y at its own stride,
    a result pitch wider than the result.  Every element within the product
    bound, symmetric results exactly symmetric, the gaps untouched."""
    batch, m = 8, 2048
    k = 2048 if sym else 1024   # enough work per tile for the symmetric split to pay
    n = m if sym else 2048 + 256
    lda = (k if form == dl.DL_NT else m) + 4
    ldb = (k if form == dl.DL_NT else n) + 4
    rows_a = m if form == dl.DL_NT else k
    rows_b = n if form == dl.DL_NT else k
    sa = lda * rows_a + 16
    sb = sa if sym else ldb * rows_b + 32   # symmetric: B is A
    ldc = n + 8
    sc, sy = ldc * m + 64, ldc * m + 128
    wsb = dl.dl_matmul_workspace_bytes_batch(m, n, k, sym, batch)
    assert dl.dl_matmul_large_tiles(m, n, k, sym, batch, wsb)
    rng = np.random.default_rng(4242 + form + 2 * sym)
    a = rng.standard_normal(sa * batch).astype(np.float32)
    b = a if sym else rng.standard_normal(sb * batch).astype(np.float32)
    c0 = rng.standard_normal(sc * batch).astype(np.float32)
    yv = rng.standard_normal(sy * batch).astype(np.float32)
    for i in range(batch):   # a symmetric Y for the symmetric case
        yy = yv[i * sy:i * sy + m * ldc].reshape(m, ldc)
        if sym:
            yy[:, :n] = (yy[:, :n] + yy[:, :n].T) * np.float32(0.5)
    alpha, beta, diag = (0.75, -0.5, 1.25) if sym else (-0.25, 2.0, 0.5)
    a_d, y_d = gpu(a), gpu(yv)
    b_d = a_d if sym else gpu(b)
    ws = torch.empty(max(wsb, 256) // 4, dtype=torch.float32, device=DEV)
    c_d = gpu(c0)
    dl.dl_matmul_f32_batch(form, a_d, lda, sa, b_d, ldb, sb, m, n, k, c_d, ldc, sc, batch,
                           y=y_d, stride_y=sy, alpha=alpha, beta=beta, diag=diag,
                           symmetric=sym, workspace=ws)
    out = host(c_d)
    a64, b64 = a_d.double(), b_d.double()
    y64 = y_d.double()
    eye = torch.eye(m, n, dtype=torch.float64, device=DEV)
    for i in range(batch):
        av = a64[i * sa:i * sa + rows_a * lda].reshape(rows_a, lda)
        bv = b64[i * sb:i * sb + rows_b * ldb].reshape(rows_b, ldb)
        ai, bi = (av[:, :m].T, bv[:, :n]) if form == dl.DL_TN else (av[:, :k], bv[:, :k].T)
        yi = y64[i * sy:i * sy + m * ldc].reshape(m, ldc)[:, :n]
        want = alpha * (ai @ bi) + beta * yi + diag * eye
        mag = abs(alpha) * (ai.abs() @ bi.abs()) + abs(beta) * yi.abs() + abs(diag) * eye
        ci = out[i * sc:i * sc + m * ldc].reshape(m, ldc)
        _bound_check(ci[:, :n], host(want), host(mag), k)
        if sym:
            assert np.array_equal(ci[:, :n], ci[:, :n].T)
        # the row padding and the gap after the matrix are untouched
        c0i = c0[i * sc:i * sc + m * ldc].reshape(m, ldc)
        assert np.array_equal(ci[:, n:], c0i[:, n:])
        assert np.array_equal(out[i * sc + m * ldc:(i + 1) * sc], c0[i * sc + m * ldc:(i + 1) * sc])


@pytest.mark.parametrize("form", [dl.DL_TN, dl.DL_NT], ids=["TN", "NT"])
@pytest.mark.parametrize("sym", [False, True], ids=["general", "symmetric"])
@pytest.mark.parametrize("ws_mode", ["stream", "none"])
def test_matmul_batch(form, sym, ws_mode):
    """A strided batch of products in one launch: every matrix within the
    product bound (and exactly mirrored when symmetric); Y read with its own
    stride; the gaps between the batch's results untouched."""
    rng = np.random.default_rng(91 + int(sym) + 2 * form)
    batch, m, k = 5, 300, 260
    n = m if sym else 170
    if form == dl.DL_TN:
        lda, sa = m + 1, (m + 1) * k + 7
        ldb, sb = (lda, sa) if sym else (n + 3, (n + 3) * k + 5)
    else:
        lda, ldb, sa = k + 2, k + 2, m * (k + 2) + 3
        sb = sa if sym else n * (k + 2) + 9
    a = rng.standard_normal(sa * batch).astype(np.float32)
    b = a if sym else rng.standard_normal(sb * batch).astype(np.float32)
    ldc, sc = n + 4, (n + 4) * m + 64
    c0 = rng.standard_normal(sc * batch).astype(np.float32)
    sy = sc + 32
    yv = rng.standard_normal(sy * batch).astype(np.float32)
    for i in range(batch):        # a symmetric Y for the symmetric case
        yy = yv[i * sy:i * sy + m * ldc].reshape(m, ldc)
        if sym:
            yy[:, :n] = (yy[:, :n] + yy[:, :n].T) * np.float32(0.5)
    a_d, c_d, y_d = gpu(a), gpu(c0), gpu(yv)
    b_d = a_d if sym else gpu(b)
    ws = None
    if ws_mode == "stream":
        ws = torch.empty(dl.dl_matmul_workspace_bytes_batch(m, n, k, sym, batch) // 4 + 64,
                         device=DEV)
    alpha, beta, diag = -0.5, 2.0315, 3.4445
    dl.dl_matmul_f32_batch(form, a_d, lda, sa, b_d, ldb, sb, m, n, k, c_d, ldc, sc, batch, y=y_d,
                           stride_y=sy, alpha=alpha, beta=beta, diag=diag, symmetric=sym,
                           workspace=ws)
    got = host(c_d)
    for i in range(batch):
        ai = a[i * sa:].astype(np.float64)
        bi = b[i * sb:].astype(np.float64)
        if form == dl.DL_TN:
            opa = ai[:k * lda].reshape(k, lda)[:, :m].T
            opb = bi[:k * ldb].reshape(k, ldb)[:, :n]
        else:
            opa = ai[:m * lda].reshape(m, lda)[:, :k]
            opb = bi[:n * ldb].reshape(n, ldb)[:, :k].T
        yi = yv[i * sy:i * sy + m * ldc].reshape(m, ldc)[:, :n].astype(np.float64)
        want = alpha * (opa @ opb) + beta * yi + diag * np.eye(m, n)
        mag = abs(alpha) * (np.abs(opa) @ np.abs(opb)) + abs(beta) * np.abs(yi) + abs(diag) * np.eye(m, n)
        gi = got[i * sc:i * sc + m * ldc].reshape(m, ldc)
        _bound_check(gi[:, :n], want, mag, k)
        if sym:
            assert np.array_equal(gi[:, :n], gi[:, :n].T)
        assert np.array_equal(gi[:, n:], c0[i * sc:i * sc + m * ldc].reshape(m, ldc)[:, n:])
        gap = slice(i * sc + m * ldc, (i + 1) * sc)
        assert np.array_equal(got[gap], c0[gap].astype(np.float64))


def test_matmul_k0_writes_the_epilogue():
    m, n = 70, 90
    c = torch.full((m, n), 7.0, device=DEV)
    y = gpu(np.arange(m * n, dtype=np.float32).reshape(m, n))
    a = torch.zeros(1, device=DEV)
    dl.dl_matmul_f32(dl.DL_NT, a, 0, a, 0, m, n, 0, c, n, y, 1.0, 0.5, 2.0)
    want = np.float32(0.5) * np.arange(m * n, dtype=np.float32).reshape(m, n) + 2.0 * np.eye(m, n)
    assert np.array_equal(host(c), want.astype(np.float32).astype(np.float64))


# -- element-wise parity helpers -------------------------------------------------

def assert_factor_elementwise(got, a64, what, quintic=12, cubic=6):
    """Every element of a computed factor within the per-element tolerance
    of the oracle's iterated factor; returns the oracle's figures."""
    e = pt.expected(a64, quintic, cubic)
    z = pt.report(got, e, what)
    assert z <= pt.Z, (what, z)
    return e


def assert_step_elementwise(got_theta, theta, upd, scale, what, e=None):
    """Every element of theta' = theta - scale * P within |scale| times the
    factor's tolerance plus the step's two binary32 roundings, about theta -
    scale * (the oracle's iterated factor of the update)."""
    if e is None:
        e = pt.expected(upd)
    want = theta - scale * e.iterated
    tol = pt.step_tolerance(theta, got_theta, e, scale)
    worst = float(np.max(np.abs(got_theta - want) / tol))
    print(f"{what}: step max |err|/tol = {worst:.3f}", flush=True)
    assert worst <= 1.0, (what, worst)
    return e


# -- the polar factor -----------------------------------------------------------

@pytest.mark.parametrize("m,n,kappa", [(256, 64, 1), (256, 64, 10), (64, 256, 10),
                                       (200, 200, 100), (300, 130, 1e3), (130, 300, 1e3),
                                       (1000, 257, 100), (129, 129, 1e4), (33, 517, 10)])
def test_polar_factor_constructed(m, n, kappa):
    rng = np.random.default_rng(int(m * 31 + n + kappa))
    a = constructed(rng, m, n, kappa)
    a64 = a.astype(np.float64)
    want = opolar.polar_factor(a64)
    out = torch.empty((m, n), device=DEV)
    a_d = gpu(a)
    dl.dl_polar_factor(out, a_d, m, n, workspace(m, n))
    got = host(out)
    assert_factor_elementwise(got, a64, f"polar {m}x{n} kappa={kappa:g}")
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    bound = polar_bound(a64)
    est = polar_estimate(a64)
    print(f"polar {m}x{n} kappa={kappa:g}: rel_F={rel:.3e} bound={bound:.3e} estimate={est:.3e} "
          f"max={np.max(np.abs(got - want)):.3e}", flush=True)
    assert rel <= bound
    assert rel <= est
    # the input is not modified
    assert np.array_equal(host(a_d), a64)


def test_polar_factor_in_place_and_vectors():
    rng = np.random.default_rng(11)
    for m, n in ((1, 300), (300, 1), (1, 1), (2, 2)):
        a = rng.standard_normal((m, n)).astype(np.float32)
        a_d = gpu(a)
        dl.dl_polar_factor(a_d, a_d, m, n, workspace(m, n))       # out == update
        want = opolar.polar_factor(a.astype(np.float64))
        got = host(a_d)
        assert_factor_elementwise(got, a.astype(np.float64), f"in place {m}x{n}")
        assert np.linalg.norm(got - want) <= polar_bound(a.astype(np.float64)) * np.linalg.norm(want)


def test_polar_factor_of_zero_is_zero():
    z = torch.zeros((40, 24), device=DEV)
    out = torch.full((40, 24), 5.0, device=DEV)
    dl.dl_polar_factor(out, z, 40, 24, workspace(40, 24))
    assert not np.any(host(out))


@pytest.mark.parametrize("m,n,rank", [(300, 120, 80), (120, 300, 80), (256, 256, 1)])
def test_polar_factor_rank_deficient(m, n, rank):
    """A rank-deficient update (the degenerate case): U V^T is unique only on
    the row space of A, where it maps V_r to U_r; on the null space any
    completion is a polar factor.  The unique part is checked against the SVD
    factors of A; for the rest, that the result is still a valid contraction
    (no singular value above 1 beyond rounding: the iteration maps [0, 1]
    into [0, 1]).  fp32 rounding gives the null space singular values of
    order u, which the iteration amplifies, so it is not left at zero."""
    rng = np.random.default_rng(m + 3 * n + rank)
    u, _ = np.linalg.qr(rng.standard_normal((m, rank)))
    v, _ = np.linalg.qr(rng.standard_normal((n, rank)))
    sv = np.logspace(0, -1, rank)
    a = ((u * sv) @ v.T).astype(np.float32)
    a64 = a.astype(np.float64)
    uu, ss, vvt = np.linalg.svd(a64, full_matrices=False)
    ur, vr = uu[:, :rank], vvt[:rank].T
    out = torch.empty((m, n), device=DEV)
    dl.dl_polar_factor(out, gpu(a), m, n, workspace(m, n))
    got = host(out)
    est = estimate_from(ss[0] / ss[rank - 1], rank)
    rel = np.linalg.norm(got @ vr - ur) / np.linalg.norm(ur)
    s_got = np.linalg.svd(got, compute_uv=False)
    null = np.linalg.norm(got @ vvt[rank:].T) if vvt.shape[0] > rank else 0.0
    print(f"rank-deficient {m}x{n} rank {rank}: unique part rel {rel:.2e} (estimate {est:.2e}), "
          f"sigma_max {s_got[0]:.6f}, null-space part {null:.2e}", flush=True)
    assert rel <= est, (rel, est)
    assert s_got[0] <= 1 + 1e-4


def test_polar_factor_scale_invariant_and_deterministic():
    rng = np.random.default_rng(12)
    a = constructed(rng, 300, 100, 50)
    ws = workspace(300, 100)
    outs = []
    for s in (1.0, 1.0, 8.0):      # powers of two: the scaled input is exact
        o = torch.empty((300, 100), device=DEV)
        dl.dl_polar_factor(o, gpu(a * np.float32(s)), 300, 100, ws)
        outs.append(host(o))
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0], outs[2])
    assert_factor_elementwise(outs[0], a.astype(np.float64), "scale-invariant 300x100")


def test_polar_steps_schedule():
    """Fewer cubic steps leave the factor less orthogonal; one quintic step
    alone is far from it (the step counts reach the kernel)."""
    rng = np.random.default_rng(13)
    a = constructed(rng, 256, 128, 100)
    want = opolar.polar_factor(a.astype(np.float64))
    ws = workspace(256, 128)
    errs = []
    for q, c in ((1, 0), (12, 0), (12, 6), (3, 2)):
        o = torch.empty((256, 128), device=DEV)
        dl.dl_polar_factor(o, gpu(a), 256, 128, ws, quintic_steps=q, cubic_steps=c)
        got = host(o)
        # each schedule's result, element by element, is that schedule's
        # exact-arithmetic iterate: the step counts reach the kernel
        assert_factor_elementwise(got, a.astype(np.float64), f"schedule {q}+{c}", q, c)
        errs.append(np.linalg.norm(got - want))
    errs = errs[:3]
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] <= polar_bound(a.astype(np.float64)) * np.linalg.norm(want)


# -- the outer step --------------------------------------------------------------

@pytest.mark.parametrize("m,n,scale", [(192, 64, 0.02), (64, 192, 1.0), (257, 255, 0.02)])
def test_outer_orthogonal_step(m, n, scale):
    """theta - scale * P from the last product's epilogue.  At scale 1 the
    rounding of theta' is no larger than P's own, so every element of P is
    resolved to its tolerance."""
    seed = 900 + m
    theta = synth.global0(seed, m * n, device=DEV)
    avg = synth.worker_checkpoint(seed, 0, 0, theta)
    th_h, avg_h = host(theta), host(avg)
    want = opolar.outer_orthogonal_step(th_h.reshape(m, n), avg_h.reshape(m, n), scale).reshape(-1)
    upd = (th_h - avg_h).reshape(m, n)
    dl.dl_outer_orthogonal_step(theta, avg, m, n, scale, workspace(m, n))
    got = host(theta)
    assert_step_elementwise(got.reshape(m, n), th_h.reshape(m, n), upd, scale, f"step {m}x{n}")
    p_err = polar_bound(upd) * math.sqrt(min(m, n))            # ||P||_F = sqrt(r)
    err = np.linalg.norm(got - want)
    print(f"step {m}x{n}: err_F={err:.3e} bound={scale * p_err:.3e}", flush=True)
    assert err <= scale * p_err + 2 * U32 * np.linalg.norm(want)
    assert np.array_equal(host(avg), avg_h)


@pytest.mark.parametrize("m,n,batch", [(192, 64, 3), (64, 192, 2), (257, 255, 4), (300, 130, 5)])
def test_outer_orthogonal_step_batch(m, n, batch):
    """A batch of equally shaped matrices, each against the oracle within
    the same bounds; the inputs are untouched; a batch of one is the
    one-matrix call bit for bit."""
    dev = DEV
    thetas, avgs = [], []
    for b in range(batch):
        th = synth.global0(700 + b, m * n, device=dev)
        thetas.append(th)
        avgs.append(synth.worker_checkpoint(700 + b, 0, 0, th))
    th_h = [host(t).reshape(m, n) for t in thetas]
    av_h = [host(a).reshape(m, n) for a in avgs]
    scale = 0.02
    ws = torch.empty(dl.dl_polar_workspace_bytes_batch(m, n, batch) // 4 + 1, device=dev)
    dl.dl_outer_orthogonal_step_batch(thetas, avgs, m, n, scale, ws)
    for b in range(batch):
        want = opolar.outer_orthogonal_step(th_h[b], av_h[b], scale)
        upd = th_h[b] - av_h[b]
        got = host(thetas[b]).reshape(m, n)
        assert_step_elementwise(got, th_h[b], upd, scale, f"batch {m}x{n} [{b}]")
        err = np.linalg.norm(got - want)
        bound = scale * polar_bound(upd) * math.sqrt(min(m, n)) + 2 * U32 * np.linalg.norm(want)
        est = scale * polar_estimate(upd) * math.sqrt(min(m, n)) + 2 * U32 * np.linalg.norm(want)
        print(f"batch {m}x{n} [{b}]: err_F={err:.3e} estimate={est:.3e}", flush=True)
        assert err <= bound and err <= est
        assert np.array_equal(host(avgs[b]).reshape(m, n), av_h[b])
    t1 = synth.global0(700, m * n, device=dev)
    t2 = t1.clone()
    a1 = synth.worker_checkpoint(700, 0, 0, t1)
    dl.dl_outer_orthogonal_step_batch([t1], [a1], m, n, scale, ws)
    dl.dl_outer_orthogonal_step(t2, a1, m, n, scale, ws)
    assert np.array_equal(host(t1), host(t2))


def test_outer_orthogonal_step_largest_batch():
    """The largest batch the library takes (64 matrices: every per-matrix
    pointer slot of the batched passes in use), and one more is refused."""
    m, n, batch = 256, 128, dl.DL_MAX_BATCH
    thetas = [synth.global0(1600 + b, m * n, device=DEV) for b in range(batch)]
    avgs = [synth.worker_checkpoint(1600 + b, 0, 0, t) for b, t in enumerate(thetas)]
    check = (0, 31, batch - 1)
    th_h = {b: host(thetas[b]).reshape(m, n) for b in check}
    av_h = {b: host(avgs[b]).reshape(m, n) for b in check}
    scale = 0.02
    ws = torch.empty(dl.dl_polar_workspace_bytes_batch(m, n, batch) // 4 + 1, device=DEV)
    dl.dl_outer_orthogonal_step_batch(thetas, avgs, m, n, scale, ws)
    for b in check:
        want = opolar.outer_orthogonal_step(th_h[b], av_h[b], scale)
        upd = th_h[b] - av_h[b]
        got = host(thetas[b]).reshape(m, n)
        assert_step_elementwise(got, th_h[b], upd, scale, f"largest batch [{b}]")
        err = np.linalg.norm(got - want)
        est = scale * polar_estimate(upd) * math.sqrt(n) + 2 * U32 * np.linalg.norm(want)
        assert err <= est, (b, err, est)
    extra = synth.global0(1700, m * n, device=DEV)
    with pytest.raises(dl.DLError) as ei:
        dl.dl_outer_orthogonal_step_batch(thetas + [extra], avgs + [extra.clone()], m, n, scale,
                                          ws)
    assert ei.value.status == dl.DL_E_INVAL


def test_outer_orthogonal_step_batch_unaligned_views():
    """Matrices that start one element past a 16-byte boundary (views into
    a flat buffer): the elementwise passes take their element-by-element
    path, and every matrix still meets the oracle's bounds."""
    m, n, batch = 192, 64, 3
    bufs_t = [synth.global0(1500 + b, m * n + 1, device=DEV) for b in range(batch)]
    bufs_a = [synth.worker_checkpoint(1500 + b, 0, 0, t) for b, t in enumerate(bufs_t)]
    thetas = [t[1:] for t in bufs_t]
    avgs = [a[1:] for a in bufs_a]
    assert all(t.data_ptr() % 16 == 4 for t in thetas)
    th_h = [host(t).reshape(m, n) for t in thetas]
    av_h = [host(a).reshape(m, n) for a in avgs]
    scale = 0.02
    ws = torch.empty(dl.dl_polar_workspace_bytes_batch(m, n, batch) // 4 + 1, device=DEV)
    dl.dl_outer_orthogonal_step_batch(thetas, avgs, m, n, scale, ws)
    for b in range(batch):
        want = opolar.outer_orthogonal_step(th_h[b], av_h[b], scale)
        upd = th_h[b] - av_h[b]
        got = host(thetas[b]).reshape(m, n)
        assert_step_elementwise(got, th_h[b], upd, scale, f"unaligned [{b}]")
        err = np.linalg.norm(got - want)
        est = scale * polar_estimate(upd) * math.sqrt(min(m, n)) + 2 * U32 * np.linalg.norm(want)
        assert err <= est, (b, err, est)
        assert float(bufs_t[b][0]) == float(synth.global0(1500 + b, 1, device=DEV)[0])


@pytest.mark.parametrize("m,n", [(2560, 1536), (1536, 2560)], ids=["tall", "wide"])
def test_outer_orthogonal_step_batch_large_tiles(m, n):
    """A batch of 12 on the large-tile path for every product (the Gram
    matrix and its square with upper tiles only, the next iterate in both
    forms, rounds not a whole multiple of the CUs): the first and the last
    matrix of the batch against the oracle."""
    batch, r, big = 12, min(m, n), max(m, n)
    for shape in ((r, r, big, True), (r, r, r, True), (m, n, r, False)):
        wsb = dl.dl_matmul_workspace_bytes_batch(*shape, batch)
        assert dl.dl_matmul_large_tiles(*shape, batch, wsb), shape
    thetas = [synth.global0(1400 + b, m * n, device=DEV) for b in range(batch)]
    avgs = [synth.worker_checkpoint(1400 + b, 0, 0, t) for b, t in enumerate(thetas)]
    check = (0, batch - 1)
    th_h = {b: host(thetas[b]).reshape(m, n) for b in check}
    av_h = {b: host(avgs[b]).reshape(m, n) for b in check}
    scale = 1.0
    ws = torch.empty(dl.dl_polar_workspace_bytes_batch(m, n, batch) // 4 + 1, device=DEV)
    dl.dl_outer_orthogonal_step_batch(thetas, avgs, m, n, scale, ws)
    for b in check:
        want = opolar.outer_orthogonal_step(th_h[b], av_h[b], scale)
        upd = th_h[b] - av_h[b]
        got = host(thetas[b]).reshape(m, n)
        assert_step_elementwise(got, th_h[b], upd, scale, f"large-tile batch {m}x{n} [{b}]")
        err = np.linalg.norm(got - want)
        est = scale * polar_estimate(upd) * math.sqrt(r) + 2 * U32 * np.linalg.norm(want)
        print(f"large-tile batch {m}x{n} [{b}]: err_F={err:.3e} estimate={est:.3e}", flush=True)
        assert err <= est


def test_outer_orthogonal_step_batch_full_size():
    """Four 2048 x 2048 attention updates in one batch against the SVD (the
    batch's 4 x 64 tiles of 256 x 256 send its next-iterate products to the
    large-tile kernel)."""
    rows = cols = 2048
    batch = 4
    thetas = [synth.global0(960 + b, rows * cols, device=DEV) for b in range(batch)]
    avgs = [synth.worker_checkpoint(960 + b, 0, 0, t) for b, t in enumerate(thetas)]
    th_h = [host(t).reshape(rows, cols) for t in thetas]
    av_h = [host(a).reshape(rows, cols) for a in avgs]
    scale = 1.0           # theta' rounds no coarser than P: P's elements are resolved
    ws = torch.empty(dl.dl_polar_workspace_bytes_batch(rows, cols, batch) // 4 + 1, device=DEV)
    dl.dl_outer_orthogonal_step_batch(thetas, avgs, rows, cols, scale, ws)
    for b in range(batch):
        upd = th_h[b] - av_h[b]
        got = host(thetas[b]).reshape(rows, cols)
        e = assert_step_elementwise(got, th_h[b], upd, scale, f"batch full 2048x2048 [{b}]")
        p_got = (th_h[b] - got) / scale
        want = e.svd
        rel = np.linalg.norm(p_got - want) / np.linalg.norm(want)
        # theta - s P loses |theta| u per element: bound that on top
        extra = 2 * U32 * np.linalg.norm(th_h[b]) / scale / np.linalg.norm(want)
        est = polar_estimate(upd) + extra
        print(f"batch full 2048x2048 [{b}]: rel_F={rel:.3e} estimate={est:.3e}", flush=True)
        assert rel <= est


@pytest.mark.parametrize("batch,streams", [(8, 1), (None, 1), (None, 2), (4, 3)])
def test_orthogonal_step_over_pythia14m_layout(batch, streams):
    """The whole-model step over the Pythia-14M layout (26 matrices in five
    shapes: the two 50304 x 128 embeddings, QKV 384 x 128, dense 128 x 128,
    MLP 512 x 128 and 128 x 512; equally shaped ones batched by 8, 4 or all
    together, on one stream or spread over several): every matrix against the
    oracle's step, and every parameter outside the matrices (the norms and
    biases) untouched."""
    from checkpoint_averaging_amd.orthogonalize import OrthogonalStep
    layout = synth.PYTHIA_14M
    n = layout.n_params
    theta = synth.global0(1201, n, device=DEV)
    avg = synth.worker_checkpoint(1201, 0, 0, theta)
    th_h, av_h = host(theta), host(avg)
    step = OrthogonalStep(layout, DEV, batch=batch, streams=streams)
    assert len(step.matrices) == 26
    scale = 2e-3
    step.run(theta, avg, scale)
    got = host(theta)
    touched = np.zeros(n, bool)
    for m in step.matrices:
        sl = slice(m.offset, m.offset + m.rows * m.cols)
        touched[sl] = True
        t, a = th_h[sl].reshape(m.rows, m.cols), av_h[sl].reshape(m.rows, m.cols)
        want = opolar.outer_orthogonal_step(t, a, scale)
        upd = t - a
        r = min(m.rows, m.cols)
        assert_step_elementwise(got[sl].reshape(m.rows, m.cols), t, upd, scale, m.name)
        err = np.linalg.norm(got[sl].reshape(m.rows, m.cols) - want)
        est = scale * polar_estimate(upd) * math.sqrt(r) + 2 * U32 * np.linalg.norm(want)
        assert err <= est, (m.name, err, est)
    assert np.array_equal(got[~touched], th_h[~touched])


# -- full-size shapes of DiffuRefill-1B's weight matrices -----------------------

@pytest.mark.parametrize("rows,cols", [(2048, 2048), (5632, 2048), (2048, 5632)],
                         ids=["attn_2048x2048", "ffn_up_5632x2048", "ffn_down_2048x5632"])
def test_polar_full_size_against_svd(rows, cols):
    seed = 950 + rows // 64
    theta = synth.global0(seed, rows * cols, device=DEV)
    avg = synth.worker_checkpoint(seed, 0, 0, theta)
    upd = host(theta) - host(avg)                     # fp64 difference of the fp32 inputs
    a32 = torch.sub(theta, avg)                       # the kernel forms it in fp32 as well
    out = torch.empty(rows * cols, device=DEV)
    dl.dl_polar_factor(out, a32, rows, cols, workspace(rows, cols))
    got = host(out).reshape(rows, cols)
    e = assert_factor_elementwise(got, upd.reshape(rows, cols), f"full {rows}x{cols}")
    want = e.svd
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    bound = polar_bound(upd.reshape(rows, cols))
    est = polar_estimate(upd.reshape(rows, cols))
    print(f"full {rows}x{cols}: rel_F={rel:.3e} bound={bound:.3e} estimate={est:.3e}", flush=True)
    assert rel <= bound
    assert rel <= est


def test_polar_full_size_embedding_rows():
    """The 73760 x 2048 embedding: every element of sampled rows against the
    oracle (through the eigendecomposition of A^T A), and orthonormal columns
    over the whole factor."""
    rows, cols = 73760, 2048
    seed = 977
    theta = synth.global0(seed, rows * cols, device=DEV)
    avg = synth.worker_checkpoint(seed, 0, 0, theta)
    upd = (host(theta) - host(avg)).reshape(rows, cols)
    out = torch.empty(rows * cols, device=DEV)
    dl.dl_polar_factor(out, torch.sub(theta, avg), rows, cols, workspace(rows, cols))
    got = host(out).reshape(rows, cols)
    pick = np.random.default_rng(5).choice(rows, 64, replace=False)
    pick = np.concatenate([[0, rows - 1], pick])
    e = pt.expected_rows(upd, pick)
    z = pt.report(got[pick], e, "embedding rows")
    assert z <= pt.Z
    want = e.svd
    kappa_f = np.linalg.norm(upd) / e.sigma[-1]
    bound = C_POLAR * math.sqrt(cols) * U32 * kappa_f
    est = estimate_from(e.sigma[0] / e.sigma[-1], cols)
    rel = np.linalg.norm(got[pick] - want) / np.linalg.norm(want)
    print(f"embedding rows: rel_F={rel:.3e} bound={bound:.3e} estimate={est:.3e}", flush=True)
    assert rel <= bound
    assert rel <= est
    gram = got.T @ got
    orth = np.max(np.abs(gram - np.eye(cols)))
    print(f"embedding orthonormality: {orth:.3e}", flush=True)
    assert orth <= 2 * bound


def test_polar_factor_unconverged_directions():
    """Directions with s / ||A||_F below about 1.4e-7 are not brought to 1 by
    12 quintic and 6 cubic steps: the iteration maps such an s to
    phi(s / ||A||_F) < 1, the oracle's iterated factor.  A 2048 x 1024
    update with a flat spectrum (so ||A||_F = 32 s_max and such directions
    are still above fp32 noise) and six small singular values at 1e-8 ..
    2e-7 ||A||_F: every element within the per-element tolerance about the
    iterated factor, the factor's gain along the small directions short of 1
    where phi is and at 1 where phi is, and no direction above 1."""
    rows, cols = 2048, 1024
    rng = np.random.default_rng(31)
    xs = np.array([2e-7, 1e-7, 5e-8, 3e-8, 2e-8, 1e-8])
    k = xs.size
    f_norm = math.sqrt(cols - k)
    sv = np.concatenate([np.ones(cols - k), xs * f_norm])
    a = ((orthonormal(rng, rows, cols) * sv) @ orthonormal(rng, cols, cols).T).astype(np.float32)
    a64 = a.astype(np.float64)
    out = torch.empty((rows, cols), device=DEV)
    dl.dl_polar_factor(out, gpu(a), rows, cols, workspace(rows, cols))
    got = host(out)
    e = assert_factor_elementwise(got, a64, "unconverged directions 2048x1024")
    _, s, vt = np.linalg.svd(a64, full_matrices=False)
    x = s[-k:] / np.linalg.norm(a64)
    gain = np.linalg.norm(got @ vt[-k:].T, axis=0)
    phi = opolar.iteration_map(x)
    for xi, g, p in zip(x, gain, phi):
        print(f"  s/||A||_F = {xi:.2e}: phi = {p:.6f}, gain of the fp32 factor = {g:.6f}", flush=True)
    assert np.all(gain[x <= 2.5e-8] <= 0.9)
    assert np.all(gain[x >= 0.9e-7] >= 0.999)
    assert np.linalg.svd(got, compute_uv=False)[0] <= 1 + 1e-5
    moved = np.max(np.abs(e.iterated - e.svd))
    print(f"  largest element gap between U phi V^T and U V^T: {moved:.3e}", flush=True)


def test_orthogonal_step_over_diffurefill1b_layout_sampled():
    """The benchmark's configuration at full size: the whole-model step over
    the DiffuRefill-1B layout (127 matrices; each shape's matrices together,
    split evenly into launches of at most 64, so the products run on the
    large-tile kernel with the last round's tiles cut along K), then sampled
    matrices against the oracle: the first and the last matrix of each
    batch (the last one holds the tiles cut along K) and sampled rows of the
    embedding; every parameter outside the matrices untouched."""
    from checkpoint_averaging_amd.orthogonalize import OrthogonalStep
    layout = synth.DIFFUREFILL_1B
    n = layout.n_params
    theta = synth.global0(1311, n, device=DEV)
    avg = synth.worker_checkpoint(1311, 0, 0, theta)
    step = OrthogonalStep(layout, DEV)
    mats = step.matrices
    assert len(mats) == 127
    # the first and the last matrix of every batch
    picks = [g[i] for g in step.groups for i in sorted({0, len(g) - 1})]
    assert len(picks) == 9
    before = {m.name: (host(theta[m.offset:m.offset + m.rows * m.cols]),
                       host(avg[m.offset:m.offset + m.rows * m.cols])) for m in picks}
    outside = torch.ones(n, dtype=torch.bool, device=DEV)
    for m in mats:
        outside[m.offset:m.offset + m.rows * m.cols] = False
    rest = theta[outside].clone()
    scale = 1.0           # theta' rounds no coarser than P: P's elements are resolved
    step.run(theta, avg, scale)
    torch.cuda.synchronize()
    assert torch.equal(theta[outside], rest)
    for m in picks:
        t, a = (x.reshape(m.rows, m.cols) for x in before[m.name])
        got = host(theta[m.offset:m.offset + m.rows * m.cols]).reshape(m.rows, m.cols)
        upd = t - a
        if m.rows > 8 * m.cols:   # the embedding: sampled rows, Gram eigendecomposition
            pick = np.random.default_rng(9).choice(m.rows, 64, replace=False)
            pick = np.concatenate([[0, m.rows - 1], pick])
            e = pt.expected_rows(upd, pick)
            est = estimate_from(e.sigma[0] / e.sigma[-1], m.cols)
            t, got = t[pick], got[pick]
        else:
            e = pt.expected(upd)
            est = estimate_from(e.sigma[0] / e.sigma[-1], min(m.rows, m.cols))
        assert_step_elementwise(got, t, None, scale, f"1B step {m.name}", e=e)
        want = e.svd
        p_got = (t - got) / scale
        rel = np.linalg.norm(p_got - want) / np.linalg.norm(want)
        # theta - s P loses |theta| u per element: bound that on top
        extra = 2 * U32 * np.linalg.norm(t) / scale / np.linalg.norm(want)
        print(f"1B step {m.name} {m.rows}x{m.cols}: rel_F={rel:.3e} "
              f"estimate={est:.3e} + {extra:.3e}", flush=True)
        assert rel <= est + extra, m.name
