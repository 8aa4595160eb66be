"""GPU parity of the side averages (uniform average of globals, averages of
the last k snapshots) and of the worker-side keep-local-drift adoption
against the CPU oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from checkpoint_averaging_amd import dlmerge as dl
from checkpoint_averaging_amd import synth
from tests import merge_cases as mc

pytestmark = pytest.mark.gpu


def globals_series(n, count, seed=1006):
    """A series of nearby globals from the seeded generator (stand-ins for
    the globals a run commits one after another)."""
    th0 = synth.global0(seed, n, device="cuda")
    return [synth.worker_checkpoint(seed, r, 0, th0) for r in range(count)]


@pytest.mark.parametrize("n", [1, 5, 4096 * 3 + 2, 1 << 20])
def test_swa_matches_oracle(n):
    gs = globals_series(n, 13)
    s = torch.full((n,), float("nan"), device="cuda")
    for k, g in enumerate(gs):
        dl.dl_swa_fold(s, g, k)
    out = torch.empty(n, device="cuda")
    dl.dl_swa_average(out, s, len(gs))
    dl.dl_swa_average(s, s, len(gs))                     # in place
    torch.cuda.synchronize()
    want = oracle.swa_average([mc.to_np(g) for g in gs])
    assert mc.bits_equal(mc.to_np(out), want), mc.first_mismatch(mc.to_np(out), want)
    assert mc.bits_equal(mc.to_np(s), want)


def test_swa_of_130_globals():
    n = 300_007
    gs = globals_series(n, 130)
    s = torch.empty(n, device="cuda")
    for k, g in enumerate(gs):
        dl.dl_swa_fold(s, g, k)
    dl.dl_swa_average(s, s, 130)
    torch.cuda.synchronize()
    want = oracle.swa_average([mc.to_np(g) for g in gs])
    assert mc.bits_equal(mc.to_np(s), want), mc.first_mismatch(mc.to_np(s), want)


@pytest.mark.parametrize("k", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("n", [3, 4096 * 5 + 3, 1 << 20])
def test_snapshot_average_matches_oracle(k, n):
    snaps = globals_series(n, k)
    out = torch.empty(n, device="cuda")
    dl.dl_snapshot_average(out, snaps)
    torch.cuda.synchronize()
    want = oracle.snapshot_average([mc.to_np(x) for x in snaps])
    assert mc.bits_equal(mc.to_np(out), want), mc.first_mismatch(mc.to_np(out), want)


def test_snapshot_average_scalar_path_and_order():
    """A snapshot at a 4-byte offset runs the scalar path; the order of the
    snapshots is the summation order (reversing it changes some bits)."""
    n = 100_003
    snaps = globals_series(n, 5)
    shifted = torch.empty(n + 1, device="cuda")
    shifted[1:] = snaps[2]
    ptrs = [snaps[0], snaps[1], shifted.data_ptr() + 4, snaps[3], snaps[4]]
    out = torch.empty(n, device="cuda")
    dl.dl_snapshot_average(out, ptrs)
    rev = torch.empty(n, device="cuda")
    dl.dl_snapshot_average(rev, list(reversed(snaps)))
    torch.cuda.synchronize()
    host = [mc.to_np(x) for x in snaps]
    want = oracle.snapshot_average(host)
    assert mc.bits_equal(mc.to_np(out), want), mc.first_mismatch(mc.to_np(out), want)
    want_rev = oracle.snapshot_average(host[::-1])
    assert mc.bits_equal(mc.to_np(rev), want_rev)
    assert not mc.bits_equal(want, want_rev)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 7, 4096 * 3 + 1, 1 << 20])
def test_adopt_keep_drift_matches_oracle(n, dtype):
    th0 = synth.global0(1007, n, device="cuda")
    theta = synth.worker_checkpoint(1007, 5, 0, th0)                 # the worker's weights
    pushed = synth.worker_checkpoint(1007, 4, 0, th0, dtype=dtype)   # what it pushed
    g = synth.worker_checkpoint(1007, 6, 1, th0)                     # the new global
    want = mc.to_np(theta)
    oracle.adopt_keep_drift(want, mc.to_np(g), mc.to_np(pushed))
    dl.dl_adopt_keep_drift(theta, g, pushed)
    torch.cuda.synchronize()
    assert mc.bits_equal(mc.to_np(theta), want), mc.first_mismatch(mc.to_np(theta), want)


def test_side_averages_and_adoption_full_size_sampled():
    """At the 1.08B size the benchmark times (the streaming kernels' non-
    temporal paths): the uniform average of 5 globals folded one by one, the
    average of the same 5 as snapshots, and the keep-local-drift adoption,
    on sampled windows against the oracle run on inputs regenerated on the
    CPU for those windows only."""
    n = synth.DIFFUREFILL_1B.n_params
    seed, count, win = 1016, 5, 4096
    th0 = synth.global0(seed, n, device="cuda")
    gs = [synth.worker_checkpoint(seed, r, 0, th0) for r in range(count)]
    s = torch.empty(n, device="cuda")
    for k, g in enumerate(gs):
        dl.dl_swa_fold(s, g, k)
    swa = torch.empty(n, device="cuda")
    dl.dl_swa_average(swa, s, count)
    del s
    snap = torch.empty(n, device="cuda")
    dl.dl_snapshot_average(snap, gs)
    theta = th0.clone()                       # the worker's weights, it pushed gs[0]
    dl.dl_adopt_keep_drift(theta, gs[1], gs[0])
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    starts = sorted({0, n - win, *(int(x) for x in rng.integers(0, n - win, size=12))})
    for st in starts:
        t0 = synth.global0(seed, win, start=st)
        g_w = [mc.to_np(synth.worker_checkpoint(seed, r, 0, t0, start=st)) for r in range(count)]
        want_swa = oracle.swa_average(g_w)
        want_snap = oracle.snapshot_average(g_w)
        want_th = mc.to_np(t0)
        oracle.adopt_keep_drift(want_th, g_w[1], g_w[0])
        for got, want, what in ((swa, want_swa, "swa"), (snap, want_snap, "snapshot"),
                                (theta, want_th, "adopt")):
            g = mc.to_np(got[st:st + win])
            assert mc.bits_equal(g, want), (what, st, mc.first_mismatch(g, want))
    del gs, swa, snap, theta, th0
    torch.cuda.empty_cache()
