"""GPU parity of the several-arrival calls (dl_fold_checkpoints and the
folding-and-closing forms) against the CPU oracle, which folds one arrival at
a time in arrival order: bit for bit, on the seeded inputs.

Cases: every arrival of a fragment in one call, calls of 2 or 3 arrivals
after a one-arrival fold, more arrivals than one pass takes (the library
splits them into passes of 8), exactly the quorum and a lone arrival, edge
sizes, unaligned fragments (scalar path), fp32 and bf16 checkpoints, and a
checkpoint buffer passed for two workers."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from checkpoint_averaging_amd import dlmerge as dl
from checkpoint_averaging_amd import synth
from tests import merge_cases as mc

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rounds(w, n_rounds=2, **kw):
    st = mc.init_state(w)
    for r in range(n_rounds):
        say(f"[several] {w.key} n={w.n_params} workers={w.workers} frags={w.frag_offsets}"
            f" round {r} {kw}")
        res = mc.run_round(w, st, r, **kw)
        mc.assert_round_equal(res, f"{w.key} n={w.n_params} round {r} {kw}")


CASES = [
    ("pythia14m_mean", (1 << 20) + 37, None),
    ("pythia14m_frag_nesterov", 777_777, [0, 123_457, 300_001, 300_002, 777_777]),  # unaligned
    ("diffurefill1b_mean_ema", 3 * 4096 * 4 + 3, None),
    ("diffurefill1b_bf16_mean_ema", (1 << 20) + 5, None),
    ("diffurefill1b_frag_nesterov_ema", (1 << 20) + 7, [0, 140_000, 428_000, 716_000, (1 << 20) + 7]),
    ("diffurefill1b_mean_ema", 300_001, [0, 100_001, 300_001]),                   # unaligned
    ("diffurefill1b_bf16_mean_ema", 200_003, [0, 66_667, 200_003]),               # unaligned
]
SCHEDULES = [
    dict(batch=8),                      # all arrivals of a fragment in one call
    dict(batch=2, single_first=1),      # a one-arrival fold, then calls of 2
    dict(batch=3),                      # a call of 3, then the rest
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate_close", "fused_close"])
@pytest.mark.parametrize("sched", SCHEDULES, ids=["all", "one_then_pairs", "threes"])
@pytest.mark.parametrize("key,n,offs", CASES, ids=[f"{k}-{n}" for k, n, _ in CASES])
def test_several_arrivals_parity(key, n, offs, sched, fused):
    rounds(synth.scaled(W[key], n, offs), fused_last=fused, **sched)


@pytest.mark.parametrize("fused", [False, True], ids=["separate_close", "fused_close"])
@pytest.mark.parametrize("key", ["diffurefill1b_mean_ema", "diffurefill1b_bf16_mean_ema",
                                 "diffurefill1b_frag_nesterov_ema"])
def test_more_arrivals_than_one_pass(key, fused):
    """19 workers in one call: three passes of 8, 8 and 3 arrivals, the last
    closing when fused; and calls of 9 after one single fold."""
    w = dataclasses.replace(synth.scaled(W[key], 200_003, [0, 100_000, 200_003]), workers=19)
    rounds(w, fused_last=fused, batch=19)
    rounds(w, n_rounds=1, fused_last=fused, batch=9, single_first=1)


@pytest.mark.parametrize("key", ["pythia14m_frag_nesterov", "diffurefill1b_frag_nesterov_ema"])
def test_several_arrivals_exactly_quorum(key):
    w = synth.scaled(W[key], 300_017, [0, 80_000, 160_000, 240_000, 300_017])
    rounds(w, exactly_quorum=True, fused_last=True, batch=8)
    rounds(w, n_rounds=1, exactly_quorum=True, fused_last=False, batch=2)


def test_lone_arrival_closes():
    """Quorum 1: one arrival passed to the closing several-arrival call is
    both the first fold and the close."""
    for key in ("diffurefill1b_mean_ema", "diffurefill1b_frag_nesterov_ema"):
        w = dataclasses.replace(synth.scaled(W[key], 60_001, [0, 30_000, 60_001]), quorum=1)
        st = mc.init_state(w)
        for r, orders in enumerate(([[3], [1, 4]], [[0, 2, 1], [2]])):
            res = mc.run_round(w, st, r, orders=orders, fused_last=True, batch=8)
            mc.assert_round_equal(res, f"{key} lone arrival, round {r}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 9, 1023, 1025, 4095, 4097, 16385])
def test_several_arrivals_edge_sizes(n):
    for key in ("diffurefill1b_bf16_mean_ema", "diffurefill1b_frag_nesterov_ema"):
        w = synth.scaled(W[key], n, [0, n])
        rounds(w, fused_last=True, batch=8)
        rounds(w, n_rounds=1, fused_last=False, batch=3)


def test_one_buffer_for_two_workers():
    """Checkpoints are only read, so two arrivals may name the same buffer;
    the oracle folds the same values twice."""
    w = synth.scaled(W["diffurefill1b_frag_nesterov_ema"], 100_003, [0, 100_003])
    theta0 = synth.global0(w.seed, w.n_params)
    ck = synth.worker_checkpoint(w.seed, 0, 0, theta0.cuda())
    g_theta, g_m = theta0.cuda(), torch.zeros(w.n_params, device="cuda")
    acc = torch.empty(w.n_params, device="cuda")
    r = dl.dl_round_begin(9, dl.DL_DELTA_NESTEROV, w.n_params, [0, w.n_params], 2, 4, acc)
    try:
        dl.dl_fold_checkpoints_and_outer_nesterov(r, 0, [1, 3], 9, [ck, ck], [250_000, 199_999],
                                                  g_theta, g_m, w.lr, w.mu)
    finally:
        dl.dl_round_end(r)
    theta, m = theta0.numpy().copy(), np.zeros(w.n_params, dtype=np.float32)
    c = mc.to_np(ck)
    oracle.load().nesterov_fragment_round(theta, m, [c, c], [250_000, 199_999], w.lr, w.mu,
                                          None, w.beta)
    torch.cuda.synchronize()
    for name, g, o in (("theta", mc.to_np(g_theta), theta), ("m", mc.to_np(g_m), m)):
        assert mc.bits_equal(g, o), f"{name}: {mc.first_mismatch(g, o)}"


@pytest.mark.parametrize("key", ["diffurefill1b_frag_nesterov_ema", "diffurefill1b_mean_ema",
                                 "diffurefill1b_bf16_mean_ema"])
def test_several_arrivals_at_nontemporal_size(key):
    """A fragment of 2^24 + 3 elements (the non-temporal kernels, both pass
    directions, a ragged tail): several-arrival rounds against the oracle's
    one-at-a-time rounds, with the closing pass both the fragment's first
    (all arrivals in one call) and after earlier folds."""
    w = synth.scaled(W[key], (1 << 24) + 7, [0, 4, (1 << 24) + 7])
    rounds(w, fused_last=True, batch=8)
    rounds(w, n_rounds=1, fused_last=True, batch=2, single_first=1)
    rounds(w, n_rounds=1, fused_last=False, batch=2, single_first=1)


@pytest.mark.parametrize("fused", [False, True], ids=["separate_close", "fused_close"])
@pytest.mark.parametrize("n", [4096 + 3, (1 << 24) + 3], ids=["cached", "non_temporal"])
def test_several_arrivals_special_values(n, fused):
    """NaN, infinities, subnormals and -0 in the checkpoints and the global
    go through the several-arrival passes as through the oracle's one-arrival
    folds (IEEE semantics, no flush to zero), on the cached and the
    non-temporal kernels."""
    rng = np.random.default_rng(11 + n)
    base = (0.02 * rng.standard_normal(n)).astype(np.float32)
    specials = np.array([np.nan, np.inf, -np.inf, 1e-40, -1e-42, 2.0 ** -149, -0.0, 3e38],
                        dtype=np.float32)
    k = max(200, n // 1000)

    def planted(a):
        a = a.copy()
        idx = np.concatenate([rng.integers(0, n, size=k), [0, n - 1]])
        a[idx] = specials[rng.integers(0, specials.size, size=idx.size)]
        return a

    cks = [planted(base) for _ in range(3)]
    dev = torch.device("cuda")
    g_cks = [torch.from_numpy(c).to(dev) for c in cks]
    acc = torch.empty(n, device=dev)
    out = torch.empty(n, device=dev)
    ema = torch.from_numpy(base.copy()).to(dev)
    e_o = base.copy()
    r = dl.dl_round_begin(1, dl.DL_MEAN, n, [0, n], 1, 3, acc)
    if fused:
        dl.dl_fold_checkpoints_and_finalize_mean(r, 0, [0, 1, 2], 1, g_cks, out, ema, 0.9)
    else:
        dl.dl_fold_checkpoints(r, 0, [0, 1, 2], 1, g_cks)
        dl.dl_finalize_mean(r, 0, out, ema, 0.9)
    dl.dl_round_end(r)
    g_o = oracle.mean_round(cks, ema=e_o)
    torch.cuda.synchronize()
    assert mc.bits_equal(mc.to_np(out), g_o), mc.first_mismatch(mc.to_np(out), g_o)
    assert mc.bits_equal(mc.to_np(ema), e_o), mc.first_mismatch(mc.to_np(ema), e_o)
    th0 = planted(base)
    theta = torch.from_numpy(th0.copy()).to(dev)
    m = torch.zeros(n, device=dev)
    ema = torch.from_numpy(th0.copy()).to(dev)
    th_o, m_o, e_o = th0.copy(), np.zeros(n, np.float32), th0.copy()
    tok = [1000, 1001, 1002]
    r = dl.dl_round_begin(2, dl.DL_DELTA_NESTEROV, n, [0, n], 1, 3, acc)
    if fused:
        dl.dl_fold_checkpoints_and_outer_nesterov(r, 0, [0, 1, 2], 2, g_cks, tok, theta, m, 0.7,
                                                  0.9, ema, 0.9)
    else:
        dl.dl_fold_checkpoints(r, 0, [0, 1, 2], 2, g_cks, theta, tok)
        dl.dl_outer_nesterov(r, 0, theta, m, 0.7, 0.9, ema, 0.9)
    dl.dl_round_end(r)
    oracle.nesterov_fragment_round(th_o, m_o, cks, tok, 0.7, 0.9, e_o, 0.9)
    torch.cuda.synchronize()
    for name, g, o in (("theta", theta, th_o), ("m", m, m_o), ("ema", ema, e_o)):
        assert mc.bits_equal(mc.to_np(g), o), (name, mc.first_mismatch(mc.to_np(g), o))


@pytest.mark.parametrize("ckdtype", ["f32", "bf16"])
def test_several_arrivals_misaligned_checkpoint(ckdtype):
    """One checkpoint of the call one element off a 16-byte boundary (8 for
    bf16): the whole pass takes the element-by-element path, same bits."""
    w = dataclasses.replace(synth.scaled(W["diffurefill1b_frag_nesterov_ema"], 50_003, [0, 50_003]),
                            ckpt_dtype=ckdtype)
    n = w.n_params
    dev = torch.device("cuda")
    theta0 = synth.global0(w.seed, n)
    cks = [synth.worker_checkpoint(w.seed, 0, i, theta0.to(dev), dtype=ckdtype) for i in range(3)]
    shifted = torch.empty(n + 1, dtype=cks[1].dtype, device=dev)
    shifted[1:] = cks[1]
    g_cks = [cks[0], shifted[1:], cks[2]]
    assert g_cks[1].data_ptr() % (16 if ckdtype == "f32" else 8) != 0
    theta, m = theta0.to(dev), torch.zeros(n, device=dev)
    ema = theta0.to(dev)
    acc = torch.empty(n, device=dev)
    tok = [200_000, 210_000, 190_000]
    r = dl.dl_round_begin(3, dl.DL_DELTA_NESTEROV, n, [0, n], 3, 3, acc)
    dl.dl_fold_checkpoints_and_outer_nesterov(r, 0, [0, 1, 2], 3, g_cks, tok, theta, m, w.lr,
                                              w.mu, ema, w.beta)
    dl.dl_round_end(r)
    th_o, m_o, e_o = theta0.numpy().copy(), np.zeros(n, np.float32), theta0.numpy().copy()
    oracle.nesterov_fragment_round(th_o, m_o, [mc.to_np(c) for c in cks], tok, w.lr, w.mu, e_o,
                                   w.beta)
    torch.cuda.synchronize()
    for name, g, o in (("theta", theta, th_o), ("m", m, m_o), ("ema", ema, e_o)):
        assert mc.bits_equal(mc.to_np(g), o), (name, mc.first_mismatch(mc.to_np(g), o))
