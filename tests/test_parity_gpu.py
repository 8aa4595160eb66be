"""GPU parity: the HIP path through the C ABI against the CPU oracle,
element by element and bit for bit, on the same seeded inputs.

Sizes span many 4096-element tiles with ragged tails; fragment boundaries
both 16-byte aligned (128-bit path) and unaligned (scalar path).  Every
workload runs three consecutive rounds so momentum and EMA evolve."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from checkpoint_averaging_amd import synth
from tests import merge_cases as mc

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def small(key, n, offsets=None):
    return synth.scaled(W[key], n, offsets)


def run_rounds(w, rounds=3, exactly_quorum=False, fused_last=False):
    st = mc.init_state(w)
    for r in range(rounds):
        say(f"[parity] {w.key} n={w.n_params} frags={w.frag_offsets} round {r}"
            f" exactly_quorum={exactly_quorum} fused_last={fused_last}")
        res = mc.run_round(w, st, r, exactly_quorum=exactly_quorum, fused_last=fused_last)
        mc.assert_round_equal(res, f"{w.key} n={w.n_params} round {r}")
    return st


CASES = [
    # (workload, n, fragment offsets or None = scaled)
    ("pythia14m_mean", (1 << 20) + 37, None),
    ("pythia14m_frag_nesterov", (1 << 20) + 45, [0, 262_144, 300_000, 338_000, (1 << 20) + 45]),
    ("pythia14m_frag_nesterov", 777_777, [0, 123_457, 300_001, 300_002, 777_777]),  # unaligned
    ("diffurefill1b_mean_ema", 3 * 4096 * 4 + 3, None),
    ("diffurefill1b_bf16_mean_ema", (1 << 20) + 5, None),
    ("diffurefill1b_bf16_mean_ema", 99_999, [0, 99_999]),
    ("diffurefill1b_frag_nesterov_ema", (1 << 20) + 7, [0, 140_000, 428_000, 716_000, (1 << 20) + 7]),
    ("diffurefill1b_frag_nesterov_ema", 500_001, [0, 70_001, 214_003, 358_005, 500_001]),
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate_close", "fused_close"])
@pytest.mark.parametrize("key,n,offs", CASES, ids=[f"{k}-{n}" for k, n, _ in CASES])
def test_parity_small(key, n, offs, fused):
    run_rounds(small(key, n, offs), fused_last=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["separate_close", "fused_close"])
@pytest.mark.parametrize("key", ["pythia14m_frag_nesterov", "diffurefill1b_frag_nesterov_ema"])
def test_parity_exactly_quorum(key, fused):
    """Rounds close with exactly the quorum (a seeded late worker misses
    each fragment's close), as in 10 of the 348 GradientMail rounds."""
    w = small(key, 300_017, [0, 80_000, 160_000, 240_000, 300_017])
    run_rounds(w, rounds=2, exactly_quorum=True, fused_last=fused)


def test_parity_mean_in_fragments_and_quorum_one():
    """Plain averaging per fragment, quorum 1 (a restarted merger draining a
    single leftover checkpoint) on one fragment."""
    w = dataclasses.replace(small("pythia14m_mean", 200_003, [0, 50_000, 50_004, 200_003]),
                            quorum=1)
    st = mc.init_state(w)
    orders = [[2], [0, 1, 2], [1, 0]]
    res = mc.run_round(w, st, 0, orders=orders)
    mc.assert_round_equal(res, "mean per fragment")
    # the same with the last arrival fused into the close (the lone arrival of
    # fragment 0 is then both the first fold and the close)
    res = mc.run_round(w, st, 1, orders=orders, fused_last=True)
    mc.assert_round_equal(res, "mean per fragment, fused close")


def test_parity_nesterov_single_participant_fused():
    """A fragment round with one participant (quorum 1), closed by the fused
    call: its lone snapshot is both the first fold and the last."""
    w = dataclasses.replace(small("diffurefill1b_frag_nesterov_ema", 60_001, [0, 30_000, 60_001]),
                            quorum=1)
    st = mc.init_state(w)
    for r, orders in enumerate(([[3], [1, 4]], [[0, 2, 1], [2]])):
        res = mc.run_round(w, st, r, orders=orders, fused_last=True)
        mc.assert_round_equal(res, f"single participant, round {r}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 9, 1023, 1024, 1025, 4095, 4096, 4097,
                               16383, 16384, 16385])
def test_parity_edge_sizes(n):
    for key in ("diffurefill1b_bf16_mean_ema", "diffurefill1b_frag_nesterov_ema"):
        w = synth.scaled(W[key], n, [0, n])
        run_rounds(w, rounds=2)
        run_rounds(w, rounds=2, fused_last=True)


def test_arrival_order_decides_bits():
    """The GPU folds in call order: the oracle in the same order matches bit
    for bit; the oracle in a different order differs somewhere.  (fp32
    checkpoints: bf16 values of similar magnitude sum exactly in an fp32
    accumulator, so their order cannot show.)"""
    w = small("diffurefill1b_mean_ema", 1 << 18)
    st = mc.init_state(w)
    order = [3, 1, 4, 0, 2]
    res = mc.run_round(w, st, 0, orders=[order])
    mc.assert_round_equal(res, "order")
    import oracle
    theta0 = synth.global0(w.seed, w.n_params).numpy()
    cks = {i: mc.to_np(c) for i, c in mc.worker_inputs(w, 0, theta0).items()}
    other = oracle.mean_round([cks[i] for i in reversed(order)])
    assert not mc.bits_equal(res["theta"][0], other)
    # bf16 arrivals: the running fp32 sum is exact here, so any order agrees
    wb = small("diffurefill1b_bf16_mean_ema", 1 << 16)
    stb = mc.init_state(wb)
    orderb = [3, 1, 7, 0, 5, 2, 6, 4]
    resb = mc.run_round(wb, stb, 0, orders=[orderb])
    mc.assert_round_equal(resb, "order bf16")
    theta0 = synth.global0(wb.seed, wb.n_params).numpy()
    cks = {i: mc.to_np(c) for i, c in mc.worker_inputs(wb, 0, theta0).items()}
    assert mc.bits_equal(resb["theta"][0], oracle.mean_round([cks[i] for i in reversed(orderb)]))


def test_reconstruction_gives_identical_bits():
    """A failed round is rebuilt by re-folding the same arrivals in a new
    round: identical bits."""
    w = small("diffurefill1b_frag_nesterov_ema", 400_000, [0, 100_000, 200_000, 300_000, 400_000])
    a = mc.init_state(w)
    b = mc.init_state(w)
    ra = mc.run_round(w, a, 0)
    rb = mc.run_round(w, b, 0)
    for k in ra:
        assert mc.bits_equal(ra[k][0], rb[k][0]), k


@pytest.mark.parametrize("fused", [False, True], ids=["separate_close", "fused_close"])
@pytest.mark.parametrize("n", [4096 + 3, (1 << 24) + 3], ids=["cached", "non_temporal"])
def test_special_values_propagate(n, fused):
    """NaN, infinities and subnormals in checkpoints (and, in the fragment
    merge, in the global) propagate exactly as in the oracle (IEEE
    semantics, no flush to zero).  At 2^24 + 3 elements the non-temporal
    kernels run, passes alternate direction and the fragment merge reads the
    global through the cache."""
    import oracle
    from checkpoint_averaging_amd import dlmerge as dl
    rng = np.random.default_rng(3 + n)
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
    acc = torch.empty(n, device=dev)
    out = torch.empty(n, device=dev)
    ema = torch.from_numpy(base.copy()).to(dev)
    e_o = base.copy()
    r = dl.dl_round_begin(1, dl.DL_MEAN, n, [0, n], 1, 3, acc)
    for i, c in enumerate(cks[:-1] if fused else cks):
        dl.dl_fold_checkpoint(r, 0, i, 1, torch.from_numpy(c).to(dev))
    if fused:
        dl.dl_fold_and_finalize_mean(r, 0, 2, 1, torch.from_numpy(cks[2]).to(dev), out, ema, 0.9)
    else:
        dl.dl_finalize_mean(r, 0, out, ema, 0.9)
    dl.dl_round_end(r)
    g_o = oracle.mean_round(cks, ema=e_o)
    torch.cuda.synchronize()
    assert mc.bits_equal(mc.to_np(out), g_o), mc.first_mismatch(mc.to_np(out), g_o)
    assert mc.bits_equal(mc.to_np(ema), e_o), mc.first_mismatch(mc.to_np(ema), e_o)
    # the fragment merge with the same checkpoints and special values in the
    # global too, EMA fused into the close
    th0 = planted(base)
    theta = torch.from_numpy(th0.copy()).to(dev)
    m = torch.zeros(n, device=dev)
    ema = torch.from_numpy(th0.copy()).to(dev)
    th_o, m_o, e_o = th0.copy(), np.zeros(n, np.float32), th0.copy()
    tok = [1000, 1001, 1002]
    r = dl.dl_round_begin(2, dl.DL_DELTA_NESTEROV, n, [0, n], 1, 3, acc)
    for i, c in enumerate(cks[:-1] if fused else cks):
        dl.dl_fold_checkpoint(r, 0, i, 2, torch.from_numpy(c).to(dev), theta, tok[i])
    if fused:
        dl.dl_fold_and_outer_nesterov(r, 0, 2, 2, torch.from_numpy(cks[2]).to(dev), tok[2], theta,
                                      m, 0.7, 0.9, ema, 0.9)
    else:
        dl.dl_outer_nesterov(r, 0, theta, m, 0.7, 0.9, ema, 0.9)
    dl.dl_round_end(r)
    oracle.nesterov_fragment_round(th_o, m_o, cks, tok, 0.7, 0.9, e_o, 0.9)
    torch.cuda.synchronize()
    for name, g, o in (("theta", theta, th_o), ("m", m, m_o), ("ema", ema, e_o)):
        assert mc.bits_equal(mc.to_np(g), o), (name, mc.first_mismatch(mc.to_np(g), o))


def test_in_place_mean_and_misaligned_checkpoint():
    """The mean written in place over the accumulator, and a checkpoint whose
    address is only 4-byte aligned (scalar path), both match the oracle."""
    import oracle
    from checkpoint_averaging_amd import dlmerge as dl
    n = 10_001
    rng = np.random.default_rng(4)
    cks = [(0.02 * rng.standard_normal(n)).astype(np.float32) for _ in range(3)]
    dev = torch.device("cuda")
    acc = torch.empty(n, device=dev)
    big = torch.empty(n + 1, device=dev)
    r = dl.dl_round_begin(9, dl.DL_MEAN, n, [0, n], 2, 3, acc)
    dl.dl_fold_checkpoint(r, 0, 0, 9, torch.from_numpy(cks[0]).to(dev))
    big[1:] = torch.from_numpy(cks[1]).to(dev)
    dl.dl_fold_checkpoint(r, 0, 1, 9, big.data_ptr() + 4, dtype=dl.DL_F32)   # misaligned
    dl.dl_fold_checkpoint(r, 0, 2, 9, torch.from_numpy(cks[2]).to(dev))
    dl.dl_finalize_mean(r, 0, acc)                                           # in place
    dl.dl_round_end(r)
    torch.cuda.synchronize()
    want = oracle.mean_round(cks)
    assert mc.bits_equal(mc.to_np(acc), want), mc.first_mismatch(mc.to_np(acc), want)


def test_generator_same_bits_on_gpu():
    """The seeded generator gives the same bits on the GPU as on the CPU
    (the oracle side regenerates windows of full-size inputs on the CPU)."""
    for start in (0, 123_456_789, (1 << 32) - 1000):
        a = synth.std_normalish(1005, 3, 2, start, 70_001)
        b = synth.std_normalish(1005, 3, 2, start, 70_001, device="cuda").cpu()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), start
    th = synth.global0(1004, 50_000, start=1000)
    th_g = synth.global0(1004, 50_000, device="cuda", start=1000)
    assert torch.equal(th.view(torch.int32), th_g.cpu().view(torch.int32))
    for dt in ("f32", "bf16"):
        c = synth.worker_checkpoint(1004, 2, 5, th, start=1000, dtype=dt)
        c_g = synth.worker_checkpoint(1004, 2, 5, th_g, start=1000, dtype=dt)
        assert torch.equal(c, c_g.cpu()), dt


def test_ema_update_standalone():
    import oracle
    from checkpoint_averaging_amd import dlmerge as dl
    for n in (1, 6, 4096 * 3 + 1, 1 << 20):
        rng = np.random.default_rng(n)
        e = (0.02 * rng.standard_normal(n)).astype(np.float32)
        g = (0.02 * rng.standard_normal(n)).astype(np.float32)
        ge = torch.from_numpy(e).cuda()
        gg = torch.from_numpy(g).cuda()
        for k in range(3):
            dl.dl_ema_update(ge, gg, 0.9)
            oracle.ema_update(e, g, 0.9)
        torch.cuda.synchronize()
        assert mc.bits_equal(mc.to_np(ge), e), (n, mc.first_mismatch(mc.to_np(ge), e))
