"""Parity at the full sizes of the five merge workloads, in the launch
configuration the benchmark times (checkpoint_averaging_amd.workload).

Every element is compared for all five workloads (for the 1.08B ones the
generator's GPU-made inputs are copied to host memory and the oracle runs the
whole rounds).  The 1.08B workloads are also compared on sampled windows with
inputs the seeded generator regenerates on the CPU for just those windows (the
merge is elementwise, so the oracle recomputes any window on its own); the
windows cover the first and last elements of every fragment plus random
positions."""
import sys

import numpy as np
import pytest
import torch

import oracle
from checkpoint_averaging_amd import dlmerge as dl
from checkpoint_averaging_amd import synth
from checkpoint_averaging_amd.workload import GpuWorkload
from tests import merge_cases as mc

pytestmark = pytest.mark.gpu

ROUNDS = 2
WIN = 4096


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def windows(w, n_random, seed):
    """Per fragment: sorted, disjoint (start, length) windows inside it."""
    rng = np.random.default_rng(seed)
    out = []
    for f in range(w.n_frags):
        o0, o1 = w.frag_offsets[f], w.frag_offsets[f + 1]
        L = min(WIN, o1 - o0)
        starts = {o0, o1 - L}
        for s in rng.integers(o0, o1 - L + 1, size=n_random):
            starts.add(int(s))
        merged = []
        for s in sorted(starts):
            e = s + L
            if merged and s <= merged[-1][1]:
                merged[-1][1] = max(merged[-1][1], e)
            else:
                merged.append([s, e])
        out.append([(s, e - s) for s, e in merged])
    return out


def oracle_on_windows(w, wins):
    """Run the oracle over the given windows for ROUNDS rounds with inputs
    regenerated on the CPU; returns {"theta", "m", "e"} per fragment."""
    orc = oracle.load()
    res = []
    for f, fw in enumerate(wins):
        th0 = np.concatenate([synth.global0(w.seed, L, start=s).numpy() for s, L in fw])
        theta = th0.copy()
        m = np.zeros_like(theta)
        e = th0.copy() if w.ema else None
        for r in range(ROUNDS):
            cks = {}
            for i in range(w.workers):
                parts = [synth.worker_checkpoint(w.seed, r, i,
                                                 synth.global0(w.seed, L, start=s),
                                                 start=s, dtype=w.ckpt_dtype) for s, L in fw]
                cks[i] = mc.to_np(torch.cat(parts))
            order = synth.arrival_order(w, r, f)
            if w.mode == "mean":
                theta = orc.mean_round([cks[i] for i in order], ema=e, beta=w.beta)
            else:
                tok = synth.token_counts(w, r)
                orc.nesterov_fragment_round(theta, m, [cks[i] for i in order],
                                            [tok[i] for i in order], w.lr, w.mu, e, w.beta)
        res.append({"theta": theta, "m": m if w.mode != "mean" else None, "e": e})
    return res


def gather(t, fw):
    return np.concatenate([mc.to_np(t[s:s + L]) for s, L in fw])


@pytest.mark.parametrize("key", ["diffurefill1b_mean_ema", "diffurefill1b_bf16_mean_ema",
                                 "diffurefill1b_frag_nesterov_ema"])
def test_full_size_sampled(key):
    """Two GPU states on the same checkpoints, one folding each arrival with
    its own call, the other taking each fragment's arrivals in one
    several-arrival call (one pass per fragment when it also closes);
    sampled windows of both against the oracle on CPU-regenerated inputs."""
    w = synth.WORKLOADS[key]
    say(f"[full] {key}: allocating and generating {w.n_params} params x {w.workers} workers")
    per_arrival = GpuWorkload(w)
    batched = GpuWorkload(w)
    batched.ckpts = per_arrival.ckpts              # the same checkpoint buffers
    torch.cuda.empty_cache()
    for r in range(ROUNDS):
        per_arrival.generate_checkpoints(r)
        # round 0 closes with the fused last arrival (the benchmark's round),
        # round 1 with a separate close
        say(f"[full] {key}: round {r} fused_close={r == 0}, per arrival and batched")
        per_arrival.run_round(r, tag=100 + r, fused_close=(r == 0))
        batched.run_round(r, tag=100 + r, fused_close=(r == 0), batched=True)
    torch.cuda.synchronize()
    wins = windows(w, 24, seed=w.seed)
    say(f"[full] {key}: oracle on {sum(L for fw in wins for _, L in fw)} sampled elements")
    want = oracle_on_windows(w, wins)
    for gw, how in ((per_arrival, "per arrival"), (batched, "batched")):
        for f, fw in enumerate(wins):
            for k in ("theta", "m", "e"):
                t = getattr(gw, k)
                if t is None:
                    continue
                g, o = gather(t, fw), want[f][k]
                assert mc.bits_equal(g, o), f"{key} {how} frag {f} {k}: {mc.first_mismatch(g, o)}"
    del per_arrival, batched
    torch.cuda.empty_cache()


def _oracle_full_round(w, r, cks, theta, m, e):
    """The oracle's round r over whole arrays (host copies of the inputs)."""
    orc = oracle.load()
    tok = synth.token_counts(w, r)
    for f in range(w.n_frags):
        o0, o1 = w.frag_offsets[f], w.frag_offsets[f + 1]
        order = synth.arrival_order(w, r, f)
        parts = [np.ascontiguousarray(cks[i][o0:o1]) for i in order]
        if w.mode == "mean":
            theta[o0:o1] = orc.mean_round(parts, None if e is None else e[o0:o1], w.beta)
        else:
            orc.nesterov_fragment_round(theta[o0:o1], m[o0:o1], parts, [tok[i] for i in order],
                                        w.lr, w.mu, None if e is None else e[o0:o1], w.beta)


@pytest.mark.parametrize("key", ["diffurefill1b_mean_ema", "diffurefill1b_bf16_mean_ema",
                                 "diffurefill1b_frag_nesterov_ema"])
def test_full_size_1b_every_element(key):
    """Every element of the 1.08B rounds, in the benchmark's launch
    configuration: the inputs the generator made on the GPU are copied to
    host memory and the oracle runs the same rounds over whole arrays, one
    arrival at a time.  Two GPU states take the same checkpoints: one folds
    each arrival with its own call, the other takes each fragment's arrivals
    in one several-arrival call (one pass per fragment); both are compared
    with the oracle."""
    w = synth.WORKLOADS[key]
    say(f"[full-all] {key}: allocating and generating")
    per_arrival = GpuWorkload(w)
    batched = GpuWorkload(w)
    batched.ckpts = per_arrival.ckpts              # the same checkpoint buffers
    torch.cuda.empty_cache()
    theta = mc.to_np(per_arrival.theta)
    m = np.zeros_like(theta) if per_arrival.m is not None else None
    e = theta.copy() if per_arrival.e is not None else None
    for r in range(ROUNDS):
        per_arrival.generate_checkpoints(r)
        say(f"[full-all] {key}: round {r} fused_close={r == 0}, per arrival and batched")
        per_arrival.run_round(r, tag=200 + r, fused_close=(r == 0))
        batched.run_round(r, tag=200 + r, fused_close=(r == 0), batched=True)
        cks = [mc.to_np(c) for c in per_arrival.ckpts]
        say(f"[full-all] {key}: oracle round {r}")
        _oracle_full_round(w, r, cks, theta, m, e)
        del cks
        for gw, how in ((per_arrival, "per arrival"), (batched, "batched")):
            for k, o in (("theta", theta), ("m", m), ("e", e)):
                if o is None:
                    continue
                g = mc.to_np(getattr(gw, k))
                assert mc.bits_equal(g, o), f"{key} {how} round {r} {k}: {mc.first_mismatch(g, o)}"
                del g
    del per_arrival, batched
    torch.cuda.empty_cache()


@pytest.mark.parametrize("key", ["pythia14m_mean", "pythia14m_frag_nesterov"])
def test_full_size_every_element(key):
    w = synth.WORKLOADS[key]
    st = mc.init_state(w)
    for r in range(3):
        say(f"[full] {key}: round {r}")
        res = mc.run_round(w, st, r, fused_last=(r != 1))
        mc.assert_round_equal(res, f"{key} round {r}")


def test_full_size_fragment_rounds_on_separate_streams():
    """The 1.08B fragment merge with each fragment's round on its own stream
    (arrivals issued round-robin across fragments, as
    `bench.py --fragment-streams 4` times it), on sampled windows of every
    fragment against the oracle's one-at-a-time rounds."""
    key = "diffurefill1b_frag_nesterov_ema"
    w = synth.WORKLOADS[key]
    say(f"[full-streams] {key}: allocating and generating")
    gw = GpuWorkload(w)
    streams = [torch.cuda.Stream() for _ in range(4)]
    for r in range(ROUNDS):
        gw.generate_checkpoints(r)
        say(f"[full-streams] {key}: round {r} on 4 streams, fused_close={r == 0}")
        gw.run_round(r, tag=200 + r, fused_close=(r == 0), streams=streams)
    torch.cuda.synchronize()
    wins = windows(w, 16, seed=w.seed + 1)
    want = oracle_on_windows(w, wins)
    for f, fw in enumerate(wins):
        for k, t in (("theta", gw.theta), ("m", gw.m), ("e", gw.e)):
            g, o = gather(t, fw), want[f][k]
            assert mc.bits_equal(g, o), f"frag {f} {k}: {mc.first_mismatch(g, o)}"
    del gw
    torch.cuda.empty_cache()


def _partial_participants(w, rnd, f, n):
    """The first n arrivals of a round and fragment that are not among its
    seeded late workers (the seeded late worker and the worker arriving right
    after it miss the close)."""
    order = synth.arrival_order(w, rnd, f)
    late = synth.late_worker(w, rnd, f)
    k = order.index(late)
    missing = {late, order[(k + 1) % len(order)]}
    return [i for i in order if i not in missing][:n]


def _run_partial_round(gw, rnd, tag, parts, quorum, fused, batched=False):
    """One round through the C ABI on the workload's full-size buffers (the
    benchmark's launch configuration), each fragment closed by the given
    participants in the given order (with `batched`: all of them in one
    several-arrival call that also closes)."""
    w = gw.w
    offs = list(w.frag_offsets)
    mode = dl.DL_DELTA_NESTEROV if gw.delta else dl.DL_MEAN
    tok = synth.token_counts(w, rnd)
    out = gw.acc if gw.close_in_place else gw.theta
    r = dl.dl_round_begin(tag, mode, w.n_params, offs, quorum, w.workers, gw.acc)
    try:
        for f in range(w.n_frags):
            o0, o1 = offs[f], offs[f + 1]
            ps = parts[f]
            if batched:
                cks = [gw.ckpts[i][o0:o1] for i in ps]
                if gw.delta:
                    dl.dl_fold_checkpoints_and_outer_nesterov(
                        r, f, ps, tag, cks, [tok[i] for i in ps], gw.theta, gw.m, w.lr, w.mu,
                        gw.e, w.beta)
                else:
                    dl.dl_fold_checkpoints_and_finalize_mean(r, f, ps, tag, cks, out, gw.e,
                                                             w.beta)
                assert dl.dl_round_participants(r, f) == list(ps)
                continue
            for i in (ps[:-1] if fused else ps):
                ck = gw.ckpts[i][o0:o1]
                if gw.delta:
                    dl.dl_fold_checkpoint(r, f, i, tag, ck, gw.theta, tok[i])
                else:
                    dl.dl_fold_checkpoint(r, f, i, tag, ck)
            if gw.delta:
                if fused:
                    dl.dl_fold_and_outer_nesterov(r, f, ps[-1], tag, gw.ckpts[ps[-1]][o0:o1],
                                                  tok[ps[-1]], gw.theta, gw.m, w.lr, w.mu,
                                                  gw.e, w.beta)
                else:
                    dl.dl_outer_nesterov(r, f, gw.theta, gw.m, w.lr, w.mu, gw.e, w.beta)
            else:
                if fused:
                    dl.dl_fold_and_finalize_mean(r, f, ps[-1], tag, gw.ckpts[ps[-1]][o0:o1], out,
                                                 gw.e, w.beta)
                else:
                    dl.dl_finalize_mean(r, f, out, gw.e, w.beta)
            assert dl.dl_round_participants(r, f) == list(ps)
    finally:
        dl.dl_round_end(r)
    gw._swap_if_in_place()


def _oracle_partial_on_windows(w, wins, parts_of):
    """The oracle's rounds over the windows, each fragment closed by
    parts_of(rnd, f) in that order."""
    orc = oracle.load()
    res = []
    for f, fw in enumerate(wins):
        th0 = np.concatenate([synth.global0(w.seed, L, start=s).numpy() for s, L in fw])
        theta, m = th0.copy(), np.zeros_like(th0)
        e = th0.copy() if w.ema else None
        for r in range(ROUNDS):
            ps = parts_of(r, f)
            cks = {i: mc.to_np(torch.cat([synth.worker_checkpoint(
                w.seed, r, i, synth.global0(w.seed, L, start=s), start=s, dtype=w.ckpt_dtype)
                for s, L in fw])) for i in ps}
            if w.mode == "mean":
                theta = orc.mean_round([cks[i] for i in ps], ema=e, beta=w.beta)
            else:
                tok = synth.token_counts(w, r)
                orc.nesterov_fragment_round(theta, m, [cks[i] for i in ps], [tok[i] for i in ps],
                                            w.lr, w.mu, e, w.beta)
        res.append({"theta": theta, "m": m if w.mode != "mean" else None, "e": e})
    return res


@pytest.mark.parametrize("key,n_close,batched", [
    # every fragment closed by exactly its quorum of 3 of the 5 workers
    # (GradientMail post, "Completing the run": 10 of 348 rounds closed with 3)
    ("diffurefill1b_frag_nesterov_ema", 3, False),
    ("diffurefill1b_frag_nesterov_ema", 3, True),
    # a drain: a single leftover checkpoint closes the round with quorum 1
    # (technical report, Table 2, row "Recovery")
    ("diffurefill1b_mean_ema", 1, False),
    ("diffurefill1b_mean_ema", 1, True),
])
def test_full_size_partial_participation(key, n_close, batched):
    """Partial participation at full size, on the non-temporal kernels the
    small parity cases never reach: round 0 closes with the fused last
    arrival (for the drain: the first arrival folded in the same pass as the
    close), round 1 with a separate close; with `batched` both rounds pass
    the participants in one call that also closes.  Sampled windows of every
    fragment against the oracle, bit for bit."""
    w = synth.WORKLOADS[key]
    quorum = min(w.quorum, n_close)
    parts_of = lambda r, f: _partial_participants(w, r, f, n_close)
    say(f"[partial] {key}: allocating and generating, {n_close} of {w.workers} close")
    gw = GpuWorkload(w)
    for r in range(ROUNDS):
        gw.generate_checkpoints(r)
        parts = [parts_of(r, f) for f in range(w.n_frags)]
        say(f"[partial] {key}: round {r} participants {parts} fused_close={r == 0}"
            f" batched={batched}")
        _run_partial_round(gw, r, 300 + r, parts, quorum, fused=(r == 0), batched=batched)
    torch.cuda.synchronize()
    wins = windows(w, 16, seed=w.seed + 2)
    want = _oracle_partial_on_windows(w, wins, parts_of)
    for f, fw in enumerate(wins):
        for k, t in (("theta", gw.theta), ("m", gw.m), ("e", gw.e)):
            if t is None:
                continue
            g, o = gather(t, fw), want[f][k]
            assert mc.bits_equal(g, o), f"{key} frag {f} {k}: {mc.first_mismatch(g, o)}"
    del gw
    torch.cuda.empty_cache()
