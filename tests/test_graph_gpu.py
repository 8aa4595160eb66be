"""A merge round captured into a HIP graph (torch.cuda.CUDAGraph around the
library's calls on torch's current stream): capture records the folds and
the close without running them, and every replay runs one more round on
the same buffers.  Replays are checked, bit for bit, against the same rounds
run eagerly on a second copy of the state, with eager work and
synchronisations between the replays, and the state after the last replay
against the CPU oracle's same four rounds.  Rounds are issued one call
per arrival, or with each fragment's arrivals in one several-arrival call."""
import numpy as np
import pytest
import torch

import oracle
from checkpoint_averaging_amd import synth
from checkpoint_averaging_amd.workload import GpuWorkload
from tests import merge_cases as mc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused,batched", [(False, False), (True, False), (True, True),
                                          (False, True)],
                         ids=["separate_close", "fused_close", "one_pass", "one_pass_then_close"])
@pytest.mark.parametrize("key,n,offs", [
    ("pythia14m_mean", 300_005, [0, 300_005]),
    ("pythia14m_frag_nesterov", 400_003, [0, 150_000, 200_004, 250_000, 400_003]),
    ("diffurefill1b_bf16_mean_ema", 200_001, [0, 200_001]),
])
def test_captured_round_replays_match_eager_rounds(key, n, offs, fused, batched):
    w = synth.scaled(synth.WORKLOADS[key], n, offs)
    eager = GpuWorkload(w)
    graphed = GpuWorkload(w)
    eager.generate_checkpoints(0)
    graphed.generate_checkpoints(0)
    eager.run_round(0, tag=1, fused_close=fused, batched=batched)   # loads the kernels
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run_round(0, tag=1, fused_close=fused, batched=batched)
    torch.cuda.synchronize()
    for k in range(4):
        g.replay()
        if k:
            eager.run_round(0, tag=2 + k, fused_close=fused, batched=batched)
        torch.cuda.synchronize()
        for name in ("theta", "m", "e"):
            a, b = getattr(graphed, name), getattr(eager, name)
            if a is None:
                continue
            ga, gb = mc.to_np(a), mc.to_np(b)
            assert mc.bits_equal(ga, gb), (k, name, mc.first_mismatch(ga, gb))
    # the oracle runs the same four rounds (round-0 inputs, orders and token
    # counts each time, as run_round(0, ...) issues them)
    orc = oracle.load()
    cks = [mc.to_np(c) for c in graphed.ckpts]
    theta = synth.global0(w.seed, w.n_params).numpy()
    m = np.zeros_like(theta)
    e = theta.copy() if w.ema else None
    tok = synth.token_counts(w, 0)
    for _ in range(4):
        for f in range(w.n_frags):
            o0, o1 = w.frag_offsets[f], w.frag_offsets[f + 1]
            order = synth.arrival_order(w, 0, f)
            parts = [np.ascontiguousarray(cks[i][o0:o1]) for i in order]
            ef = None if e is None else e[o0:o1]
            if w.mode == "mean":
                theta[o0:o1] = orc.mean_round(parts, ef, w.beta)
            else:
                orc.nesterov_fragment_round(theta[o0:o1], m[o0:o1], parts,
                                            [tok[i] for i in order], w.lr, w.mu, ef, w.beta)
    for name, want in (("theta", theta), ("m", m if graphed.m is not None else None), ("e", e)):
        if want is None:
            continue
        got = mc.to_np(getattr(graphed, name))
        assert mc.bits_equal(got, want), ("oracle", name, mc.first_mismatch(got, want))
