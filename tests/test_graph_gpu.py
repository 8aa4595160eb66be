"""A merge round captured into a HIP graph (torch.cuda.CUDAGraph around the
library's calls on torch's current stream): capture records the folds and
the close without running them, and every replay runs one more round on
the same buffers.  Replays are checked, bit for bit, against the same rounds
run eagerly on a second copy of the state, with eager work and
synchronisations between the replays."""
import pytest
import torch

from checkpoint_averaging_amd import synth
from checkpoint_averaging_amd.workload import GpuWorkload
from tests import merge_cases as mc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True], ids=["separate_close", "fused_close"])
@pytest.mark.parametrize("key,n,offs", [
    ("pythia14m_mean", 300_005, [0, 300_005]),
    ("pythia14m_frag_nesterov", 400_003, [0, 150_000, 200_004, 250_000, 400_003]),
    ("diffurefill1b_bf16_mean_ema", 200_001, [0, 200_001]),
])
def test_captured_round_replays_match_eager_rounds(key, n, offs, fused):
    w = synth.scaled(synth.WORKLOADS[key], n, offs)
    eager = GpuWorkload(w)
    graphed = GpuWorkload(w)
    eager.generate_checkpoints(0)
    graphed.generate_checkpoints(0)
    eager.run_round(0, tag=1, fused_close=fused)        # also loads the kernels before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run_round(0, tag=1, fused_close=fused)
    torch.cuda.synchronize()
    for k in range(4):
        g.replay()
        if k:
            eager.run_round(0, tag=2 + k, fused_close=fused)
        torch.cuda.synchronize()
        for name in ("theta", "m", "e"):
            a, b = getattr(graphed, name), getattr(eager, name)
            if a is None:
                continue
            ga, gb = mc.to_np(a), mc.to_np(b)
            assert mc.bits_equal(ga, gb), (k, name, mc.first_mismatch(ga, gb))
