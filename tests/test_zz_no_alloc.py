"""The allocation-free outer orthogonal step (dl_outer_orthogonal_step_noalloc)
against the workspace entry point (dl_outer_orthogonal_step) through the C
ABI.  Calls come in a row on shrinking matrices: the first near the largest
the library's scratch holds, then smaller ones that find the scratch holding
the previous call's values.  Each result equals the workspace call on the
same inputs bit for bit (same kernels, same workspace layout).  The last is
also checked, every element, against the oracle's per-element tolerance
(DiffuRefill-1B technical report, "What we measured", "Optimisers")."""
import numpy as np
import pytest
import torch

from checkpoint_averaging_amd import dlmerge as dl
from checkpoint_averaging_amd import synth
from tests import polar_tolerance as pt

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


def _inputs(seed, rows, cols):
    theta = synth.global0(seed, rows * cols, device=DEV)
    return theta, synth.worker_checkpoint(seed, 0, 0, theta)


def test_noalloc_step_matches_workspace_step_on_successive_calls():
    scale = 1.0
    shapes = ((2101, 5632, 2048), (2102, 2048, 2048), (2103, 300, 130))
    for seed, rows, cols in shapes:
        print(f"noalloc step {rows}x{cols}", flush=True)
        assert dl.dl_polar_workspace_bytes(rows, cols) <= dl.DL_NOALLOC_SCRATCH_BYTES
        theta, avg = _inputs(seed, rows, cols)
        th_h = theta.cpu().numpy().astype(np.float64).reshape(rows, cols)
        av_h = avg.cpu().numpy().astype(np.float64).reshape(rows, cols)
        ref = theta.clone()
        ws = torch.empty(dl.dl_polar_workspace_bytes(rows, cols) // 4 + 64, device=DEV)
        dl.dl_outer_orthogonal_step(ref, avg, rows, cols, scale, ws)
        dl.dl_outer_orthogonal_step_noalloc(theta, avg, rows, cols, scale)
        torch.cuda.synchronize()
        assert torch.equal(theta.view(torch.int32), ref.view(torch.int32)), (rows, cols)
        assert np.array_equal(avg.cpu().numpy().astype(np.float64).reshape(rows, cols), av_h)
    got = theta.cpu().numpy().astype(np.float64).reshape(rows, cols)
    e = pt.expected(th_h - av_h)
    want = th_h - scale * e.iterated
    worst = float(np.max(np.abs(got - want) / pt.step_tolerance(th_h, got, e, scale)))
    print(f"noalloc step {rows}x{cols}: max |err|/tol = {worst:.3f}", flush=True)
    assert worst <= 1.0


def test_noalloc_step_refuses_a_matrix_beyond_its_scratch():
    theta, avg = _inputs(2104, 64, 64)      # never touched: refused on the host
    with pytest.raises(dl.DLError) as ei:
        dl.dl_outer_orthogonal_step_noalloc(theta.data_ptr(), avg.data_ptr(), 73760, 2048, 1.0)
    assert ei.value.status == dl.DL_E_TOO_LARGE
