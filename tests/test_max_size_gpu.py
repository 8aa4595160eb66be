"""Ranges larger than one launch's 2^32 - 1 work-items: a fragment of
2^32 + 37 elements (17.2 GB of fp32), so the 128-bit path loops over more
tiles than its capped grid and the scalar path (forced by a misaligned
checkpoint) loops too.  Inputs are constants whose merge is exact, so every
element is checked against its closed value."""
import numpy as np
import pytest
import torch

from checkpoint_averaging_amd import dlmerge as dl

pytestmark = pytest.mark.gpu

N = (1 << 32) + 37


def test_mean_round_above_launch_limit():
    dev = torch.device("cuda")
    acc = torch.empty(N, device=dev)
    c1 = torch.full((N,), 1.5, device=dev)
    c2 = torch.empty(N + 1, device=dev)          # offset by one element: scalar path
    c2.fill_(2.5)
    ema = torch.full((N,), 4.0, device=dev)
    r = dl.dl_round_begin(1, dl.DL_MEAN, N, [0, N], 2, 2, acc)
    dl.dl_fold_checkpoint(r, 0, 0, 1, c1)
    dl.dl_fold_and_finalize_mean(r, 0, 1, 1, c2.data_ptr() + 4, acc, ema, 0.5,
                                 dtype=dl.DL_F32)
    dl.dl_round_end(r)
    torch.cuda.synchronize()
    assert bool((acc == 2.0).all())              # (1.5 + 2.5) / 2
    assert bool((ema == 3.0).all())              # 0.5 * 4 + 0.5 * 2
    del acc, c1, c2, ema
    torch.cuda.empty_cache()


def test_nesterov_round_above_launch_limit():
    dev = torch.device("cuda")
    theta = torch.zeros(N, device=dev)
    m = torch.zeros(N, device=dev)
    acc = torch.empty(N, device=dev)
    c1 = torch.full((N,), -1.0, device=dev)      # delta theta - c = 1
    c2 = torch.full((N,), -1.0, device=dev)
    r = dl.dl_round_begin(2, dl.DL_DELTA_NESTEROV, N, [0, N], 1, 2, acc)
    dl.dl_fold_checkpoint(r, 0, 0, 2, c1, theta, 1)
    dl.dl_fold_and_outer_nesterov(r, 0, 1, 2, c2, 3, theta, m, 0.7, 0.9)
    dl.dl_round_end(r)
    torch.cuda.synchronize()
    # dbar = 4/4 = 1; m' = 0.9*0 + 1 = 1; u = 1 + 0.9*1; theta' = 0 - 0.7*u (binary32)
    f = np.float32
    u = f(1.0) + f(0.9) * f(1.0)
    want = f(0.0) - f(0.7) * u
    assert bool((m == 1.0).all())
    assert bool((theta == float(want)).all())
    del theta, m, acc, c1, c2
    torch.cuda.empty_cache()


def test_several_arrival_passes_above_launch_limit():
    """The several-arrival passes over 2^32 + 37 elements: the mean with one
    misaligned checkpoint (element-by-element path), the Nesterov close on
    the 128-bit path; both loop over more tiles than their capped grids."""
    dev = torch.device("cuda")
    acc = torch.empty(N, device=dev)
    c1 = torch.full((N,), 1.5, device=dev)
    c2 = torch.empty(N + 1, device=dev)          # offset by one element: scalar path
    c2.fill_(2.5)
    ema = torch.full((N,), 4.0, device=dev)
    r = dl.dl_round_begin(3, dl.DL_MEAN, N, [0, N], 2, 2, acc)
    dl.dl_fold_checkpoints_and_finalize_mean(r, 0, [0, 1], 3, [c1, c2.data_ptr() + 4], acc, ema,
                                             0.5, dtype=dl.DL_F32)
    dl.dl_round_end(r)
    torch.cuda.synchronize()
    assert bool((acc == 2.0).all())
    assert bool((ema == 3.0).all())
    del c2, ema
    torch.cuda.empty_cache()
    theta = torch.zeros(N, device=dev)
    m = torch.zeros(N, device=dev)
    c1.fill_(-1.0)
    r = dl.dl_round_begin(4, dl.DL_DELTA_NESTEROV, N, [0, N], 1, 2, acc)
    dl.dl_fold_checkpoints_and_outer_nesterov(r, 0, [0, 1], 4, [c1, c1], [1, 3], theta, m, 0.7,
                                              0.9)
    dl.dl_round_end(r)
    torch.cuda.synchronize()
    f = np.float32
    u = f(1.0) + f(0.9) * f(1.0)
    want = f(0.0) - f(0.7) * u
    assert bool((m == 1.0).all())
    assert bool((theta == float(want)).all())
    del theta, m, acc, c1
    torch.cuda.empty_cache()
