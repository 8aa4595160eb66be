"""Drivers that run merge rounds of a workload through the C ABI on the GPU
and through the CPU oracle on the same seeded inputs, for the parity tests.

Inputs are produced by checkpoint_averaging_amd.synth only.  Worker
checkpoints of round r are generated from the oracle's round-r global (the
generator runs on the GPU for speed; its bits do not depend on the device)
and copied to the host for the oracle, so no oracle input ever comes from the
merge kernels.  The GPU keeps its own global / momentum / EMA state across
rounds and is compared with the oracle's after every round.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle
from checkpoint_averaging_amd import synth
from checkpoint_averaging_amd import dlmerge as dl


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def _mismatch_mask(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Elements whose bits differ, except where both are NaN: IEEE fixes that
    an operation yields NaN, not the sign or payload of a NaN it creates (x86
    SSE and the GPU create different ones for inf - inf)."""
    diff = a.view(np.uint32) != b.view(np.uint32)
    return diff & ~(np.isnan(a) & np.isnan(b))


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    return (a.dtype == b.dtype and a.shape == b.shape
            and not np.any(_mismatch_mask(a, b)))


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    bad = np.nonzero(_mismatch_mask(a, b))[0]
    if bad.size == 0:
        return "none"
    j = bad[0]
    return f"{bad.size} mismatches, first at {j}: gpu {a[j]!r} oracle {b[j]!r}"


@dataclasses.dataclass
class State:
    theta: np.ndarray                       # oracle global
    m: Optional[np.ndarray]                 # oracle momentum (delta mode)
    e: Optional[np.ndarray]                 # oracle EMA
    g_theta: torch.Tensor                   # GPU global
    g_m: Optional[torch.Tensor]
    g_e: Optional[torch.Tensor]
    g_acc: torch.Tensor


def init_state(w: synth.Workload, device="cuda") -> State:
    theta = synth.global0(w.seed, w.n_params, device=device).cpu().numpy()
    delta = w.mode == "delta_nesterov"
    m = np.zeros_like(theta) if delta else None
    e = theta.copy() if w.ema else None                 # EMA starts at the first global
    dev = torch.device(device)
    return State(theta=theta, m=m, e=e,
                 g_theta=torch.from_numpy(theta).to(dev),
                 g_m=torch.zeros(w.n_params, dtype=torch.float32, device=dev) if delta else None,
                 g_e=torch.from_numpy(e).to(dev) if e is not None else None,
                 g_acc=torch.full((w.n_params,), float("nan"), dtype=torch.float32, device=dev))


def worker_inputs(w: synth.Workload, rnd: int, theta: np.ndarray,
                  device="cuda") -> Dict[int, torch.Tensor]:
    """Full-length checkpoints of every worker for round rnd, made by the
    seeded generator from the oracle's round-rnd global.  The generator runs
    on `device` (its bits do not depend on the device)."""
    th = torch.from_numpy(theta).to(device)
    return {i: synth.worker_checkpoint(w.seed, rnd, i, th, dtype=w.ckpt_dtype)
            for i in range(w.workers)}


def participants(w: synth.Workload, rnd: int, frag: int, exactly_quorum: bool) -> List[int]:
    order = synth.arrival_order(w, rnd, frag)
    if exactly_quorum:
        late = synth.late_worker(w, rnd, frag)
        order = [i for i in order if i != late][: w.quorum]
    return order


def _calls(order: Sequence[int], fused_last: bool, batch: Optional[int], single_first: int):
    """How the GPU side issues a fragment's arrivals: a list of (kind, ids)
    with kind "one" (dl_fold_checkpoint), "many" (dl_fold_checkpoints),
    "one_close" / "many_close" (the folding-and-closing calls) or "close"."""
    order = list(order)
    if batch is None:
        calls = [("one", [i]) for i in order]
        if fused_last:
            calls[-1] = ("one_close", calls[-1][1])
        else:
            calls.append(("close", []))
        return calls
    calls = [("one", [i]) for i in order[:single_first]]
    rest = order[single_first:]
    chunks = [rest[k:k + batch] for k in range(0, len(rest), batch)]
    calls += [("many", c) for c in chunks]
    if fused_last:
        kind, ids = calls[-1]
        calls[-1] = ("many_close" if kind == "many" else "one_close", ids)
    else:
        calls.append(("close", []))
    return calls


def run_round(w: synth.Workload, st: State, rnd: int, exactly_quorum: bool = False,
              orders: Optional[Sequence[Sequence[int]]] = None, stream=None,
              fused_last: bool = False, batch: Optional[int] = None,
              single_first: int = 0) -> dict:
    """One round on both sides.  Returns the GPU and oracle results (numpy).

    With `fused_last` the GPU folds each fragment's last arrival and closes
    the fragment in one call (dl_fold_and_*); the oracle always folds and
    closes in separate steps, so the comparison also checks that the fused
    pass gives the same bits.  With `batch`, the GPU folds the arrivals after
    the first `single_first` in calls of up to `batch` arrivals each
    (dl_fold_checkpoints, and with `fused_last` the last call also closes);
    the oracle still folds one arrival at a time."""
    cks_gpu = worker_inputs(w, rnd, st.theta, st.g_theta.device)
    cks_np = {i: to_np(c) for i, c in cks_gpu.items()}
    offs = list(w.frag_offsets)
    tag = 1000 + rnd
    if orders is None:
        orders = [participants(w, rnd, f, exactly_quorum) for f in range(w.n_frags)]
    orc = oracle.load()

    if w.mode == "mean":
        # ---- GPU ----
        r = dl.dl_round_begin(tag, dl.DL_MEAN, w.n_params, offs, w.quorum, w.workers, st.g_acc,
                              stream=stream)
        try:
            for f in range(w.n_frags):
                o0, o1 = offs[f], offs[f + 1]
                for kind, ids in _calls(orders[f], fused_last, batch, single_first):
                    cks = [cks_gpu[i][o0:o1] for i in ids]
                    if kind == "one":
                        dl.dl_fold_checkpoint(r, f, ids[0], tag, cks[0])
                    elif kind == "many":
                        dl.dl_fold_checkpoints(r, f, ids, tag, cks)
                    elif kind == "one_close":
                        dl.dl_fold_and_finalize_mean(r, f, ids[0], tag, cks[0], st.g_theta,
                                                     st.g_e, w.beta)
                    elif kind == "many_close":
                        dl.dl_fold_checkpoints_and_finalize_mean(r, f, ids, tag, cks, st.g_theta,
                                                                 st.g_e, w.beta)
                    else:
                        dl.dl_finalize_mean(r, f, st.g_theta, st.g_e, w.beta)
            parts = [dl.dl_round_participants(r, f) for f in range(w.n_frags)]
        finally:
            dl.dl_round_end(r)
        # ---- oracle ----
        for f in range(w.n_frags):
            o0, o1 = offs[f], offs[f + 1]
            g = orc.mean_round([np.ascontiguousarray(cks_np[i][o0:o1]) for i in orders[f]],
                               ema=None if st.e is None else st.e[o0:o1], beta=w.beta)
            st.theta[o0:o1] = g
    else:
        tokens = synth.token_counts(w, rnd)
        r = dl.dl_round_begin(tag, dl.DL_DELTA_NESTEROV, w.n_params, offs, w.quorum, w.workers,
                              st.g_acc, stream=stream)
        try:
            for f in range(w.n_frags):
                o0, o1 = offs[f], offs[f + 1]
                for kind, ids in _calls(orders[f], fused_last, batch, single_first):
                    cks = [cks_gpu[i][o0:o1] for i in ids]
                    tok = [tokens[i] for i in ids]
                    if kind == "one":
                        dl.dl_fold_checkpoint(r, f, ids[0], tag, cks[0], st.g_theta, tok[0])
                    elif kind == "many":
                        dl.dl_fold_checkpoints(r, f, ids, tag, cks, st.g_theta, tok)
                    elif kind == "one_close":
                        dl.dl_fold_and_outer_nesterov(r, f, ids[0], tag, cks[0], tok[0],
                                                      st.g_theta, st.g_m, w.lr, w.mu, st.g_e,
                                                      w.beta)
                    elif kind == "many_close":
                        dl.dl_fold_checkpoints_and_outer_nesterov(r, f, ids, tag, cks, tok,
                                                                  st.g_theta, st.g_m, w.lr, w.mu,
                                                                  st.g_e, w.beta)
                    else:
                        dl.dl_outer_nesterov(r, f, st.g_theta, st.g_m, w.lr, w.mu, st.g_e, w.beta)
                assert dl.dl_round_tokens(r, f) == sum(tokens[i] for i in orders[f])
            parts = [dl.dl_round_participants(r, f) for f in range(w.n_frags)]
        finally:
            dl.dl_round_end(r)
        for f in range(w.n_frags):
            o0, o1 = offs[f], offs[f + 1]
            orc.nesterov_fragment_round(
                st.theta[o0:o1], st.m[o0:o1],
                [np.ascontiguousarray(cks_np[i][o0:o1]) for i in orders[f]],
                [tokens[i] for i in orders[f]], w.lr, w.mu,
                None if st.e is None else st.e[o0:o1], w.beta)
    torch.cuda.synchronize()
    assert parts == [list(o) for o in orders]
    out = {"theta": (to_np(st.g_theta), st.theta)}
    if st.g_m is not None:
        out["m"] = (to_np(st.g_m), st.m)
    if st.g_e is not None:
        out["e"] = (to_np(st.g_e), st.e)
    return out


def assert_round_equal(res: dict, what: str) -> None:
    for k, (g, o) in res.items():
        assert bits_equal(g, o), f"{what}: {k}: {first_mismatch(g, o)}"
