"""A merge workload resident on the GPU, and one merge round of it issued
through the C ABI.

The benchmark times `GpuWorkload.run_round`; the full-size parity tests run
the very same calls.  Inputs come from the seeded generator
(checkpoint_averaging_amd.synth): the initial global, and for round r the
worker checkpoints c_i = global0 + drift(r, i), generated on the GPU before the
round starts (never inside a timed region).

Round structure (all on torch's current stream):
* plain mean:      for each fragment, fold every worker in its seeded arrival
                   order, then close the fragment with the mean (+ EMA).
                   The mean is written over the running sum (out == acc),
                   and after the round the two buffers swap roles: the sum's
                   buffer is the new global, the old global's the next
                   round's accumulator.  The mean round never reads the old
                   global, so this only changes where the result lands.  The
                   close then writes lines it has just read.  At 1.08B
                   elements that ran 6-8% faster on MI355X than writing the
                   mean to a buffer the pass does not read (75% against 70-71%
                   of 8 TB/s).
* delta Nesterov:  for each fragment, fold every worker's token-weighted delta
                   in arrival order, then close with the outer Nesterov step
                   (+ EMA)
* batched:         every checkpoint of the round is already resident, so each
                   fragment's arrivals go to the library in one call (still in
                   arrival order) and the fragment's whole merge is one pass
                   that reads each buffer once
"""
from __future__ import annotations

import ctypes
import struct
from typing import Callable, Dict, List, Optional

import torch

from . import dlmerge as dl
from . import synth

_GEN_CHUNK = 1 << 25
_HIP = None


def _hip():
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipMemsetD32Async.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t,
                                           ctypes.c_void_p]
        _HIP.hipMemsetD16Async.argtypes = [ctypes.c_void_p, ctypes.c_ushort, ctypes.c_size_t,
                                           ctypes.c_void_p]
    return _HIP


def _runtime_fill(t: torch.Tensor, value: float) -> None:
    """Fills t with one constant through the HIP runtime's own memset on
    torch's current stream: no torch kernel is launched (for runs under a
    counter-collecting profiler, whose host side crashed on one of torch's
    kernel launches)."""
    bits = struct.unpack("<I", struct.pack("<f", value))[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if t.dtype == torch.bfloat16:
        st = _hip().hipMemsetD16Async(t.data_ptr(), bits >> 16, t.numel(), stream)
    else:
        st = _hip().hipMemsetD32Async(t.data_ptr(), ctypes.c_int(bits - (1 << 32)
                                                                  if bits >= 1 << 31 else bits),
                                      t.numel(), stream)
    if st != 0:
        raise RuntimeError(f"hipMemset failed ({st})")


class GpuWorkload:
    """fill="philox": the seeded generator's values (parity tests, the
    benchmark).  fill="runtime": constants written by the HIP runtime's
    memset, so that the process launches no torch kernel (counter runs; the
    merge's timing and traffic do not depend on the values)."""

    def __init__(self, w: synth.Workload, device="cuda", close_in_place: bool = True,
                 fill: str = "philox"):
        if fill not in ("philox", "runtime"):
            raise ValueError(fill)
        self.w = w
        self.close_in_place = close_in_place
        self.fill = fill
        self.dev = torch.device(device)
        n = w.n_params
        self.delta = w.mode == "delta_nesterov"
        f32 = dict(dtype=torch.float32, device=self.dev)
        if fill == "philox":
            self.theta = synth.global0(w.seed, n, device=self.dev)
            self.m = torch.zeros(n, **f32) if self.delta else None
            self.e = self.theta.clone() if w.ema else None
        else:
            self.theta = torch.empty(n, **f32)
            _runtime_fill(self.theta, 0.02)
            self.m = torch.empty(n, **f32) if self.delta else None
            if self.m is not None:
                _runtime_fill(self.m, 0.0)
            self.e = torch.empty(n, **f32) if w.ema else None
            if self.e is not None:
                _runtime_fill(self.e, 0.02)
        self.acc = torch.empty(n, **f32)
        cdt = torch.bfloat16 if w.ckpt_dtype == "bf16" else torch.float32
        self.ckpts: List[torch.Tensor] = [torch.empty(n, dtype=cdt, device=self.dev)
                                          for _ in range(w.workers)]
        self.ckpt_round = None

    def generate_checkpoints(self, rnd: int) -> None:
        """Worker checkpoints of round rnd: global0 + seeded drift (chunked so
        the generator's temporaries stay small)."""
        w, n = self.w, self.w.n_params
        if self.fill == "runtime":
            for i, c in enumerate(self.ckpts):
                _runtime_fill(c, 0.02 + 1e-3 * (i + 1))
            self.ckpt_round = rnd
            return
        for s in range(0, n, _GEN_CHUNK):
            c = min(_GEN_CHUNK, n - s)
            th0 = synth.global0(w.seed, c, device=self.dev, start=s)
            for i in range(w.workers):
                synth.worker_checkpoint(w.seed, rnd, i, th0, start=s, dtype=w.ckpt_dtype,
                                        out=self.ckpts[i][s:s + c])
            del th0
        self.ckpt_round = rnd

    def orders(self, rnd: int) -> List[List[int]]:
        return [synth.arrival_order(self.w, rnd, f) for f in range(self.w.n_frags)]

    def tokens(self, rnd: int) -> List[int]:
        return synth.token_counts(self.w, rnd)

    def run_round(self, rnd: int, tag: int,
                  timer: Optional[Callable[[str, int, Callable[[], None]], None]] = None,
                  fused_close: bool = True,
                  streams: Optional[List[torch.cuda.Stream]] = None,
                  batched: bool = False) -> None:
        """Issue one merge round.  `timer(kind, elements, call)` (if given)
        wraps every kernel-launching call, e.g. to record events around it.

        With `fused_close`, the fragment's last expected arrival is folded and
        the fragment closed in one pass (the merger closes as soon as every
        worker of the round is in); otherwise the close is a separate pass.

        With `streams`, every fragment's round is its own handle on its own
        stream (fragment f on streams[f % len(streams)]), so the fragments'
        rounds are in flight together; they touch disjoint element ranges.
        The streams wait for the caller's stream first and the caller's
        stream waits for all of them at the end.  With `batched` too, each
        fragment's arrivals go in one call on the fragment's stream.

        With `batched`, each fragment's arrivals are passed in one
        several-arrival call (dl_fold_checkpoints_and_*, or
        dl_fold_checkpoints and a separate close): same results, bit for bit,
        in one pass per fragment."""
        if streams:
            self._run_round_streams(rnd, tag, timer, fused_close, streams, batched)
            return
        if batched:
            self._run_round_batched(rnd, tag, timer, fused_close)
            return
        w = self.w
        offs = list(w.frag_offsets)
        orders = self.orders(rnd)
        run = timer if timer is not None else (lambda kind, n, call: call())
        ema = "_ema" if self.e is not None else ""
        if not self.delta:
            out = self.acc if self.close_in_place else self.theta
            r = dl.dl_round_begin(tag, dl.DL_MEAN, w.n_params, offs, w.quorum, w.workers,
                                  self.acc)
            try:
                for f in range(w.n_frags):
                    o0, o1 = offs[f], offs[f + 1]
                    order = orders[f]
                    folds = order[:-1] if fused_close else order
                    for k, i in enumerate(folds):
                        ck = self.ckpts[i][o0:o1]
                        run("fold_first" if k == 0 else "fold", o1 - o0,
                            lambda f=f, i=i, ck=ck: dl.dl_fold_checkpoint(r, f, i, tag, ck))
                    if fused_close:
                        i = order[-1]
                        ck = self.ckpts[i][o0:o1]
                        kind = "fold_finalize_mean" + ema + ("_first" if not folds else "")
                        run(kind, o1 - o0, lambda f=f, i=i, ck=ck: dl.dl_fold_and_finalize_mean(
                            r, f, i, tag, ck, out, self.e, w.beta))
                    else:
                        run("finalize_mean" + ema, o1 - o0,
                            lambda f=f: dl.dl_finalize_mean(r, f, out, self.e, w.beta))
            finally:
                dl.dl_round_end(r)
            self._swap_if_in_place()
        else:
            tok = self.tokens(rnd)
            r = dl.dl_round_begin(tag, dl.DL_DELTA_NESTEROV, w.n_params, offs, w.quorum,
                                  w.workers, self.acc)
            try:
                for f in range(w.n_frags):
                    o0, o1 = offs[f], offs[f + 1]
                    order = orders[f]
                    folds = order[:-1] if fused_close else order
                    for k, i in enumerate(folds):
                        ck = self.ckpts[i][o0:o1]
                        run("fold_delta_first" if k == 0 else "fold_delta", o1 - o0,
                            lambda f=f, i=i, ck=ck:
                            dl.dl_fold_checkpoint(r, f, i, tag, ck, self.theta, tok[i]))
                    if fused_close:
                        i = order[-1]
                        ck = self.ckpts[i][o0:o1]
                        kind = "fold_nesterov" + ema + ("_first" if not folds else "")
                        run(kind, o1 - o0, lambda f=f, i=i, ck=ck: dl.dl_fold_and_outer_nesterov(
                            r, f, i, tag, ck, tok[i], self.theta, self.m, w.lr, w.mu, self.e,
                            w.beta))
                    else:
                        run("nesterov" + ema, o1 - o0,
                            lambda f=f: dl.dl_outer_nesterov(r, f, self.theta, self.m, w.lr,
                                                             w.mu, self.e, w.beta))
            finally:
                dl.dl_round_end(r)


    def _fragment_batched(self, r, f, tag, order, tok, out, run, ema, fused_close):
        """Fragment f's arrivals in one several-arrival call on torch's
        current stream (and the close, when it is not fused)."""
        w = self.w
        o0, o1 = w.frag_offsets[f], w.frag_offsets[f + 1]
        ids = list(order)
        cks = [self.ckpts[i][o0:o1] for i in ids]
        if not self.delta:
            if fused_close:
                run("fold_all_finalize_mean" + ema, o1 - o0,
                    lambda: dl.dl_fold_checkpoints_and_finalize_mean(r, f, ids, tag, cks, out,
                                                                     self.e, w.beta))
            else:
                run("fold_all", o1 - o0, lambda: dl.dl_fold_checkpoints(r, f, ids, tag, cks))
                run("finalize_mean" + ema, o1 - o0,
                    lambda: dl.dl_finalize_mean(r, f, out, self.e, w.beta))
        else:
            t = [tok[i] for i in ids]
            if fused_close:
                run("fold_all_nesterov" + ema, o1 - o0,
                    lambda: dl.dl_fold_checkpoints_and_outer_nesterov(
                        r, f, ids, tag, cks, t, self.theta, self.m, w.lr, w.mu, self.e, w.beta))
            else:
                run("fold_delta_all", o1 - o0,
                    lambda: dl.dl_fold_checkpoints(r, f, ids, tag, cks, self.theta, t))
                run("nesterov" + ema, o1 - o0,
                    lambda: dl.dl_outer_nesterov(r, f, self.theta, self.m, w.lr, w.mu, self.e,
                                                 w.beta))

    def _run_round_batched(self, rnd, tag, timer, fused_close):
        w = self.w
        orders = self.orders(rnd)
        run = timer if timer is not None else (lambda kind, n, call: call())
        ema = "_ema" if self.e is not None else ""
        mode = dl.DL_DELTA_NESTEROV if self.delta else dl.DL_MEAN
        out = self.acc if self.close_in_place else self.theta
        tok = self.tokens(rnd) if self.delta else None
        r = dl.dl_round_begin(tag, mode, w.n_params, list(w.frag_offsets), w.quorum, w.workers,
                              self.acc)
        try:
            for f in range(w.n_frags):
                self._fragment_batched(r, f, tag, orders[f], tok, out, run, ema, fused_close)
        finally:
            dl.dl_round_end(r)
        self._swap_if_in_place()

    def _swap_if_in_place(self) -> None:
        """After a mean round closed in place, the accumulator holds the new
        global: the buffers swap roles."""
        if not self.delta and self.close_in_place:
            self.theta, self.acc = self.acc, self.theta

    def _run_round_streams(self, rnd, tag, timer, fused_close, streams, batched=False):
        w = self.w
        offs = list(w.frag_offsets)
        orders = self.orders(rnd)
        tok = self.tokens(rnd)
        run = timer if timer is not None else (lambda kind, n, call: call())
        ema = "_ema" if self.e is not None else ""
        cur = torch.cuda.current_stream()
        start = torch.cuda.Event()
        start.record(cur)
        mode = dl.DL_DELTA_NESTEROV if self.delta else dl.DL_MEAN
        out = self.acc if self.close_in_place else self.theta
        handles = []
        try:
            for f in range(w.n_frags):
                st = streams[f % len(streams)]
                st.wait_event(start)
                handles.append(dl.dl_round_begin(tag, mode, w.n_params, offs, w.quorum,
                                                 w.workers, self.acc, stream=st))
            if batched:
                for f in range(w.n_frags):
                    with torch.cuda.stream(streams[f % len(streams)]):
                        self._fragment_batched(handles[f], f, tag, orders[f], tok, out, run, ema,
                                               fused_close)
            # issue arrivals round-robin across fragments, as they would come
            for k in range(0 if batched else w.workers):
                for f in range(w.n_frags):
                    st = streams[f % len(streams)]
                    r = handles[f]
                    o0, o1 = offs[f], offs[f + 1]
                    i = orders[f][k]
                    ck = self.ckpts[i][o0:o1]
                    last = k == w.workers - 1
                    with torch.cuda.stream(st):
                        if not self.delta:
                            if last and fused_close:
                                kind = "fold_finalize_mean" + ema + ("_first" if k == 0 else "")
                                run(kind, o1 - o0, lambda: dl.dl_fold_and_finalize_mean(
                                    r, f, i, tag, ck, out, self.e, w.beta))
                            else:
                                run("fold_first" if k == 0 else "fold", o1 - o0,
                                    lambda: dl.dl_fold_checkpoint(r, f, i, tag, ck))
                                if last:
                                    run("finalize_mean" + ema, o1 - o0,
                                        lambda: dl.dl_finalize_mean(r, f, out, self.e, w.beta))
                        else:
                            if last and fused_close:
                                kind = "fold_nesterov" + ema + ("_first" if k == 0 else "")
                                run(kind, o1 - o0, lambda: dl.dl_fold_and_outer_nesterov(
                                    r, f, i, tag, ck, tok[i], self.theta, self.m, w.lr, w.mu,
                                    self.e, w.beta))
                            else:
                                run("fold_delta_first" if k == 0 else "fold_delta", o1 - o0,
                                    lambda: dl.dl_fold_checkpoint(r, f, i, tag, ck, self.theta,
                                                                  tok[i]))
                                if last:
                                    run("nesterov" + ema, o1 - o0,
                                        lambda: dl.dl_outer_nesterov(r, f, self.theta, self.m,
                                                                     w.lr, w.mu, self.e, w.beta))
        finally:
            for r in handles:
                dl.dl_round_end(r)
        for st in streams:
            done = torch.cuda.Event()
            done.record(st)
            cur.wait_event(done)
        self._swap_if_in_place()


def algorithmic_bytes(w: synth.Workload, fused_close: bool = False) -> Dict[str, int]:
    """Bytes each kernel kind must move per element, and per round in total.

    Each arriving checkpoint is read once; the accumulator is read and written
    per arrival except the first, which only writes it; the delta fold also
    reads the global; the close reads and writes each state buffer once, with
    the EMA fused in.  This is the round with a separate close (`per_param`,
    `per_round`).  With `fused_close` the last arrival's fold and the close
    share one pass, which moves fewer bytes (`per_param_fused`)."""
    cb = 2 if w.ckpt_dtype == "bf16" else 4
    per_elem = {
        "fold_first": cb + 4, "fold": cb + 8,
        "fold_delta_first": cb + 8, "fold_delta": cb + 12,
        "finalize_mean": 8, "finalize_mean_ema": 16,
        "nesterov": 20, "nesterov_ema": 28,
        # last arrival folded and the fragment closed in one pass
        "fold_finalize_mean": cb + 8, "fold_finalize_mean_ema": cb + 16,
        "fold_finalize_mean_first": cb + 4, "fold_finalize_mean_ema_first": cb + 12,
        "fold_nesterov": cb + 20, "fold_nesterov_ema": cb + 28,
        "fold_nesterov_first": cb + 16, "fold_nesterov_ema_first": cb + 24,
        "ema": 12,
    }
    # every arrival of the fragment in one call (k = all workers): each
    # checkpoint read once, the accumulator written once (not at all when the
    # same pass closes), the state buffers read and written once
    k = w.workers
    per_elem.update({
        "fold_all": k * cb + 4, "fold_delta_all": k * cb + 8,
        "fold_all_finalize_mean": k * cb + 4, "fold_all_finalize_mean_ema": k * cb + 12,
        "fold_all_nesterov": k * cb + 16, "fold_all_nesterov_ema": k * cb + 24,
    })
    ema = "_ema" if w.ema else ""
    if w.mode == "mean":
        first, fold, close, fused = "fold_first", "fold", "finalize_mean", "fold_finalize_mean"
    else:
        first, fold, close, fused = ("fold_delta_first", "fold_delta", "nesterov",
                                     "fold_nesterov")
    per_param = per_elem[first] + (w.workers - 1) * per_elem[fold] + per_elem[close + ema]
    if w.workers > 1:
        per_param_fused = (per_elem[first] + (w.workers - 2) * per_elem[fold]
                           + per_elem[fused + ema])
    else:
        per_param_fused = per_elem[fused + ema + "_first"]
    batched = "fold_all_finalize_mean" if w.mode == "mean" else "fold_all_nesterov"
    per_param_batched = per_elem[batched + ema]
    fold_all = "fold_all" if w.mode == "mean" else "fold_delta_all"
    per_param_batched_separate = per_elem[fold_all] + per_elem[close + ema]
    return {"per_elem": per_elem, "per_param": per_param, "per_round": per_param * w.n_params,
            "per_param_fused": per_param_fused,
            "per_round_fused": per_param_fused * w.n_params,
            "per_param_batched": per_param_batched,
            "per_round_batched": per_param_batched * w.n_params,
            "per_param_batched_separate": per_param_batched_separate,
            "per_round_batched_separate": per_param_batched_separate * w.n_params}
