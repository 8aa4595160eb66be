"""ctypes wrapper over the C oracle (dl_oracle.c) and the round drivers that
apply its steps in the order the pages give.

TEST INFRASTRUCTURE ONLY: never imported by the product library.  Arrays are
numpy: float32 for fp32 data, uint16 holding the bit patterns for bf16 data.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

F32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdloracle.so")


def _f32(a: np.ndarray, name: str) -> np.ndarray:
    if not isinstance(a, np.ndarray) or a.dtype != np.float32 or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a contiguous float32 array")
    return a


def _ckpt_dtype(c: np.ndarray) -> int:
    if not c.flags.c_contiguous:
        raise TypeError("checkpoint must be contiguous")
    if c.dtype == np.float32:
        return F32
    if c.dtype == np.uint16:
        return BF16
    raise TypeError("checkpoint must be float32 or uint16 (bf16 bits)")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


class Oracle:
    """The oracle's steps bound to one build of dl_oracle.c."""

    def __init__(self, path: str = LIB_PATH):
        lib = ctypes.CDLL(path)
        p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.oracle_fold_mean.argtypes = [p, p, i32, i64, i32]
        lib.oracle_finalize_mean.argtypes = [p, p, i64, i32, p, f32]
        lib.oracle_fold_delta.argtypes = [p, p, p, i32, i64, i64, i32]
        lib.oracle_outer_nesterov.argtypes = [p, p, p, i64, i64, f32, f32, p, f32]
        lib.oracle_ema.argtypes = [p, p, i64, f32]
        lib.oracle_adopt_keep_drift.argtypes = [p, p, p, i32, i64]
        lib.oracle_threads.restype = i32
        lib.oracle_set_threads.argtypes = [i32]
        for name in ("oracle_fold_mean", "oracle_finalize_mean", "oracle_fold_delta",
                     "oracle_outer_nesterov", "oracle_ema", "oracle_adopt_keep_drift",
                     "oracle_set_threads"):
            getattr(lib, name).restype = None
        self.lib = lib
        self.path = path

    # -- single steps -------------------------------------------------------

    def fold_mean(self, acc: np.ndarray, ckpt: np.ndarray, first: bool) -> None:
        """Running-sum fold of one arriving checkpoint (in place on acc)."""
        _f32(acc, "acc")
        if ckpt.size != acc.size:
            raise ValueError("size mismatch")
        self.lib.oracle_fold_mean(_ptr(acc), _ptr(ckpt), _ckpt_dtype(ckpt), acc.size,
                                  int(bool(first)))

    def finalize_mean(self, out: np.ndarray, acc: np.ndarray, count: int,
                      ema: Optional[np.ndarray] = None, beta: float = 0.9) -> None:
        """global = acc / count, then the optional EMA step (out may be acc)."""
        _f32(out, "out"), _f32(acc, "acc")
        if out.size != acc.size or (ema is not None and _f32(ema, "ema").size != acc.size):
            raise ValueError("size mismatch")
        self.lib.oracle_finalize_mean(_ptr(out), _ptr(acc), acc.size, int(count), _ptr(ema),
                                      float(beta))

    def fold_delta(self, acc: np.ndarray, theta: np.ndarray, ckpt: np.ndarray, tokens: int,
                   first: bool) -> None:
        """Token-weighted delta fold of one arriving fragment snapshot."""
        _f32(acc, "acc"), _f32(theta, "theta")
        if ckpt.size != acc.size or theta.size != acc.size:
            raise ValueError("size mismatch")
        self.lib.oracle_fold_delta(_ptr(acc), _ptr(theta), _ptr(ckpt), _ckpt_dtype(ckpt),
                                   acc.size, int(tokens), int(bool(first)))

    def outer_nesterov(self, theta: np.ndarray, m: np.ndarray, acc: np.ndarray,
                       total_tokens: int, lr: float, mu: float,
                       ema: Optional[np.ndarray] = None, beta: float = 0.9) -> None:
        """Outer Nesterov step on one fragment (theta, m, ema updated in place)."""
        _f32(theta, "theta"), _f32(m, "m"), _f32(acc, "acc")
        if theta.size != acc.size or m.size != acc.size or \
                (ema is not None and _f32(ema, "ema").size != acc.size):
            raise ValueError("size mismatch")
        self.lib.oracle_outer_nesterov(_ptr(theta), _ptr(m), _ptr(acc), acc.size,
                                       int(total_tokens), float(lr), float(mu), _ptr(ema),
                                       float(beta))

    def ema_update(self, ema: np.ndarray, g: np.ndarray, beta: float = 0.9) -> None:
        _f32(ema, "ema"), _f32(g, "g")
        if ema.size != g.size:
            raise ValueError("size mismatch")
        self.lib.oracle_ema(_ptr(ema), _ptr(g), ema.size, float(beta))

    def adopt_keep_drift(self, theta: np.ndarray, g: np.ndarray, pushed: np.ndarray) -> None:
        """Worker-side adoption that keeps local drift: theta += (g - pushed)."""
        _f32(theta, "theta"), _f32(g, "g")
        if g.size != theta.size or pushed.size != theta.size:
            raise ValueError("size mismatch")
        self.lib.oracle_adopt_keep_drift(_ptr(theta), _ptr(g), _ptr(pushed), _ckpt_dtype(pushed),
                                         theta.size)

    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    # -- round drivers: the steps above in the order the pages give ---------

    def mean_round(self, ckpts_in_arrival_order: Sequence[np.ndarray],
                   ema: Optional[np.ndarray] = None, beta: float = 0.9) -> np.ndarray:
        """One plain-replacement round: fold every arrival into a running fp32
        sum in arrival order, divide by the number of arrivals, then advance
        the EMA of globals if one is given."""
        if len(ckpts_in_arrival_order) == 0:
            raise ValueError("a round needs at least one checkpoint")
        acc = np.empty(ckpts_in_arrival_order[0].size, dtype=np.float32)
        for k, c in enumerate(ckpts_in_arrival_order):
            self.fold_mean(acc, c, first=(k == 0))
        self.finalize_mean(acc, acc, len(ckpts_in_arrival_order), ema, beta)
        return acc

    def nesterov_fragment_round(self, theta: np.ndarray, m: np.ndarray,
                                ckpts_in_arrival_order: Sequence[np.ndarray],
                                tokens_in_arrival_order: Sequence[int], lr: float, mu: float,
                                ema: Optional[np.ndarray] = None, beta: float = 0.9) -> None:
        """One fragment round of the token-weighted delta merge followed by the
        outer Nesterov step; theta, m and ema are that fragment's slices and
        are updated in place."""
        if len(ckpts_in_arrival_order) == 0:
            raise ValueError("a round needs at least one snapshot")
        if len(ckpts_in_arrival_order) != len(tokens_in_arrival_order):
            raise ValueError("one token count per snapshot")
        acc = np.empty(theta.size, dtype=np.float32)
        for k, (c, t) in enumerate(zip(ckpts_in_arrival_order, tokens_in_arrival_order)):
            self.fold_delta(acc, theta, c, int(t), first=(k == 0))
        self.outer_nesterov(theta, m, acc, sum(int(t) for t in tokens_in_arrival_order),
                            lr, mu, ema, beta)

    # -- side averages (technical report, "Training system", Table 2, row
    # "Side averages"; "Data and schedule": the published model is an
    # equal-weight average of the globals committed in the final stretch;
    # "The final stretch", Table 5: averages of the last 3 and 5 snapshots) --

    def swa_average(self, globals_in_commit_order: Sequence[np.ndarray]) -> np.ndarray:
        """Uniform average of globals: a plain mean, the globals added to an
        fp32 running sum in the order they were committed."""
        return self.mean_round(globals_in_commit_order)

    def snapshot_average(self, snapshots_oldest_first: Sequence[np.ndarray]) -> np.ndarray:
        """Average of the last k snapshots: their plain mean, summed oldest
        first."""
        return self.mean_round(snapshots_oldest_first)


_default: Optional[Oracle] = None


def load() -> Oracle:
    """The oracle built from oracle/dl_oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _default = Oracle(LIB_PATH)
    return _default


def fold_mean(*a, **k):
    return load().fold_mean(*a, **k)


def finalize_mean(*a, **k):
    return load().finalize_mean(*a, **k)


def fold_delta(*a, **k):
    return load().fold_delta(*a, **k)


def outer_nesterov(*a, **k):
    return load().outer_nesterov(*a, **k)


def ema_update(*a, **k):
    return load().ema_update(*a, **k)


def mean_round(*a, **k):
    return load().mean_round(*a, **k)


def nesterov_fragment_round(*a, **k):
    return load().nesterov_fragment_round(*a, **k)


def swa_average(*a, **k):
    return load().swa_average(*a, **k)


def adopt_keep_drift(*a, **k):
    return load().adopt_keep_drift(*a, **k)


def snapshot_average(*a, **k):
    return load().snapshot_average(*a, **k)


def threads() -> int:
    return load().threads()


def set_threads(n: int) -> None:
    load().set_threads(n)
