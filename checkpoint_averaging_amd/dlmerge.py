"""ctypes binding of libdlmerge.so (C ABI in include/dlmerge.h).

Argument marshalling only: torch tensors become (device pointer, dtype), the
stream defaults to torch's current stream, and a negative status becomes a
DLError.  Every step of the merge runs in the library's HIP kernels; there is
no fallback, and importing this module raises if the library is not built.

Function names and arguments mirror the C functions.  An array argument is a
torch tensor on the GPU or, for tests that need exact pointers, a plain
integer device address (then ``dtype`` must be given where it matters).
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdlmerge.so")

DL_MEAN = 0
DL_DELTA_NESTEROV = 1
DL_F32 = 0
DL_BF16 = 1

DL_OK = 0
DL_E_INVAL = -1
DL_E_STALE = -2
DL_E_DUP = -3
DL_E_QUORUM = -4
DL_E_STATE = -5
DL_E_ALIGN = -6
DL_E_HIP = -7
DL_E_CAPACITY = -8
DL_E_NOMEM = -9
DL_E_TOO_LARGE = -10
DL_NOALLOC_SCRATCH_BYTES = 192 << 20

SYMBOLS = ("dl_round_begin", "dl_fold_checkpoint", "dl_finalize_mean", "dl_outer_nesterov",
           "dl_fold_and_finalize_mean", "dl_fold_and_outer_nesterov",
           "dl_fold_checkpoints", "dl_fold_checkpoints_and_finalize_mean",
           "dl_fold_checkpoints_and_outer_nesterov",
           "dl_ema_update", "dl_swa_fold", "dl_swa_average", "dl_snapshot_average",
           "dl_adopt_keep_drift", "dl_polar_workspace_bytes", "dl_polar_workspace_bytes_batch",
           "dl_polar_factor", "dl_outer_orthogonal_step", "dl_outer_orthogonal_step_batch",
           "dl_outer_orthogonal_step_noalloc",
           "dl_matmul_workspace_bytes", "dl_matmul_f32",
           "dl_matmul_workspace_bytes_batch", "dl_matmul_f32_batch", "dl_matmul_large_tiles",
           "dl_frag_range", "dl_round_participants", "dl_round_tokens",
           "dl_round_end", "dl_strerror")
DL_MAX_SNAPSHOTS = 16
DL_MAX_BATCH = 64
DL_TN = 0
DL_NT = 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m checkpoint_averaging_amd.build` "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)
_p, _i32, _i64, _u64, _f32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                              ctypes.c_float)
_lib.dl_round_begin.argtypes = [ctypes.POINTER(_p), _u64, _i32, _i64, _i32,
                                ctypes.POINTER(_i64), _i32, _i32, _p, _p]
_lib.dl_fold_checkpoint.argtypes = [_p, _i32, _i32, _u64, _p, _i32, _p, _i64]
_lib.dl_finalize_mean.argtypes = [_p, _i32, _p, _p, _f32]
_lib.dl_outer_nesterov.argtypes = [_p, _i32, _p, _p, _f32, _f32, _p, _f32]
_lib.dl_fold_and_finalize_mean.argtypes = [_p, _i32, _i32, _u64, _p, _i32, _p, _p, _f32]
_lib.dl_fold_and_outer_nesterov.argtypes = [_p, _i32, _i32, _u64, _p, _i32, _i64, _p, _p, _f32,
                                            _f32, _p, _f32]
_lib.dl_fold_checkpoints.argtypes = [_p, _i32, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_u64),
                                     ctypes.POINTER(_p), _i32, _p, ctypes.POINTER(_i64)]
_lib.dl_fold_checkpoints_and_finalize_mean.argtypes = [_p, _i32, _i32, ctypes.POINTER(_i32),
                                                       ctypes.POINTER(_u64), ctypes.POINTER(_p),
                                                       _i32, _p, _p, _f32]
_lib.dl_fold_checkpoints_and_outer_nesterov.argtypes = [_p, _i32, _i32, ctypes.POINTER(_i32),
                                                        ctypes.POINTER(_u64), ctypes.POINTER(_p),
                                                        _i32, ctypes.POINTER(_i64), _p, _p, _f32,
                                                        _f32, _p, _f32]
_lib.dl_ema_update.argtypes = [_p, _p, _i64, _f32, _p]
_lib.dl_swa_fold.argtypes = [_p, _p, _i64, _i64, _p]
_lib.dl_swa_average.argtypes = [_p, _p, _i64, _i64, _p]
_lib.dl_snapshot_average.argtypes = [_p, ctypes.POINTER(_p), _i32, _i64, _p]
_lib.dl_adopt_keep_drift.argtypes = [_p, _p, _p, _i32, _i64, _p]
_lib.dl_polar_workspace_bytes.argtypes = [_i64, _i64, ctypes.POINTER(_i64)]
_lib.dl_polar_workspace_bytes_batch.argtypes = [_i64, _i64, _i32, ctypes.POINTER(_i64)]
_lib.dl_polar_factor.argtypes = [_p, _p, _i64, _i64, _i32, _i32, _p, _i64, _p]
_lib.dl_outer_orthogonal_step_batch.argtypes = [ctypes.POINTER(_p), ctypes.POINTER(_p), _i32,
                                                _i64, _i64, _f32, _i32, _i32, _p, _i64, _p]
_lib.dl_outer_orthogonal_step.argtypes = [_p, _p, _i64, _i64, _f32, _i32, _i32, _p, _i64, _p]
_lib.dl_outer_orthogonal_step_noalloc.argtypes = [_p, _p, _i64, _i64, _f32, _i32, _i32, _p]
_lib.dl_matmul_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, ctypes.POINTER(_i64)]
_lib.dl_matmul_workspace_bytes_batch.argtypes = [_i64, _i64, _i64, _i32, _i32,
                                                 ctypes.POINTER(_i64)]
_lib.dl_matmul_large_tiles.argtypes = [_i64, _i64, _i64, _i32, _i32, _i64,
                                       ctypes.POINTER(_i32)]
_lib.dl_matmul_f32_batch.argtypes = [_i32, _p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _i64, _p,
                                     _i64, _i64, _p, _i64, _f32, _f32, _f32, _i32, _i32, _p, _i64,
                                     _p]
_lib.dl_matmul_f32.argtypes = [_i32, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64, _p, _f32,
                               _f32, _f32, _i32, _p, _i64, _p]
_lib.dl_frag_range.argtypes = [_p, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
_lib.dl_round_participants.argtypes = [_p, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32), _i32]
_lib.dl_round_tokens.argtypes = [_p, _i32, ctypes.POINTER(_i64)]
_lib.dl_round_end.argtypes = [_p]
_lib.dl_strerror.argtypes = [_i32]
_lib.dl_strerror.restype = ctypes.c_char_p
for _name in SYMBOLS[:-1]:
    getattr(_lib, _name).restype = _i32


class DLError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {dl_strerror(status)} ({status})")


def _check(status: int, call: str) -> None:
    if status != DL_OK:
        raise DLError(status, call)


Array = Union[torch.Tensor, int, None]


def _addr(a: Array) -> Optional[int]:
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        if not a.is_cuda:
            raise TypeError("device tensor required")
        if not a.is_contiguous():
            raise TypeError("contiguous tensor required")
        return a.data_ptr()
    return int(a)


def _f32_addr(a: Array, name: str) -> Optional[int]:
    if isinstance(a, torch.Tensor) and a.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return _addr(a)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def dl_strerror(status: int) -> str:
    return _lib.dl_strerror(int(status)).decode()


class Round:
    """Handle of an open round (wraps the C dl_round pointer)."""

    def __init__(self, handle: ctypes.c_void_p, n_frags: int):
        self._h = handle
        self.n_frags = n_frags

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("round already ended")
        return self._h

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        dl_round_end(self)


def dl_round_begin(round_tag: int, mode: int, n_params: int, frag_offsets: Sequence[int],
                   quorum: int, max_workers: int, acc: Array, stream=None) -> Round:
    offs = (_i64 * len(frag_offsets))(*[int(o) for o in frag_offsets])
    h = _p()
    _check(_lib.dl_round_begin(ctypes.byref(h), int(round_tag), int(mode), int(n_params),
                               len(frag_offsets) - 1, offs, int(quorum), int(max_workers),
                               _f32_addr(acc, "acc"), _stream(stream)),
           "dl_round_begin")
    return Round(h, len(frag_offsets) - 1)


def _ckpt_dtype(ckpt: Array, dtype: Optional[int]) -> int:
    if dtype is not None:
        return int(dtype)
    if not isinstance(ckpt, torch.Tensor):
        raise TypeError("dtype is required for a raw checkpoint address")
    if ckpt.dtype == torch.float32:
        return DL_F32
    if ckpt.dtype == torch.bfloat16:
        return DL_BF16
    raise TypeError("checkpoint must be float32 or bfloat16")


def dl_fold_checkpoint(r: Round, frag: int, worker_id: int, ckpt_round_tag: int, ckpt: Array,
                       global_: Array = None, tokens: int = 0,
                       dtype: Optional[int] = None) -> None:
    dtype = _ckpt_dtype(ckpt, dtype)
    _check(_lib.dl_fold_checkpoint(r.handle, int(frag), int(worker_id), int(ckpt_round_tag),
                                   _addr(ckpt), int(dtype), _f32_addr(global_, "global"),
                                   int(tokens)),
           "dl_fold_checkpoint")


def dl_finalize_mean(r: Round, frag: int, out_global: Array, ema: Array = None,
                     beta: float = 0.9) -> None:
    _check(_lib.dl_finalize_mean(r.handle, int(frag), _f32_addr(out_global, "out_global"),
                                 _f32_addr(ema, "ema"), float(beta)),
           "dl_finalize_mean")


def dl_outer_nesterov(r: Round, frag: int, global_: Array, momentum: Array, lr: float = 0.7,
                      mu: float = 0.9, ema: Array = None, beta: float = 0.9) -> None:
    _check(_lib.dl_outer_nesterov(r.handle, int(frag), _f32_addr(global_, "global"),
                                  _f32_addr(momentum, "momentum"), float(lr), float(mu),
                                  _f32_addr(ema, "ema"), float(beta)),
           "dl_outer_nesterov")


def dl_fold_and_finalize_mean(r: Round, frag: int, worker_id: int, ckpt_round_tag: int,
                              ckpt: Array, out_global: Array, ema: Array = None,
                              beta: float = 0.9, dtype: Optional[int] = None) -> None:
    dtype = _ckpt_dtype(ckpt, dtype)
    _check(_lib.dl_fold_and_finalize_mean(r.handle, int(frag), int(worker_id),
                                          int(ckpt_round_tag), _addr(ckpt), int(dtype),
                                          _f32_addr(out_global, "out_global"),
                                          _f32_addr(ema, "ema"), float(beta)),
           "dl_fold_and_finalize_mean")


def dl_fold_and_outer_nesterov(r: Round, frag: int, worker_id: int, ckpt_round_tag: int,
                               ckpt: Array, tokens: int, global_: Array, momentum: Array,
                               lr: float = 0.7, mu: float = 0.9, ema: Array = None,
                               beta: float = 0.9, dtype: Optional[int] = None) -> None:
    dtype = _ckpt_dtype(ckpt, dtype)
    _check(_lib.dl_fold_and_outer_nesterov(r.handle, int(frag), int(worker_id),
                                           int(ckpt_round_tag), _addr(ckpt), int(dtype),
                                           int(tokens), _f32_addr(global_, "global"),
                                           _f32_addr(momentum, "momentum"), float(lr),
                                           float(mu), _f32_addr(ema, "ema"), float(beta)),
           "dl_fold_and_outer_nesterov")


def _arrivals(worker_ids: Sequence[int], ckpt_round_tags, ckpts: Sequence[Array],
              tokens: Optional[Sequence[int]], dtype: Optional[int]):
    """Host arrays of a several-arrival call.  An int tag applies to every
    arrival; the dtype comes from the first checkpoint tensor unless given."""
    count = len(worker_ids)
    if isinstance(ckpt_round_tags, int):
        ckpt_round_tags = [ckpt_round_tags] * count
    if len(ckpt_round_tags) != count or len(ckpts) != count or \
            (tokens is not None and len(tokens) != count):
        raise ValueError("worker_ids, tags, checkpoints and tokens differ in length")
    if dtype is None:
        if count == 0:
            dtype = DL_F32
        else:
            dtype = _ckpt_dtype(ckpts[0], None)
            for c in ckpts[1:]:
                if isinstance(c, torch.Tensor) and _ckpt_dtype(c, None) != dtype:
                    raise TypeError("checkpoints of one call share one dtype")
    n = max(1, count)
    ids = (_i32 * n)(*[int(x) for x in worker_ids])
    tags = (_u64 * n)(*[int(x) for x in ckpt_round_tags])
    ptrs = (_p * n)(*[_addr(c) for c in ckpts])
    tok = None if tokens is None else (_i64 * n)(*[int(x) for x in tokens])
    return count, ids, tags, ptrs, tok, int(dtype)


def dl_fold_checkpoints(r: Round, frag: int, worker_ids: Sequence[int], ckpt_round_tags,
                        ckpts: Sequence[Array], global_: Array = None,
                        tokens: Optional[Sequence[int]] = None,
                        dtype: Optional[int] = None) -> None:
    count, ids, tags, ptrs, tok, dtype = _arrivals(worker_ids, ckpt_round_tags, ckpts, tokens,
                                                   dtype)
    _check(_lib.dl_fold_checkpoints(r.handle, int(frag), count, ids, tags, ptrs, dtype,
                                    _f32_addr(global_, "global"), tok),
           "dl_fold_checkpoints")


def dl_fold_checkpoints_and_finalize_mean(r: Round, frag: int, worker_ids: Sequence[int],
                                          ckpt_round_tags, ckpts: Sequence[Array],
                                          out_global: Array, ema: Array = None,
                                          beta: float = 0.9,
                                          dtype: Optional[int] = None) -> None:
    count, ids, tags, ptrs, _, dtype = _arrivals(worker_ids, ckpt_round_tags, ckpts, None, dtype)
    _check(_lib.dl_fold_checkpoints_and_finalize_mean(r.handle, int(frag), count, ids, tags, ptrs,
                                                      dtype, _f32_addr(out_global, "out_global"),
                                                      _f32_addr(ema, "ema"), float(beta)),
           "dl_fold_checkpoints_and_finalize_mean")


def dl_fold_checkpoints_and_outer_nesterov(r: Round, frag: int, worker_ids: Sequence[int],
                                           ckpt_round_tags, ckpts: Sequence[Array],
                                           tokens: Sequence[int], global_: Array,
                                           momentum: Array, lr: float = 0.7, mu: float = 0.9,
                                           ema: Array = None, beta: float = 0.9,
                                           dtype: Optional[int] = None) -> None:
    count, ids, tags, ptrs, tok, dtype = _arrivals(worker_ids, ckpt_round_tags, ckpts, tokens,
                                                   dtype)
    _check(_lib.dl_fold_checkpoints_and_outer_nesterov(
        r.handle, int(frag), count, ids, tags, ptrs, dtype, tok, _f32_addr(global_, "global"),
        _f32_addr(momentum, "momentum"), float(lr), float(mu), _f32_addr(ema, "ema"),
        float(beta)),
        "dl_fold_checkpoints_and_outer_nesterov")


def dl_ema_update(ema: Array, global_: Array, beta: float = 0.9, n: Optional[int] = None,
                  stream=None) -> None:
    if n is None:
        if not isinstance(ema, torch.Tensor):
            raise TypeError("n is required for raw addresses")
        n = ema.numel()
        if isinstance(global_, torch.Tensor) and global_.numel() != n:
            raise ValueError("ema and global differ in size")
    _check(_lib.dl_ema_update(_f32_addr(ema, "ema"), _f32_addr(global_, "global"), int(n),
                              float(beta), _stream(stream)),
           "dl_ema_update")


def _n_of(a: Array, n: Optional[int]) -> int:
    if n is not None:
        return int(n)
    if not isinstance(a, torch.Tensor):
        raise TypeError("n is required for raw addresses")
    return a.numel()


def dl_swa_fold(sum_: Array, global_: Array, folded_before: int, n: Optional[int] = None,
                stream=None) -> None:
    _check(_lib.dl_swa_fold(_f32_addr(sum_, "sum"), _f32_addr(global_, "global"),
                            _n_of(sum_, n), int(folded_before), _stream(stream)),
           "dl_swa_fold")


def dl_swa_average(out: Array, sum_: Array, count: int, n: Optional[int] = None,
                   stream=None) -> None:
    _check(_lib.dl_swa_average(_f32_addr(out, "out"), _f32_addr(sum_, "sum"), _n_of(out, n),
                               int(count), _stream(stream)),
           "dl_swa_average")


def dl_snapshot_average(out: Array, snapshots: Sequence[Array], n: Optional[int] = None,
                        stream=None) -> None:
    ptrs = (_p * max(1, len(snapshots)))(*[_f32_addr(x, "snapshot") for x in snapshots])
    _check(_lib.dl_snapshot_average(_f32_addr(out, "out"), ptrs, len(snapshots), _n_of(out, n),
                                    _stream(stream)),
           "dl_snapshot_average")


def dl_adopt_keep_drift(theta: Array, global_: Array, pushed: Array, n: Optional[int] = None,
                        dtype: Optional[int] = None, stream=None) -> None:
    _check(_lib.dl_adopt_keep_drift(_f32_addr(theta, "theta"), _f32_addr(global_, "global"),
                                    _addr(pushed), _ckpt_dtype(pushed, dtype), _n_of(theta, n),
                                    _stream(stream)),
           "dl_adopt_keep_drift")


def dl_polar_workspace_bytes(rows: int, cols: int) -> int:
    b = _i64()
    _check(_lib.dl_polar_workspace_bytes(int(rows), int(cols), ctypes.byref(b)),
           "dl_polar_workspace_bytes")
    return b.value


def _ws(workspace: Array, workspace_bytes: Optional[int]):
    if workspace_bytes is None:
        if not isinstance(workspace, torch.Tensor):
            raise TypeError("workspace_bytes is required for a raw workspace address")
        workspace_bytes = workspace.numel() * workspace.element_size()
    return _addr(workspace), int(workspace_bytes)


def dl_polar_factor(out: Array, update: Array, rows: int, cols: int, workspace: Array,
                    quintic_steps: int = 12, cubic_steps: int = 6,
                    workspace_bytes: Optional[int] = None, stream=None) -> None:
    w, wb = _ws(workspace, workspace_bytes)
    _check(_lib.dl_polar_factor(_f32_addr(out, "out"), _f32_addr(update, "update"), int(rows),
                                int(cols), int(quintic_steps), int(cubic_steps), w, wb,
                                _stream(stream)),
           "dl_polar_factor")


def dl_outer_orthogonal_step(theta: Array, averaged: Array, rows: int, cols: int, scale: float,
                             workspace: Array, quintic_steps: int = 12, cubic_steps: int = 6,
                             workspace_bytes: Optional[int] = None, stream=None) -> None:
    w, wb = _ws(workspace, workspace_bytes)
    _check(_lib.dl_outer_orthogonal_step(_f32_addr(theta, "theta"), _f32_addr(averaged, "averaged"),
                                         int(rows), int(cols), float(scale), int(quintic_steps),
                                         int(cubic_steps), w, wb, _stream(stream)),
           "dl_outer_orthogonal_step")


def dl_outer_orthogonal_step_noalloc(theta: Array, averaged: Array, rows: int, cols: int,
                                     scale: float, quintic_steps: int = 12, cubic_steps: int = 6,
                                     stream=None) -> None:
    _check(_lib.dl_outer_orthogonal_step_noalloc(_f32_addr(theta, "theta"),
                                                 _f32_addr(averaged, "averaged"), int(rows),
                                                 int(cols), float(scale), int(quintic_steps),
                                                 int(cubic_steps), _stream(stream)),
           "dl_outer_orthogonal_step_noalloc")


def dl_polar_workspace_bytes_batch(rows: int, cols: int, batch: int) -> int:
    b = _i64()
    _check(_lib.dl_polar_workspace_bytes_batch(int(rows), int(cols), int(batch), ctypes.byref(b)),
           "dl_polar_workspace_bytes_batch")
    return b.value


def dl_outer_orthogonal_step_batch(thetas: Sequence[Array], averaged: Sequence[Array], rows: int,
                                   cols: int, scale: float, workspace: Array,
                                   quintic_steps: int = 12, cubic_steps: int = 6,
                                   workspace_bytes: Optional[int] = None, stream=None) -> None:
    if len(thetas) != len(averaged):
        raise ValueError("one averaged matrix per theta")
    n = len(thetas)
    tp = (_p * max(1, n))(*[_f32_addr(t, "theta") for t in thetas])
    ap = (_p * max(1, n))(*[_f32_addr(a, "averaged") for a in averaged])
    w, wb = _ws(workspace, workspace_bytes)
    _check(_lib.dl_outer_orthogonal_step_batch(tp, ap, n, int(rows), int(cols), float(scale),
                                               int(quintic_steps), int(cubic_steps), w, wb,
                                               _stream(stream)),
           "dl_outer_orthogonal_step_batch")


def dl_matmul_workspace_bytes(m: int, n: int, k: int, symmetric: bool = False) -> int:
    b = _i64()
    _check(_lib.dl_matmul_workspace_bytes(int(m), int(n), int(k), int(bool(symmetric)),
                                          ctypes.byref(b)),
           "dl_matmul_workspace_bytes")
    return b.value


def dl_matmul_f32(form: int, a: Array, lda: int, b: Array, ldb: int, m: int, n: int, k: int,
                  c: Array, ldc: int, y: Array = None, alpha: float = 1.0, beta: float = 0.0,
                  diag: float = 0.0, symmetric: bool = False, workspace: Array = None,
                  workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace is None:
        w, wb = None, 0
    else:
        w, wb = _ws(workspace, workspace_bytes)
    _check(_lib.dl_matmul_f32(int(form), _f32_addr(a, "a"), int(lda), _f32_addr(b, "b"), int(ldb),
                              int(m), int(n), int(k), _f32_addr(c, "c"), int(ldc),
                              _f32_addr(y, "y"), float(alpha), float(beta), float(diag),
                              int(bool(symmetric)), w, wb, _stream(stream)),
           "dl_matmul_f32")


def dl_matmul_workspace_bytes_batch(m: int, n: int, k: int, symmetric: bool, batch: int) -> int:
    b = _i64()
    _check(_lib.dl_matmul_workspace_bytes_batch(int(m), int(n), int(k), int(bool(symmetric)),
                                                int(batch), ctypes.byref(b)),
           "dl_matmul_workspace_bytes_batch")
    return b.value


def dl_matmul_large_tiles(m: int, n: int, k: int, symmetric: bool, batch: int,
                          workspace_bytes: int) -> bool:
    out = _i32()
    _check(_lib.dl_matmul_large_tiles(int(m), int(n), int(k), int(bool(symmetric)), int(batch),
                                      int(workspace_bytes), ctypes.byref(out)),
           "dl_matmul_large_tiles")
    return bool(out.value)


def dl_matmul_f32_batch(form: int, a: Array, lda: int, stride_a: int, b: Array, ldb: int,
                        stride_b: int, m: int, n: int, k: int, c: Array, ldc: int, stride_c: int,
                        batch: int, y: Array = None, stride_y: int = 0, alpha: float = 1.0,
                        beta: float = 0.0, diag: float = 0.0, symmetric: bool = False,
                        workspace: Array = None, workspace_bytes: Optional[int] = None,
                        stream=None) -> None:
    if workspace is None:
        w, wb = None, 0
    else:
        w, wb = _ws(workspace, workspace_bytes)
    _check(_lib.dl_matmul_f32_batch(int(form), _f32_addr(a, "a"), int(lda), int(stride_a),
                                    _f32_addr(b, "b"), int(ldb), int(stride_b), int(m), int(n),
                                    int(k), _f32_addr(c, "c"), int(ldc), int(stride_c),
                                    _f32_addr(y, "y"), int(stride_y), float(alpha), float(beta),
                                    float(diag), int(bool(symmetric)), int(batch), w, wb,
                                    _stream(stream)),
           "dl_matmul_f32_batch")


def dl_frag_range(r: Round, frag: int) -> Tuple[int, int]:
    off, length = _i64(), _i64()
    _check(_lib.dl_frag_range(r.handle, int(frag), ctypes.byref(off), ctypes.byref(length)),
           "dl_frag_range")
    return off.value, length.value


def dl_round_participants(r: Round, frag: int) -> List[int]:
    count = _i32()
    _check(_lib.dl_round_participants(r.handle, int(frag), ctypes.byref(count), None, 0),
           "dl_round_participants")
    buf = (_i32 * max(1, count.value))()
    _check(_lib.dl_round_participants(r.handle, int(frag), ctypes.byref(count), buf,
                                      count.value),
           "dl_round_participants")
    return list(buf[:count.value])


def dl_round_tokens(r: Round, frag: int) -> int:
    t = _i64()
    _check(_lib.dl_round_tokens(r.handle, int(frag), ctypes.byref(t)), "dl_round_tokens")
    return t.value


def dl_round_end(r: Round) -> None:
    if r._h is not None:
        _check(_lib.dl_round_end(r._h), "dl_round_end")
        r._h = None


def raw_lib() -> ctypes.CDLL:
    """The loaded library (status-code level access for tests)."""
    return _lib
