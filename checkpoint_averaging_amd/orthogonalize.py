"""Outer orthogonalisation over a whole model (DiffuRefill-1B technical report,
"What we measured", "Optimisers": the averaged outer update of each weight
matrix is replaced by its polar factor).

The flat parameter buffer holds every tensor back to back; the weight
matrices are row-major views into it.  Vectors (norm weights) have no polar
factor of interest and are left to the plain merge.  Matrices of one shape
go through dl_outer_orthogonal_step_batch together (by default all of them,
split evenly into as few launches of at most DL_MAX_BATCH as hold them), on
one stream, all sharing one workspace sized for the largest batch.
"""
from __future__ import annotations

import math
from typing import List, NamedTuple, Optional

import torch

from . import dlmerge as dl
from . import synth


class Matrix(NamedTuple):
    name: str
    offset: int        # element offset in the flat buffer
    rows: int
    cols: int


def _shapes(layout: synth.Layout):
    if layout.name == "diffurefill-1b":
        d, vocab, ff = 2048, 73760, 5632
        shape = {"embed": (vocab, d), "attn.wq": (d, d), "attn.wk": (d, d), "attn.wv": (d, d),
                 "attn.wo": (d, d), "ffn.w_gate": (ff, d), "ffn.w_up": (ff, d),
                 "ffn.w_down": (d, ff)}
    elif layout.name == "pythia-14m":
        d, vocab, ff = 128, 50304, 512
        shape = {"embed_in": (vocab, d), "embed_out": (vocab, d),
                 "attention.query_key_value.weight": (3 * d, d),
                 "attention.dense.weight": (d, d), "mlp.dense_h_to_4h.weight": (ff, d),
                 "mlp.dense_4h_to_h.weight": (d, ff)}
    else:
        raise KeyError(layout.name)
    return shape


def weight_matrices(layout: synth.Layout) -> List[Matrix]:
    """The layout's weight matrices in flat order, with their offsets."""
    shape = _shapes(layout)
    out, off = [], 0
    for name, n in layout.tensors:
        key = name.split(".", 2)[-1] if name.startswith(("blocks.", "layers.")) else name
        if key in shape:
            r, c = shape[key]
            if r * c != n:
                raise ValueError(f"{name}: {r}x{c} != {n}")
            out.append(Matrix(name, off, r, c))
        off += n
    return out


def gemm_flops(rows: int, cols: int, quintic: int = 12, cubic: int = 6):
    """Algorithmic flops (2 per product term) of the iteration on one matrix,
    by product form.  r is the short side, L the long one.  Per step: the
    Gram matrix over the long side, symmetric, so r (r + 1) / 2 distinct
    outputs of 2 L flops each; per quintic step its square, also symmetric
    (r (r + 1) / 2 outputs of 2 r flops); per step the next iterate (2 L r^2).
    Tall matrices run the Gram product as TN and the next iterate as NT; wide
    ones the other way round; the square (of an exactly symmetric matrix, so
    G G = G G^T) is NT."""
    r, L = min(rows, cols), max(rows, cols)
    sym = r * (r + 1) // 2
    gram, square, nxt = 2 * sym * L, 2 * sym * r, 2 * L * r * r
    steps = quintic + cubic
    tn = (gram * steps if rows >= cols else nxt * steps)
    nt = (nxt * steps if rows >= cols else gram * steps) + square * quintic
    return {"TN": tn, "NT": nt}


def batch_sizes(count: int, batch: Optional[int] = None) -> List[int]:
    """Sizes of the batches `count` equally shaped matrices run in: chunks
    of `batch`, or (None) an even split into ceil(count / DL_MAX_BATCH)."""
    if batch is not None:
        if not 1 <= batch <= dl.DL_MAX_BATCH:
            raise ValueError(f"batch {batch} not in [1, {dl.DL_MAX_BATCH}]")
        return [min(batch, count - c) for c in range(0, count, batch)]
    n = math.ceil(count / dl.DL_MAX_BATCH)
    return [count // n + (1 if i < count % n else 0) for i in range(n)]


def product_kernel(form: str, m: int, n: int, k: int, batch: int, symmetric: bool) -> str:
    """The kernel a product's main block runs on, asked of the library (its
    rule for aligned, contiguous operands with the workspace the product
    asks for): "k_gemm_big<TN>" / "k_gemm_big<NT>" for the large-tile
    kernel, else "k_gemm<TN>" / "k_gemm<NT>"."""
    ws = dl.dl_matmul_workspace_bytes_batch(m, n, k, symmetric, batch)
    big = dl.dl_matmul_large_tiles(m, n, k, symmetric, batch, ws)
    return f"k_gemm_big<{form}>" if big else f"k_gemm<{form}>"


class OrthogonalStep:
    """theta = theta - scale * P(theta - averaged) for every weight matrix of
    a layout, on one stream, with one workspace.  Matrices of one shape run
    in batches (one launch per product for the whole batch): of up to
    `batch`, or by default all of a shape, split evenly into launches of at
    most DL_MAX_BATCH; batch 1 runs them one by one."""

    def __init__(self, layout: synth.Layout, device: Optional[torch.device] = None,
                 quintic: int = 12, cubic: int = 6, batch: Optional[int] = None,
                 streams: int = 1):
        self.matrices = weight_matrices(layout)
        self.quintic, self.cubic = quintic, cubic
        by_shape = {}
        for m in self.matrices:
            by_shape.setdefault((m.rows, m.cols), []).append(m)
        self.groups = []
        for ms in by_shape.values():
            i = 0
            for b in batch_sizes(len(ms), batch):
                self.groups.append(ms[i:i + b])
                i += b
        if streams < 1:
            raise ValueError("streams must be at least 1")
        # batches dealt to the streams, largest first to the least loaded
        self.lanes: List[List[List[Matrix]]] = [[] for _ in range(streams)]
        load = [0] * streams
        for g in sorted(self.groups, key=self._group_flops, reverse=True):
            s = load.index(min(load))
            self.lanes[s].append(g)
            load[s] += self._group_flops(g)
        dev = device or torch.device("cuda")
        # one workspace per stream (batches in flight together must not share one)
        self.workspaces = []
        for lane in self.lanes:
            need = max((dl.dl_polar_workspace_bytes_batch(g[0].rows, g[0].cols, len(g))
                        for g in lane), default=256)
            self.workspaces.append(torch.empty((need + 3) // 4, dtype=torch.float32, device=dev))
        self.workspace = self.workspaces[0]
        self._streams = None

    def _group_flops(self, g: List[Matrix]) -> int:
        return len(g) * sum(gemm_flops(g[0].rows, g[0].cols, self.quintic, self.cubic).values())

    def flops(self):
        tot = {"TN": 0, "NT": 0}
        for m in self.matrices:
            for k, v in gemm_flops(m.rows, m.cols, self.quintic, self.cubic).items():
                tot[k] += v
        return tot

    def run(self, theta: torch.Tensor, averaged: torch.Tensor, scale: float, timer=None):
        """One orthogonalised outer step over the flat buffers.  `timer`, if
        given, is called as timer(matrices, call) for each batch and must
        call call().  With several streams, stream s runs lane s's batches
        in order; the streams start after the caller's stream and the
        caller's stream waits for all of them."""
        def issue(g, ws):
            rows, cols = g[0].rows, g[0].cols
            n = rows * cols
            ts = [theta[m.offset:m.offset + n] for m in g]
            avs = [averaged[m.offset:m.offset + n] for m in g]

            def call(ts=ts, avs=avs, rows=rows, cols=cols):
                if len(ts) == 1:
                    dl.dl_outer_orthogonal_step(ts[0], avs[0], rows, cols, scale, ws,
                                                self.quintic, self.cubic)
                else:
                    dl.dl_outer_orthogonal_step_batch(ts, avs, rows, cols, scale, ws,
                                                      self.quintic, self.cubic)
            if timer is None:
                call()
            else:
                timer(g, call)

        if len(self.lanes) == 1:
            for g in self.lanes[0]:
                issue(g, self.workspaces[0])
            return
        if self._streams is None:
            self._streams = [torch.cuda.Stream(device=theta.device) for _ in self.lanes]
        cur = torch.cuda.current_stream(theta.device)
        for st in self._streams:
            st.wait_stream(cur)
        for st, lane, ws in zip(self._streams, self.lanes, self.workspaces):
            with torch.cuda.stream(st):
                for g in lane:
                    issue(g, ws)
        for st in self._streams:
            cur.wait_stream(st)
