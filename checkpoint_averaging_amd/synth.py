"""Seeded synthetic inputs for the DiLoCo merge: parameter layouts, globals,
worker checkpoints, token counts and arrival orders.

This module is the one piece shared by the GPU path (benchmark, tests) and the
CPU oracle side (tests, smoke check, CPU baseline).  It holds none of the
merge arithmetic: it only lays out flat parameter vectors and draws values.

Stand-ins.  The real checkpoints of the pages (Pythia-14M on the Pile, the
DiffuRefill-1B globals) are not available, so inputs take those models'
shapes and sizes with synthetic values:

* global      theta0[j] = fp32(0.02 * z0[j])
* worker i    c_i[j]    = fp32(theta[j] + fp32(1e-3 * z_i[j]))
* bf16 worker c_i rounded to bfloat16 (nearest-even) after the above

where z is a standardised Irwin-Hall(4) variate built from one Philox4x32-10
draw per element.  Philox is counter based, so any element range of any
stream can be produced on its own, on the CPU or on the GPU, with identical
bits: the integer steps are exact and the float steps are single IEEE
binary32 operations (one multiply or add per torch call, so nothing can be
fused).

Layouts.
* Pythia-14M (page "Pythia-14M on four rented GPUs and a bucket", section
  "Choosing a reference run": six layers of width 128, 14M parameters, 12.9M
  of them in two embeddings).  GPT-NeoX order with untied input/output
  embeddings of 50304 x 128.
* DiffuRefill-1B (page "DiffuRefill-1B" technical report, section "Model",
  Table 1: 18 layers, width 2048, 16 heads of 128, SwiGLU 5632, RMSNorm,
  vocabulary 73,760, embedding tied to the head, 1.08B parameters).  No biases
  and full multi-head attention, the plainest reading that gives 1.08B.

Fragments.
* Pythia-14M in 4 fragments (GradientMail post, section "Getting updates
  through the bucket": four fragments, each embedding a 25.8 MB fp32
  fragment, the transformer blocks in the other two): embed_in | blocks 0-2 |
  blocks 3-5 + final norm | embed_out.
* DiffuRefill-1B in 4 fragments (the pages give no split at 1B): the tied
  embedding alone, then the 18 blocks in three groups of six, the final norm
  with the last group.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np
import torch

# ----------------------------------------------------------------------------
# Layouts
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Layout:
    name: str
    tensors: Tuple[Tuple[str, int], ...]      # (name, numel) in flat order

    @property
    def n_params(self) -> int:
        return sum(n for _, n in self.tensors)

    def offset_of(self, tensor_name: str) -> int:
        off = 0
        for name, n in self.tensors:
            if name == tensor_name:
                return off
            off += n
        raise KeyError(tensor_name)

    def numel_of(self, tensor_name: str) -> int:
        for name, n in self.tensors:
            if name == tensor_name:
                return n
        raise KeyError(tensor_name)


def _pythia14m() -> Layout:
    d, vocab, ff = 128, 50304, 512
    t: List[Tuple[str, int]] = [("embed_in", vocab * d)]
    for b in range(6):
        p = f"layers.{b}."
        t += [
            (p + "input_layernorm.weight", d), (p + "input_layernorm.bias", d),
            (p + "post_attention_layernorm.weight", d),
            (p + "post_attention_layernorm.bias", d),
            (p + "attention.query_key_value.weight", 3 * d * d),
            (p + "attention.query_key_value.bias", 3 * d),
            (p + "attention.dense.weight", d * d), (p + "attention.dense.bias", d),
            (p + "mlp.dense_h_to_4h.weight", ff * d), (p + "mlp.dense_h_to_4h.bias", ff),
            (p + "mlp.dense_4h_to_h.weight", d * ff), (p + "mlp.dense_4h_to_h.bias", d),
        ]
    t += [("final_layer_norm.weight", d), ("final_layer_norm.bias", d),
          ("embed_out", vocab * d)]
    return Layout("pythia-14m", tuple(t))


def _diffurefill1b() -> Layout:
    d, vocab, ff, layers = 2048, 73760, 5632, 18
    t: List[Tuple[str, int]] = [("embed", vocab * d)]
    for b in range(layers):
        p = f"blocks.{b}."
        t += [
            (p + "attn_norm.weight", d),
            (p + "attn.wq", d * d), (p + "attn.wk", d * d),
            (p + "attn.wv", d * d), (p + "attn.wo", d * d),
            (p + "ffn_norm.weight", d),
            (p + "ffn.w_gate", ff * d), (p + "ffn.w_up", ff * d), (p + "ffn.w_down", d * ff),
        ]
    t += [("final_norm.weight", d)]
    return Layout("diffurefill-1b", tuple(t))


PYTHIA_14M = _pythia14m()
DIFFUREFILL_1B = _diffurefill1b()


def pythia14m_fragments() -> List[int]:
    """Offsets (n_frags + 1) of the 4-fragment split of Pythia-14M."""
    L = PYTHIA_14M
    return [0,
            L.offset_of("layers.0.input_layernorm.weight"),
            L.offset_of("layers.3.input_layernorm.weight"),
            L.offset_of("embed_out"),
            L.n_params]


def diffurefill1b_fragments() -> List[int]:
    """Offsets (n_frags + 1) of the 4-fragment split of DiffuRefill-1B."""
    L = DIFFUREFILL_1B
    return [0,
            L.offset_of("blocks.0.attn_norm.weight"),
            L.offset_of("blocks.6.attn_norm.weight"),
            L.offset_of("blocks.12.attn_norm.weight"),
            L.n_params]


# ----------------------------------------------------------------------------
# Workload descriptions (the five merge configurations)
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    description: str
    n_params: int
    frag_offsets: Tuple[int, ...]
    mode: str                 # "mean" | "delta_nesterov"
    workers: int
    ckpt_dtype: str           # "f32" | "bf16"
    quorum: int
    ema: bool
    lr: float = 0.7
    mu: float = 0.9
    beta: float = 0.9
    tokens: str = "none"      # "none" | "uniform_int" | "scaled_step"
    seed: int = 0

    @property
    def n_frags(self) -> int:
        return len(self.frag_offsets) - 1


WORKLOADS = {
    "pythia14m_mean": Workload(
        "pythia14m_mean",
        "Pythia-14M flat fp32 (14,067,712 params), 3 fp32 workers, plain mean "
        "by running fp32 sum in arrival order",
        PYTHIA_14M.n_params, (0, PYTHIA_14M.n_params), "mean", 3, "f32",
        quorum=2, ema=False, seed=1001),
    "pythia14m_frag_nesterov": Workload(
        "pythia14m_frag_nesterov",
        "Pythia-14M fp32 in 4 fragments, 4 workers, quorum 3, token counts "
        "U[200k,270k]; token-weighted delta mean + outer Nesterov lr 0.7 mu 0.9",
        PYTHIA_14M.n_params, tuple(pythia14m_fragments()), "delta_nesterov", 4,
        "f32", quorum=3, ema=False, tokens="uniform_int", seed=1002),
    "diffurefill1b_mean_ema": Workload(
        "diffurefill1b_mean_ema",
        "DiffuRefill-1B flat fp32 (1,075,980,288 params), 5 fp32 workers, "
        "plain mean + fused EMA beta 0.9",
        DIFFUREFILL_1B.n_params, (0, DIFFUREFILL_1B.n_params), "mean", 5, "f32",
        quorum=2, ema=True, seed=1003),
    "diffurefill1b_bf16_mean_ema": Workload(
        "diffurefill1b_bf16_mean_ema",
        "DiffuRefill-1B, 8 bf16 workers folded into an fp32 running sum in "
        "seeded random arrival order; fused mean + EMA beta 0.9",
        DIFFUREFILL_1B.n_params, (0, DIFFUREFILL_1B.n_params), "mean", 8, "bf16",
        quorum=2, ema=True, seed=1004),
    "diffurefill1b_frag_nesterov_ema": Workload(
        "diffurefill1b_frag_nesterov_ema",
        "DiffuRefill-1B in 4 fragments, 5 fp32 workers, token weights "
        "U[0.5,1.5)x131072x150, quorum 3; token-weighted delta mean + outer "
        "Nesterov lr 0.7 mu 0.9 + EMA beta 0.9, fused per fragment",
        DIFFUREFILL_1B.n_params, tuple(diffurefill1b_fragments()), "delta_nesterov",
        5, "f32", quorum=3, ema=True, tokens="scaled_step", seed=1005),
}

WORKLOAD_ORDER = ["pythia14m_mean", "pythia14m_frag_nesterov", "diffurefill1b_mean_ema",
                  "diffurefill1b_bf16_mean_ema", "diffurefill1b_frag_nesterov_ema"]


def scaled(w: Workload, n_params: int, frag_offsets: Sequence[int] | None = None) -> Workload:
    """The same workload on a smaller flat vector (parity cases).  Fragment
    boundaries are scaled proportionally unless given."""
    if frag_offsets is None:
        if w.n_frags == 1:
            frag_offsets = (0, n_params)
        else:
            frag_offsets = tuple([0] + [int(o * n_params // w.n_params) for o in w.frag_offsets[1:-1]]
                                 + [n_params])
    return dataclasses.replace(w, n_params=n_params, frag_offsets=tuple(frag_offsets))


# ----------------------------------------------------------------------------
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
# as 1, 2, 3", SC'11), on int64 torch tensors holding uint32 values.
# ----------------------------------------------------------------------------

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def _mulhilo(a: torch.Tensor, m: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """(hi, lo) 32-bit halves of the 64-bit product m * a, a < 2^32.

    The product would overflow int64, so a is split in 16-bit halves; every
    intermediate stays below 2^49."""
    a_lo = a & 0xFFFF
    a_hi = a >> 16
    p1 = a_lo * m                 # < 2^48
    p2 = a_hi * m                 # < 2^48
    t = p1 + ((p2 & 0xFFFF) << 16)
    lo = t & _MASK32
    hi = (p2 >> 16) + (t >> 32)
    return hi, lo


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds.  c* are int64 tensors with values < 2^32."""
    for r in range(10):
        hi0, lo0 = _mulhilo(c0, _M0)
        hi1, lo1 = _mulhilo(c2, _M1)
        kk0 = (k0 + r * _W0) & _MASK32
        kk1 = (k1 + r * _W1) & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ kk0), lo1, (hi0 ^ c3 ^ kk1), lo0
    return c0, c1, c2, c3


_SQRT3_F32 = float(np.float32(np.sqrt(3.0)))


def std_normalish(seed: int, stream: int, rnd: int, start: int, count: int,
                  device="cpu") -> torch.Tensor:
    """fp32 standardised Irwin-Hall(4) variates for elements [start, start+count)
    of (seed, stream, round).  Identical bits on every device."""
    j = torch.arange(start, start + count, dtype=torch.int64, device=device)
    c0 = j & _MASK32
    c1 = j >> 32
    c2 = torch.full_like(j, stream & _MASK32)
    c3 = torch.full_like(j, rnd & _MASK32)
    del j
    x0, x1, x2, x3 = philox4x32_10(c0, c1, c2, c3, seed & _MASK32, 0x5EED0000 ^ (seed >> 32))
    s = (x0 >> 10) + (x1 >> 10) + (x2 >> 10) + (x3 >> 10)   # < 2^24: exact in fp32
    z = (s - (1 << 23)).to(torch.float32)                      # exact
    z = torch.mul(z, 2.0 ** -22)                                # exact (power of two)
    z = torch.mul(z, _SQRT3_F32)                                # one rounding
    return z


_CHUNK = 1 << 25


def _fill(out: torch.Tensor, start: int, fn) -> torch.Tensor:
    n = out.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = fn(start + s, e - s)
    return out


def global0(seed: int, n: int, device="cpu", start: int = 0, out: torch.Tensor | None = None):
    """Initial global theta0[start:start+n] = fp32(0.02 * z)."""
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=device)
    dev = out.device
    return _fill(out, start, lambda s, c: torch.mul(std_normalish(seed, 0, 0, s, c, dev),
                                                    np.float32(0.02).item()))


def worker_checkpoint(seed: int, rnd: int, worker: int, theta: torch.Tensor, start: int = 0,
                      dtype: str = "f32", out: torch.Tensor | None = None) -> torch.Tensor:
    """Worker checkpoint c = fp32(theta + fp32(1e-3 * z)) for elements
    [start, start + theta.numel()) (theta is that slice of the round's global),
    rounded to bf16 if dtype == "bf16"."""
    n = theta.numel()
    dev = theta.device
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if out is None:
        out = torch.empty(n, dtype=tdt, device=dev)

    def gen(s, c):
        drift = torch.mul(std_normalish(seed, 1 + worker, rnd, start + s, c, dev),
                          np.float32(1e-3).item())
        v = torch.add(theta[s:s + c], drift)
        return v.to(tdt)
    return _fill(out, 0, gen)


def token_counts(w: Workload, rnd: int) -> List[int]:
    """Per-worker token counts of one round (host integers)."""
    rng = np.random.default_rng([w.seed, 7, rnd])
    if w.tokens == "uniform_int":
        return [int(x) for x in rng.integers(200_000, 270_001, size=w.workers)]
    if w.tokens == "scaled_step":
        u = rng.uniform(0.5, 1.5, size=w.workers)
        return [int(round(x * 131072 * 150)) for x in u]
    return [0] * w.workers


def arrival_order(w: Workload, rnd: int, frag: int) -> List[int]:
    """Seeded arrival order of the workers for one round and fragment."""
    rng = np.random.default_rng([w.seed, 11, rnd, frag])
    return [int(x) for x in rng.permutation(w.workers)]


def late_worker(w: Workload, rnd: int, frag: int) -> int:
    """A seeded worker that misses the close of an exactly-quorum round."""
    rng = np.random.default_rng([w.seed, 13, rnd, frag])
    return int(rng.integers(0, w.workers))
