"""Host checks of the orthogonalised step's bookkeeping: which tensors of a
layout are weight matrices (and where they sit in the flat buffer), how the
matrices of one shape are batched, and the algorithmic flop count."""
import pytest
import torch

from checkpoint_averaging_amd import dlmerge as dl
from checkpoint_averaging_amd import synth
from checkpoint_averaging_amd.orthogonalize import (OrthogonalStep, batch_sizes, gemm_flops,
                                                    weight_matrices)


def _check_layout(layout):
    mats = weight_matrices(layout)
    offs = {}
    off = 0
    for name, n in layout.tensors:
        offs[name] = (off, n)
        off += n
    assert off == layout.n_params
    end = 0
    for m in mats:
        o, n = offs[m.name]
        assert m.offset == o and m.rows * m.cols == n
        assert m.offset >= end          # flat order, no overlap
        end = m.offset + n
    return mats


def test_diffurefill1b_weight_matrices():
    mats = _check_layout(synth.DIFFUREFILL_1B)
    shapes = {}
    for m in mats:
        shapes[(m.rows, m.cols)] = shapes.get((m.rows, m.cols), 0) + 1
    # tied embedding, 18 blocks of 4 attention projections and 3 SwiGLU ones
    assert shapes == {(73760, 2048): 1, (2048, 2048): 72, (5632, 2048): 36, (2048, 5632): 18}
    # everything but the 18 x 2 + 1 RMSNorm weight vectors of 2048
    assert sum(m.rows * m.cols for m in mats) == synth.DIFFUREFILL_1B.n_params - 37 * 2048


def test_pythia14m_weight_matrices():
    mats = _check_layout(synth.PYTHIA_14M)
    assert len(mats) == 26
    assert {(m.rows, m.cols) for m in mats} == {(50304, 128), (384, 128), (128, 128), (512, 128),
                                               (128, 512)}


@pytest.mark.parametrize("count", [1, 17, 18, 36, 64, 65, 72, 127, 128, 130])
def test_even_batches(count):
    b = batch_sizes(count)
    assert sum(b) == count and max(b) <= dl.DL_MAX_BATCH
    assert len(b) == -(-count // dl.DL_MAX_BATCH)          # as few launches as hold them
    assert max(b) - min(b) <= 1                            # split evenly, larger first
    assert b == sorted(b, reverse=True)


def test_fixed_batches():
    assert batch_sizes(72, 8) == [8] * 9
    assert batch_sizes(18, 8) == [8, 8, 2]
    assert batch_sizes(5, 1) == [1] * 5
    with pytest.raises(ValueError):
        batch_sizes(5, 0)
    with pytest.raises(ValueError):
        batch_sizes(5, dl.DL_MAX_BATCH + 1)


def test_step_groups_pythia14m_on_host():
    # the grouping and the workspace size need no GPU
    step = OrthogonalStep(synth.PYTHIA_14M, device=torch.device("cpu"))
    sizes = sorted((len(g), g[0].rows, g[0].cols) for g in step.groups)
    # the untied input and output embeddings share a shape and a batch
    assert sizes == [(2, 50304, 128), (6, 128, 128), (6, 128, 512), (6, 384, 128),
                     (6, 512, 128)]
    assert all(len({(m.rows, m.cols) for m in g}) == 1 for g in step.groups)
    need = max(dl.dl_polar_workspace_bytes_batch(g[0].rows, g[0].cols, len(g))
               for g in step.groups)
    assert step.workspace.numel() * 4 >= need


def test_flops_square_and_rectangular():
    r = 2048
    f = gemm_flops(r, r)
    sym = r * (r + 1) // 2
    # per step: the Gram product (TN) and the next iterate (NT); per quintic
    # step also the square of the Gram matrix (NT); symmetric products at
    # their distinct outputs
    assert f["TN"] == 18 * 2 * sym * r
    assert f["NT"] == 18 * 2 * r ** 3 + 12 * 2 * sym * r
    tall, wide = gemm_flops(5632, 2048), gemm_flops(2048, 5632)
    assert tall["TN"] + tall["NT"] == wide["TN"] + wide["NT"]   # the same work, transposed
    # the whole DiffuRefill-1B step
    total = sum(sum(gemm_flops(m.rows, m.cols).values())
                for m in weight_matrices(synth.DIFFUREFILL_1B))
    assert total == 132103250509824


def test_product_kernel_rule():
    """The library's choice of kernel for the step's products (a host-side
    query, no GPU): large tiles where 256 x 256 tiles fill the CUs, with the
    last round's tiles cut along K where that evens them out."""
    from checkpoint_averaging_amd.orthogonalize import product_kernel
    # next iterates (tall: X M as NT; wide: M X as TN) fill their rounds
    assert product_kernel("NT", 2048, 2048, 2048, 36, False) == "k_gemm_big<NT>"   # 2304 tiles
    assert product_kernel("NT", 5632, 2048, 2048, 36, False) == "k_gemm_big<NT>"   # 6336 tiles
    assert product_kernel("NT", 73760, 2048, 2048, 1, False) == "k_gemm_big<NT>"   # + a strip
    assert product_kernel("TN", 2048, 5632, 2048, 18, False) == "k_gemm_big<TN>"   # 3168 tiles
    # symmetric Gram products and squares: 36 upper tiles per 2048^2 result
    assert product_kernel("TN", 2048, 2048, 2048, 36, True) == "k_gemm_big<TN>"    # 1296: split
    assert product_kernel("NT", 2048, 2048, 2048, 36, True) == "k_gemm_big<NT>"
    assert product_kernel("TN", 2048, 2048, 73760, 1, True) == "k_gemm_big<TN>"   # all in pieces
    # too few tiles to fill the CUs, or rounds that no split evens out
    assert product_kernel("NT", 2048, 2048, 2048, 1, True) == "k_gemm<NT>"
    assert product_kernel("NT", 2048, 2048, 5632, 18, True) == "k_gemm<NT>"       # 648 tiles
    assert product_kernel("NT", 2048, 2048, 2048, 3, False) == "k_gemm<NT>"       # 192 tiles
    # K not a multiple of 16; a symmetric result not a multiple of 256
    assert product_kernel("NT", 2048, 2048, 2040, 36, False) == "k_gemm<NT>"
    assert product_kernel("TN", 2000, 2000, 4096, 36, True) == "k_gemm<TN>"
    # the small model's matrices never fill large tiles
    assert product_kernel("TN", 128, 128, 50304, 2, True) == "k_gemm<TN>"