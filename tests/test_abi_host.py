"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and its host-side round rules reject bad calls before any device
work (these paths make no HIP call, so they run without a GPU).  Also checks
the gfx950 assembly of the kernels for the arithmetic the merge requires."""
import collections
import os
import re

import pytest
import torch

from checkpoint_averaging_amd import build as cabuild
from checkpoint_averaging_amd import dlmerge as dl

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "dlmerge.h")
FAKE = 0x7F0000000000        # never dereferenced: every call below fails before use
OFFS1 = [0, 1000]
OFFS4 = [0, 96, 200, 208, 1000]


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const\s+)?\w+\s*\*?\s*(dl_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    declared = header_functions()
    assert len(declared) == 30
    assert sorted(dl.SYMBOLS) == declared
    lib = dl.raw_lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name in ("DL_OK", "DL_E_INVAL", "DL_E_STALE", "DL_E_DUP", "DL_E_QUORUM", "DL_E_STATE",
                 "DL_E_ALIGN", "DL_E_HIP", "DL_E_CAPACITY", "DL_E_NOMEM", "DL_E_TOO_LARGE",
                 "DL_MEAN",
                 "DL_DELTA_NESTEROV",
                 "DL_F32", "DL_BF16"):
        m = re.search(rf"\b{name}\s*=\s*(-?\d+)", text)
        assert m and int(m.group(1)) == getattr(dl, name), name
    for s in range(-10, 1):
        assert dl.dl_strerror(s) != "unknown status"
    assert dl.dl_strerror(-99) == "unknown status"


def _expect(status, fn, *a, **k):
    with pytest.raises(dl.DLError) as ei:
        fn(*a, **k)
    assert ei.value.status == status, (ei.value.status, status)


@pytest.mark.parametrize("kw,status", [
    (dict(mode=2), dl.DL_E_INVAL),
    (dict(n_params=0, frag_offsets=[0, 0]), dl.DL_E_INVAL),
    (dict(frag_offsets=[0, 500]), dl.DL_E_INVAL),           # does not end at n_params
    (dict(frag_offsets=[1, 1000]), dl.DL_E_INVAL),          # does not start at 0
    (dict(frag_offsets=[0, 500, 500, 1000]), dl.DL_E_INVAL),  # empty fragment
    (dict(frag_offsets=[0, 600, 400, 1000]), dl.DL_E_INVAL),  # decreasing
    (dict(quorum=0), dl.DL_E_INVAL),
    (dict(quorum=9, max_workers=8), dl.DL_E_INVAL),
    (dict(max_workers=0, quorum=0), dl.DL_E_INVAL),
    (dict(max_workers=70000), dl.DL_E_INVAL),
    (dict(acc=0), dl.DL_E_INVAL),
    (dict(acc=FAKE + 2), dl.DL_E_ALIGN),
])
def test_round_begin_rejects(kw, status):
    args = dict(round_tag=5, mode=dl.DL_MEAN, n_params=1000, frag_offsets=OFFS1, quorum=2,
                max_workers=8, acc=FAKE, stream=0)
    args.update(kw)
    _expect(status, dl.dl_round_begin, **args)


def test_host_round_rules_without_device_work():
    r = dl.dl_round_begin(7, dl.DL_MEAN, 1000, OFFS4, 3, 4, FAKE, stream=0)
    try:
        assert dl.dl_frag_range(r, 0) == (0, 96)
        assert dl.dl_frag_range(r, 3) == (208, 792)
        _expect(dl.DL_E_INVAL, dl.dl_frag_range, r, 4)
        assert dl.dl_round_participants(r, 1) == []
        assert dl.dl_round_tokens(r, 2) == 0
        # checks that come before any device access
        _expect(dl.DL_E_STALE, dl.dl_fold_checkpoint, r, 0, 1, 6, FAKE, dtype=dl.DL_F32)
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 4, 1, 7, FAKE, dtype=dl.DL_F32)
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, -1, 1, 7, FAKE, dtype=dl.DL_F32)
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 4, 7, FAKE, dtype=dl.DL_F32)
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, -1, 7, FAKE, dtype=dl.DL_F32)
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 1, 7, FAKE, dtype=5)
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 1, 7, FAKE, global_=FAKE,
                dtype=dl.DL_F32)                              # global in MEAN mode
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 1, 7, 0, dtype=dl.DL_F32)
        _expect(dl.DL_E_ALIGN, dl.dl_fold_checkpoint, r, 0, 1, 7, FAKE + 2, dtype=dl.DL_F32)
        _expect(dl.DL_E_ALIGN, dl.dl_fold_checkpoint, r, 0, 1, 7, FAKE + 1, dtype=dl.DL_BF16)
        # checkpoint overlapping the accumulator's fragment range
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 1, 1, 7, FAKE + 4 * 100,
                dtype=dl.DL_F32)
        # closing
        _expect(dl.DL_E_QUORUM, dl.dl_finalize_mean, r, 0, FAKE + (1 << 20))
        _expect(dl.DL_E_STATE, dl.dl_outer_nesterov, r, 0, FAKE, FAKE + 4096)
        _expect(dl.DL_E_INVAL, dl.dl_finalize_mean, r, 9, FAKE)
        # nothing was folded
        assert dl.dl_round_participants(r, 0) == []
    finally:
        dl.dl_round_end(r)


def test_host_rules_delta_mode():
    r = dl.dl_round_begin(1, dl.DL_DELTA_NESTEROV, 1000, OFFS4, 1, 4, FAKE, stream=0)
    try:
        g = FAKE + (1 << 24)
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 0, 1, FAKE + (1 << 22),
                dtype=dl.DL_F32, global_=None, tokens=5)          # no global
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 0, 1, FAKE + (1 << 22),
                dtype=dl.DL_F32, global_=g, tokens=0)             # no tokens
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 0, 1, FAKE + (1 << 22),
                dtype=dl.DL_F32, global_=g, tokens=-3)
        _expect(dl.DL_E_ALIGN, dl.dl_fold_checkpoint, r, 0, 0, 1, FAKE + (1 << 22),
                dtype=dl.DL_F32, global_=g + 1, tokens=3)
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 0, 1, g + 8,
                dtype=dl.DL_F32, global_=g, tokens=3)             # ckpt overlaps global
        _expect(dl.DL_E_STALE, dl.dl_fold_checkpoint, r, 0, 0, 2, FAKE + (1 << 22),
                dtype=dl.DL_F32, global_=g, tokens=3)
        _expect(dl.DL_E_QUORUM, dl.dl_outer_nesterov, r, 0, g, FAKE + (1 << 26))
        _expect(dl.DL_E_STATE, dl.dl_finalize_mean, r, 0, g)
    finally:
        dl.dl_round_end(r)


def test_host_rules_fused_close():
    g = FAKE + (1 << 24)
    r = dl.dl_round_begin(3, dl.DL_MEAN, 1000, OFFS4, 2, 4, FAKE, stream=0)
    try:
        # one arrival short of the quorum even counting this one
        _expect(dl.DL_E_QUORUM, dl.dl_fold_and_finalize_mean, r, 0, 1, 3, FAKE + (1 << 22), g,
                dtype=dl.DL_F32)
        _expect(dl.DL_E_STALE, dl.dl_fold_and_finalize_mean, r, 0, 1, 4, FAKE + (1 << 22), g,
                dtype=dl.DL_F32)
        _expect(dl.DL_E_STATE, dl.dl_fold_and_outer_nesterov, r, 0, 1, 3, FAKE + (1 << 22), 5, g,
                g + (1 << 20), dtype=dl.DL_F32)
        _expect(dl.DL_E_ALIGN, dl.dl_fold_and_finalize_mean, r, 0, 1, 3, FAKE + (1 << 22) + 2, g,
                dtype=dl.DL_F32)
        assert dl.dl_round_participants(r, 0) == []
    finally:
        dl.dl_round_end(r)
    r = dl.dl_round_begin(3, dl.DL_DELTA_NESTEROV, 1000, OFFS4, 1, 4, FAKE, stream=0)
    try:
        ck = FAKE + (1 << 22)
        _expect(dl.DL_E_STATE, dl.dl_fold_and_finalize_mean, r, 0, 1, 3, ck, g, dtype=dl.DL_F32)
        _expect(dl.DL_E_INVAL, dl.dl_fold_and_outer_nesterov, r, 0, 1, 3, ck, 0, g,
                g + (1 << 20), dtype=dl.DL_F32)                      # no tokens
        _expect(dl.DL_E_INVAL, dl.dl_fold_and_outer_nesterov, r, 0, 1, 3, ck, 5, g, g + 4,
                dtype=dl.DL_F32)                                     # momentum overlaps global
        _expect(dl.DL_E_INVAL, dl.dl_fold_and_outer_nesterov, r, 0, 1, 3, g + 8, 5, g,
                g + (1 << 20), dtype=dl.DL_F32)                      # snapshot overlaps global
        _expect(dl.DL_E_STALE, dl.dl_fold_and_outer_nesterov, r, 0, 1, 9, ck, 5, g,
                g + (1 << 20), dtype=dl.DL_F32)
    finally:
        dl.dl_round_end(r)


def test_host_rules_several_arrivals():
    """The several-arrival calls check every arrival as the one-arrival call
    would, after those before it, and record nothing on any error."""
    g = FAKE + (1 << 24)
    ck = [FAKE + (1 << 22) + i * 4096 for i in range(4)]
    r = dl.dl_round_begin(3, dl.DL_MEAN, 1000, OFFS4, 3, 4, FAKE, stream=0)
    try:
        fold = lambda ids, tags, cks, **k: dl.dl_fold_checkpoints(r, 0, ids, tags, cks,
                                                                  dtype=dl.DL_F32, **k)
        _expect(dl.DL_E_INVAL, fold, [], 3, [])                               # count 0
        _expect(dl.DL_E_INVAL, fold, [0, 1, 2, 3, 0], 3, ck + [ck[0]])        # count > workers
        _expect(dl.DL_E_DUP, fold, [0, 1, 0], 3, ck[:3])                      # within the call
        _expect(dl.DL_E_STALE, fold, [0, 1], [3, 4], ck[:2])                  # second tag
        _expect(dl.DL_E_INVAL, fold, [0, 4], 3, ck[:2])                       # worker range
        _expect(dl.DL_E_INVAL, fold, [0, 1], 3, [ck[0], 0])                   # NULL checkpoint
        _expect(dl.DL_E_ALIGN, fold, [0, 1], 3, [ck[0], ck[1] + 2])
        _expect(dl.DL_E_INVAL, fold, [0, 1], 3, [ck[0], FAKE + 4 * 90])       # overlaps acc
        _expect(dl.DL_E_INVAL, fold, [0, 1], 3, ck[:2], global_=g)            # global in MEAN
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoints, r, 4, [0], 3, ck[:1], dtype=dl.DL_F32)
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoints, r, 0, [0], 3, ck[:1], dtype=2)
        close = lambda ids, cks, out, **k: dl.dl_fold_checkpoints_and_finalize_mean(
            r, 0, ids, 3, cks, out, dtype=dl.DL_F32, **k)
        _expect(dl.DL_E_QUORUM, close, [0, 1], ck[:2], g)                     # 2 < quorum 3
        _expect(dl.DL_E_INVAL, close, [0, 1, 2], ck[:3], ck[2] - 8)           # out over a ckpt
        _expect(dl.DL_E_INVAL, close, [0, 1, 2], ck[:3], g, ema=ck[1] + 4)    # ema over a ckpt
        _expect(dl.DL_E_STATE, dl.dl_fold_checkpoints_and_outer_nesterov, r, 0, [0, 1, 2], 3,
                ck[:3], [5, 5, 5], g, g + (1 << 20), dtype=dl.DL_F32)
        assert dl.dl_round_participants(r, 0) == []
        # the binding checks that the per-arrival arrays agree in length
        with pytest.raises(ValueError):
            fold([0, 1], 3, ck[:3])
    finally:
        dl.dl_round_end(r)
    r = dl.dl_round_begin(3, dl.DL_DELTA_NESTEROV, 1000, OFFS4, 1, 4, FAKE, stream=0)
    try:
        fold = lambda ids, cks, tokens, **k: dl.dl_fold_checkpoints(
            r, 0, ids, 3, cks, global_=g, tokens=tokens, dtype=dl.DL_F32, **k)
        _expect(dl.DL_E_INVAL, fold, [0, 1], ck[:2], None)                    # no tokens
        _expect(dl.DL_E_INVAL, fold, [0, 1], ck[:2], [5, 0])
        _expect(dl.DL_E_INVAL, fold, [0, 1], ck[:2], [(1 << 62), (1 << 62)])  # sum overflows
        _expect(dl.DL_E_INVAL, fold, [0, 1], [ck[0], g + 8], [5, 5])          # ckpt over global
        _expect(dl.DL_E_INVAL, dl.dl_fold_checkpoints, r, 0, [0], 3, ck[:1], dtype=dl.DL_F32,
                tokens=[5])                                                   # no global
        nest = lambda ids, cks, tokens, mom, **k: dl.dl_fold_checkpoints_and_outer_nesterov(
            r, 0, ids, 3, cks, tokens, g, mom, dtype=dl.DL_F32, **k)
        _expect(dl.DL_E_INVAL, nest, [0, 1], ck[:2], [5, 5], ck[1])           # momentum = ckpt
        _expect(dl.DL_E_INVAL, nest, [0, 1], ck[:2], [5, 5], g + (1 << 20), ema=ck[0])
        _expect(dl.DL_E_INVAL, nest, [0, 1], ck[:2], [5, 5], g + 4)           # momentum over global
        _expect(dl.DL_E_STATE, dl.dl_fold_checkpoints_and_finalize_mean, r, 0, [0], 3, ck[:1],
                g, dtype=dl.DL_F32)
        assert dl.dl_round_participants(r, 0) == []
        assert dl.dl_round_tokens(r, 0) == 0
    finally:
        dl.dl_round_end(r)


def test_ema_update_host_rules():
    dl.dl_ema_update(FAKE, FAKE + 4096, n=0, stream=0)                    # empty: no-op
    _expect(dl.DL_E_INVAL, dl.dl_ema_update, FAKE, FAKE + 4096, n=-1, stream=0)
    _expect(dl.DL_E_INVAL, dl.dl_ema_update, 0, FAKE, n=4, stream=0)
    _expect(dl.DL_E_ALIGN, dl.dl_ema_update, FAKE + 2, FAKE + 4096, n=4, stream=0)
    _expect(dl.DL_E_INVAL, dl.dl_ema_update, FAKE, FAKE + 8, n=4, stream=0)  # overlap


def test_side_average_host_rules():
    dl.dl_swa_fold(FAKE, FAKE + 4096, 0, n=0, stream=0)                   # empty: no-op
    _expect(dl.DL_E_INVAL, dl.dl_swa_fold, FAKE, FAKE + 4096, -1, n=4, stream=0)
    _expect(dl.DL_E_INVAL, dl.dl_swa_fold, FAKE, FAKE + 8, 0, n=4, stream=0)   # overlap
    _expect(dl.DL_E_ALIGN, dl.dl_swa_fold, FAKE + 1, FAKE + 4096, 0, n=4, stream=0)
    _expect(dl.DL_E_INVAL, dl.dl_swa_average, FAKE, FAKE + 4096, 0, n=4, stream=0)  # count 0
    _expect(dl.DL_E_INVAL, dl.dl_swa_average, FAKE, FAKE + 4, 3, n=4, stream=0)     # partial
    _expect(dl.DL_E_INVAL, dl.dl_snapshot_average, FAKE, [], n=4, stream=0)
    _expect(dl.DL_E_INVAL, dl.dl_snapshot_average, FAKE, [FAKE + 4096 * (i + 1) for i in range(17)],
            n=4, stream=0)
    _expect(dl.DL_E_INVAL, dl.dl_snapshot_average, FAKE, [FAKE + 4096, FAKE + 8], n=4,
            stream=0)                                                     # overlaps out
    _expect(dl.DL_E_ALIGN, dl.dl_snapshot_average, FAKE, [FAKE + 4096, FAKE + 8194], n=4,
            stream=0)
    dl.dl_snapshot_average(FAKE, [FAKE + 4096], n=0, stream=0)            # empty: no-op
    assert dl.DL_MAX_SNAPSHOTS == int(re.search(r"#define DL_MAX_SNAPSHOTS (\d+)",
                                                open(HEADER).read()).group(1))


def test_adopt_keep_drift_host_rules():
    dl.dl_adopt_keep_drift(FAKE, FAKE + 4096, FAKE + 8192, n=0, dtype=dl.DL_F32, stream=0)
    _expect(dl.DL_E_INVAL, dl.dl_adopt_keep_drift, FAKE, FAKE + 4096, FAKE + 8192, n=-1,
            dtype=dl.DL_F32, stream=0)
    _expect(dl.DL_E_INVAL, dl.dl_adopt_keep_drift, FAKE, FAKE + 4096, FAKE + 8192, n=4,
            dtype=7, stream=0)
    _expect(dl.DL_E_INVAL, dl.dl_adopt_keep_drift, FAKE, FAKE + 8, FAKE + 8192, n=4,
            dtype=dl.DL_F32, stream=0)                                 # theta overlaps global
    _expect(dl.DL_E_ALIGN, dl.dl_adopt_keep_drift, FAKE, FAKE + 4096, FAKE + 8193, n=4,
            dtype=dl.DL_BF16, stream=0)


def test_polar_host_rules():
    ws_need = dl.dl_polar_workspace_bytes(300, 200)
    r = 200
    assert ws_need >= 2 * 300 * 200 * 4 + 2 * r * r * 4
    assert dl.dl_polar_workspace_bytes(200, 300) == ws_need       # symmetric in the shape
    for rows, cols in ((0, 5), (5, 0), (-1, 5), ((1 << 31) + 1, 1), (1 << 24, 1 << 17)):
        _expect(dl.DL_E_INVAL, dl.dl_polar_workspace_bytes, rows, cols)
    ws, up, out = FAKE, FAKE + (1 << 30), FAKE + (1 << 31)
    call = lambda **k: dl.dl_polar_factor(**{**dict(out=out, update=up, rows=300, cols=200,
                                                     workspace=ws, workspace_bytes=ws_need,
                                                     stream=0), **k})
    for kw in (dict(quintic_steps=0, cubic_steps=0), dict(quintic_steps=-1),
               dict(cubic_steps=65), dict(quintic_steps=65),
               dict(workspace_bytes=ws_need - 1), dict(workspace=0), dict(out=0),
               dict(update=0), dict(rows=0),
               dict(out=up + 4),                                   # overlaps update
               dict(workspace=up - 256),                           # overlaps update
               dict(out=ws + 256)):                                # overlaps workspace
        _expect(dl.DL_E_INVAL, call, **kw)
    _expect(dl.DL_E_ALIGN, call, workspace=ws + 128)
    _expect(dl.DL_E_ALIGN, call, out=out + 2)
    _expect(dl.DL_E_ALIGN, call, update=up + 1)
    step = lambda **k: dl.dl_outer_orthogonal_step(**{**dict(theta=out, averaged=up, rows=300,
                                                             cols=200, scale=0.1, workspace=ws,
                                                             workspace_bytes=ws_need, stream=0),
                                                      **k})
    _expect(dl.DL_E_INVAL, step, averaged=out)                     # in place is not allowed
    _expect(dl.DL_E_INVAL, step, averaged=out + 1024)
    _expect(dl.DL_E_INVAL, step, theta=ws + 512)
    _expect(dl.DL_E_INVAL, step, cubic_steps=-2)
    _expect(dl.DL_E_ALIGN, step, theta=out + 3)


def test_polar_batch_host_rules():
    wsb = dl.dl_polar_workspace_bytes_batch(300, 200, 4)
    assert wsb > 2 * 4 * 300 * 200 * 4
    assert dl.dl_polar_workspace_bytes_batch(300, 200, 1) == dl.dl_polar_workspace_bytes(300, 200)
    for bad in ((300, 200, 0), (300, 200, 65), (0, 200, 2)):
        _expect(dl.DL_E_INVAL, dl.dl_polar_workspace_bytes_batch, *bad)
    ws = FAKE + (1 << 34)
    th = [FAKE + (i << 24) for i in range(4)]
    av = [FAKE + (1 << 30) + (i << 24) for i in range(4)]
    step = lambda **k: dl.dl_outer_orthogonal_step_batch(**{**dict(
        thetas=th, averaged=av, rows=300, cols=200, scale=0.1, workspace=ws,
        workspace_bytes=wsb, stream=0), **k})
    _expect(dl.DL_E_INVAL, step, workspace_bytes=wsb - 1)
    _expect(dl.DL_E_INVAL, step, thetas=th[:3] + [0])
    _expect(dl.DL_E_INVAL, step, thetas=th[:3] + [th[1] + 4096])        # two thetas meet
    _expect(dl.DL_E_INVAL, step, thetas=th[:3] + [av[0] + 4])           # theta meets an averaged
    _expect(dl.DL_E_INVAL, step, thetas=th[:3] + [ws + 256])            # theta meets the workspace
    _expect(dl.DL_E_ALIGN, step, averaged=av[:3] + [av[3] + 2])
    with pytest.raises(ValueError):
        step(averaged=av[:3])
    # averaged matrices may be shared (read only): fails only at the device
    # check, where the fake addresses are not allocations (DL_E_INVAL) or,
    # on a host with no GPU, the runtime's own error is pending (DL_E_HIP)
    no_gpu = torch.cuda.device_count() == 0
    _expect(dl.DL_E_HIP if no_gpu else dl.DL_E_INVAL, step, averaged=[av[0]] * 4)


def test_matmul_host_rules():
    a, b, c = FAKE, FAKE + (1 << 28), FAKE + (1 << 29)
    mm = lambda **k: dl.dl_matmul_f32(**{**dict(form=dl.DL_TN, a=a, lda=64, b=b, ldb=32, m=64,
                                                n=32, k=16, c=c, ldc=32, stream=0), **k})
    mm(m=0)                                                        # empty: no-op
    mm(n=0)
    for kw in (dict(form=2), dict(m=-1), dict(k=-1), dict(lda=63), dict(ldb=31), dict(ldc=31),
               dict(form=dl.DL_NT, lda=15), dict(form=dl.DL_NT, ldb=15, lda=16),
               dict(a=0), dict(c=0), dict(c=a + 4), dict(c=b), dict(y=c + 4),
               dict(m=(1 << 31) + 1), dict(m=1 << 24, n=1 << 17)):
        _expect(dl.DL_E_INVAL, mm, **kw)
    _expect(dl.DL_E_ALIGN, mm, c=c + 2)
    _expect(dl.DL_E_ALIGN, mm, y=b + (1 << 20) + 1)
    ws = FAKE + (1 << 32)
    wsb = dl.dl_matmul_workspace_bytes(64, 64, 16, True)
    assert wsb == 2 * 128 * 128 * 4            # 4 K-tiles: one workgroup, two slots
    _expect(dl.DL_E_INVAL, mm, symmetric=True)                     # 64 x 32 is not square
    _expect(dl.DL_E_ALIGN, mm, workspace=ws + 16, workspace_bytes=1 << 20)
    _expect(dl.DL_E_INVAL, mm, workspace=c - 256, workspace_bytes=1 << 20)    # overlaps C
    _expect(dl.DL_E_INVAL, mm, workspace=a, workspace_bytes=1 << 20)          # overlaps A
    _expect(dl.DL_E_INVAL, mm, workspace=ws, workspace_bytes=-1)


def test_matmul_batch_host_rules():
    a, b, c = FAKE, FAKE + (1 << 28), FAKE + (1 << 29)
    mm = lambda **k: dl.dl_matmul_f32_batch(**{**dict(
        form=dl.DL_NT, a=a, lda=16, stride_a=64 * 16, b=b, ldb=16, stride_b=32 * 16, m=64, n=32,
        k=16, c=c, ldc=32, stride_c=64 * 32, batch=4, stream=0), **k})
    for kw in (dict(batch=0), dict(batch=65), dict(stride_c=64 * 32 - 1),   # results overlap
               dict(stride_a=-1), dict(c=a + 4 * 64 * 16 * 3),             # C meets A's last matrix
               dict(y=c + 4, stride_y=64 * 32)):                           # Y meets C, not equal
        _expect(dl.DL_E_INVAL, mm, **kw)
    assert dl.dl_matmul_workspace_bytes_batch(2048, 2048, 2048, True, 8) == 2 * 512 * 128 * 128 * 4
    assert dl.dl_matmul_workspace_bytes_batch(64, 32, 16, False, 1) == \
        dl.dl_matmul_workspace_bytes(64, 32, 16, False)
    for bad in ((64, 32, 16, False, 0), (64, 64, 16, True, 65), (64, 32, 16, True, 2)):
        _expect(dl.DL_E_INVAL, dl.dl_matmul_workspace_bytes_batch, *bad)


def test_matmul_workspace_sizes():
    """Stream-K: two partial slots per workgroup; up to 512 workgroups (two
    per CU), each with at least 8 K-tiles of 32, in multiples of 8 (one per
    XCD).  Split-K (fewer tiles than 512 over a long K): one slot per (K
    range, tile) unit, S ranges of at least 64 K-tiles filling R rounds of
    512 units, taken when the busiest workgroup stays within 3% of an even
    split."""
    tile = 128 * 128 * 4
    full = 2 * 512 * tile
    # 136 upper tiles x 2305 K-tiles: S = 15 ranges of 154 (4 rounds)
    assert dl.dl_matmul_workspace_bytes(2048, 2048, 73760, True) == 136 * 15 * tile
    # 36 upper tiles x 896 K-tiles: S = 14 ranges of 64 (1 round)
    assert dl.dl_matmul_workspace_bytes(1024, 1024, 28672, True) == 36 * 14 * tile
    # 16 tiles x 2048 K-tiles: 32 ranges of 64; 1 tile x 32768: 512 of 64
    assert dl.dl_matmul_workspace_bytes(512, 512, 65536, False) == 16 * 32 * tile
    assert dl.dl_matmul_workspace_bytes(100, 100, 1 << 20, False) == 512 * tile
    # too short a K for ranges of 64 K-tiles to fill the rounds: stream-K
    assert dl.dl_matmul_workspace_bytes(512, 512, 40000, False) == full
    assert dl.dl_matmul_workspace_bytes(2048, 2048, 5632, True) == full
    assert dl.dl_matmul_workspace_bytes(2048, 2048, 2048, True) == full
    assert dl.dl_matmul_workspace_bytes(2048, 2048, 2048, False) == full
    assert dl.dl_matmul_workspace_bytes(5632, 2048, 2048, False) == full
    # 136 upper tiles x 4 K-tiles = 544 units: 68 workgroups, rounded to 64
    assert dl.dl_matmul_workspace_bytes(2048, 2048, 100, True) == 2 * 64 * tile
    # one tile of 32 K-tiles: 4 workgroups
    assert dl.dl_matmul_workspace_bytes(100, 100, 1000, False) == 2 * 4 * tile
    assert dl.dl_matmul_workspace_bytes(0, 5, 5, False) == 0
    for bad in ((5, 6, 7, True), (-1, 5, 5, False), (5, 5, -1, False)):
        _expect(dl.DL_E_INVAL, dl.dl_matmul_workspace_bytes, *bad)
    # the polar workspace includes the largest partial buffer of its products
    ws = dl.dl_polar_workspace_bytes(2048, 2048)
    assert ws >= 2 * 2048 * 2048 * 4 * 2 + full


def test_matmul_large_tiles_query():
    """Which kernel a shape's main block runs on (asked on the host, nothing
    launched): large tiles need K a multiple of 16, at least one whole row
    and column of 256 x 256 tiles, enough of them to fill the CUs (the last
    round's tiles possibly cut along K, within the workspace), and for a
    symmetric result M a multiple of 256."""
    full = dl.dl_matmul_workspace_bytes_batch(2048, 2048, 2048, True, 36)
    assert dl.dl_matmul_large_tiles(2048, 2048, 2048, True, 36, full)
    assert not dl.dl_matmul_large_tiles(2048, 2048, 2048, True, 36, 0)    # its tail needs pieces
    assert dl.dl_matmul_large_tiles(2048, 2048, 2048, False, 4, 0)        # 256 whole tiles
    assert not dl.dl_matmul_large_tiles(2048, 2048, 2040, False, 4, 0)    # K % 16
    assert not dl.dl_matmul_large_tiles(2048, 2048, 2048, False, 3, 0)    # 192 tiles
    assert not dl.dl_matmul_large_tiles(2000, 2000, 4096, True, 36, full)
    assert not dl.dl_matmul_large_tiles(255, 4096, 4096, False, 64, full)
    assert not dl.dl_matmul_large_tiles(0, 5, 5, False, 1, 0)
    for bad in ((5, 6, 7, True, 1, 0), (-1, 5, 5, False, 1, 0), (5, 5, 5, False, 0, 0),
                (5, 5, 5, False, 1, -1)):
        _expect(dl.DL_E_INVAL, dl.dl_matmul_large_tiles, *bad)


def test_participants_capacity():
    lib = dl.raw_lib()
    import ctypes
    r = dl.dl_round_begin(1, dl.DL_MEAN, 1000, OFFS1, 1, 4, FAKE, stream=0)
    try:
        c = ctypes.c_int()
        buf = (ctypes.c_int * 1)()
        assert lib.dl_round_participants(r.handle, 0, ctypes.byref(c), buf, 0) == dl.DL_OK
        assert c.value == 0
        assert lib.dl_round_participants(r.handle, 0, None, None, 0) == dl.DL_E_INVAL
        assert lib.dl_round_begin(None, 1, 0, 10, 1, None, 1, 1, None, None) == dl.DL_E_INVAL
        assert lib.dl_round_end(None) == dl.DL_OK
    finally:
        dl.dl_round_end(r)


def _kernel_instr_counts(asm_text):
    counts = collections.OrderedDict()
    cur = None
    for line in asm_text.split("\n"):
        m = re.match(r"^(_ZN3dlk\S*):", line)
        if m:
            cur = m.group(1)
            counts[cur] = collections.Counter()
            continue
        if cur and line.startswith(".Lfunc_end"):
            cur = None
        if cur:
            m = re.match(r"^\s+(v_\w+)", line)
            if m:
                counts[cur][m.group(1)] += 1
    return counts


def test_isa_has_no_contraction_and_ieee_division(tmp_path):
    """Every fused multiply-add in the gfx950 code belongs to the correctly
    rounded division sequence (3 v_fma_f32 + 2 v_fmac_f32 per v_div_fixup_f32);
    the folds and the EMA have none; no packed fp32 instruction appears."""
    asm = open(cabuild.device_asm(str(tmp_path / "k.s"))).read()
    counts = _kernel_instr_counts(asm)
    assert len(counts) >= 40
    for name, c in counts.items():
        fixups = c.get("v_div_fixup_f32", 0)
        assert c.get("v_fma_f32", 0) == 3 * fixups, name
        assert c.get("v_fmac_f32_e32", 0) + c.get("v_fmac_f32_e64", 0) == 2 * fixups, name
        assert c.get("v_rcp_f32_e32", 0) + c.get("v_rcp_f32_e64", 0) == fixups, name
        assert not [k for k in c if k.startswith(("v_pk_fma", "v_pk_mul_f32", "v_pk_add_f32",
                                                  "v_mad", "v_fmamk", "v_fmaak"))], name
        if "Close" in name or "SnapshotMean" in name:
            assert fixups > 0, name      # the means and the Nesterov closes divide
        else:
            assert fixups == 0, name     # folds and the EMA do not


def test_orthogonalisation_isa(tmp_path):
    """The product kernel runs on fp32 MFMA with no scratch and no packed fp32
    arithmetic; its epilogue multiplies and adds separately (no contraction)."""
    asm = open(cabuild.device_asm(str(tmp_path / "p.s"), source="polar.hip")).read()
    counts = _kernel_instr_counts(asm)
    gemms = [n for n in counts if "k_gemm" in n]
    assert len(gemms) == 4   # general and large-tile, each k-major and row-major
    for name, c in counts.items():
        assert not [k for k in c if k.startswith(("v_pk_fma", "v_pk_mul_f32", "v_pk_add_f32",
                                                  "v_mad_f32", "v_fmamk", "v_fmaak",
                                                  "v_fma_f32", "v_fmac_f32"))], name
    for name in gemms:
        assert counts[name].get("v_mfma_f32_32x32x2_f32", 0) >= 32, name
    assert "scratch_" not in asm
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)
    assert sizes and all(int(s) == 0 for s in sizes)


def test_noalloc_step_host_rules():
    """The allocation-free outer step: a matrix whose workspace exceeds the
    library's scratch is refused before anything else runs; so are bad sizes,
    steps and overlapping or unaligned matrices."""
    t, a = FAKE, FAKE + (1 << 34)
    step = lambda **k: dl.dl_outer_orthogonal_step_noalloc(**{**dict(
        theta=t, averaged=a, rows=300, cols=200, scale=0.1, stream=0), **k})
    assert dl.dl_polar_workspace_bytes(73760, 2048) > dl.DL_NOALLOC_SCRATCH_BYTES
    assert dl.dl_polar_workspace_bytes(5632, 2048) <= dl.DL_NOALLOC_SCRATCH_BYTES
    assert dl.dl_polar_workspace_bytes(50304, 128) <= dl.DL_NOALLOC_SCRATCH_BYTES
    _expect(dl.DL_E_TOO_LARGE, step, rows=73760, cols=2048)
    _expect(dl.DL_E_TOO_LARGE, step, rows=2048, cols=73760)
    _expect(dl.DL_E_INVAL, step, rows=0)
    _expect(dl.DL_E_INVAL, step, quintic_steps=0, cubic_steps=0)
    _expect(dl.DL_E_INVAL, step, cubic_steps=65)
    _expect(dl.DL_E_INVAL, step, averaged=t + 4 * 1000)            # overlaps theta
    _expect(dl.DL_E_INVAL, step, theta=0)
    _expect(dl.DL_E_ALIGN, step, theta=t + 2)
    assert dl.dl_strerror(dl.DL_E_TOO_LARGE) != "unknown status"
