"""Random calls of the several-arrival entry points on the CPU (no GPU: every
call that passes the host rules stops at the device checks with DL_E_HIP).
Whatever the arguments (worker ids out of range or repeated, stale tags,
misaligned or overlapping pointers, zero or negative token counts, counts
out of range), each call returns a documented status, launches nothing and
leaves the handle unchanged; the status is the one the host rules give for
the first failing arrival."""
import pytest
import torch
from hypothesis import given, settings, strategies as st

from checkpoint_averaging_amd import dlmerge as dl

FAKE = 0x7F0000000000          # never dereferenced
N = 1000
OFFS = [0, 96, 200, 1000]
MAXW = 6
TAG = 11
STATUSES = {dl.DL_E_INVAL, dl.DL_E_STALE, dl.DL_E_DUP, dl.DL_E_QUORUM, dl.DL_E_STATE,
            dl.DL_E_ALIGN, dl.DL_E_HIP}

arrival = st.tuples(
    st.integers(-2, MAXW + 1),                      # worker id
    st.sampled_from([TAG, TAG, TAG, TAG + 1]),      # tag
    st.sampled_from([0, 1, 2, 4, 16, 1 << 22, (1 << 22) + 2, 4 * 50]),   # ckpt offset
    st.sampled_from([1, 5, 250_000, 0, -3]),        # tokens
)


def expected(mode, frag, arrivals, dtype, with_global):
    """The first status the host rules give, arrival by arrival (None when
    every host rule passes)."""
    if frag < 0 or frag >= len(OFFS) - 1:
        return dl.DL_E_INVAL
    if not 1 <= len(arrivals) <= MAXW:
        return dl.DL_E_INVAL
    seen, total = set(), 0
    n = OFFS[frag + 1] - OFFS[frag]
    esize = 2 if dtype == dl.DL_BF16 else 4
    acc = (FAKE + 4 * OFFS[frag], FAKE + 4 * OFFS[frag] + 4 * n)
    g = FAKE + (1 << 24)
    th = (g + 4 * OFFS[frag], g + 4 * OFFS[frag] + 4 * n)
    for wid, tag, off, tok in arrivals:
        if not 0 <= wid < MAXW:
            return dl.DL_E_INVAL
        if tag != TAG:
            return dl.DL_E_STALE
        if wid in seen:
            return dl.DL_E_DUP
        if mode == dl.DL_MEAN:
            if with_global:
                return dl.DL_E_INVAL
        else:
            if not with_global or tok <= 0:
                return dl.DL_E_INVAL
            total += tok
        p = FAKE + off if off else 0
        if p == 0:
            return dl.DL_E_INVAL
        if p % esize:
            return dl.DL_E_ALIGN
        span = (p, p + esize * n)
        if span[0] < acc[1] and acc[0] < span[1]:
            return dl.DL_E_INVAL
        if mode != dl.DL_MEAN and span[0] < th[1] and th[0] < span[1]:
            return dl.DL_E_INVAL
        seen.add(wid)
    return None


@settings(max_examples=300, deadline=None)
@given(mode=st.sampled_from([dl.DL_MEAN, dl.DL_DELTA_NESTEROV]),
       frag=st.integers(-1, 3),
       arrivals=st.lists(arrival, min_size=0, max_size=MAXW + 2),
       bf16=st.booleans(), with_global=st.booleans())
def test_several_arrival_calls_fail_cleanly(mode, frag, arrivals, bf16, with_global):
    if torch.cuda.device_count() > 0:
        pytest.skip("the device checks would run on a GPU host")
    dtype = dl.DL_BF16 if bf16 else dl.DL_F32
    g = FAKE + (1 << 24) if with_global else None
    r = dl.dl_round_begin(TAG, mode, N, OFFS, 1, MAXW, FAKE, stream=0)
    try:
        ids = [a[0] for a in arrivals]
        tags = [a[1] for a in arrivals]
        cks = [FAKE + a[2] if a[2] else 0 for a in arrivals]
        toks = [a[3] for a in arrivals]
        with pytest.raises(dl.DLError) as ei:
            dl.dl_fold_checkpoints(r, frag, ids, tags, cks, global_=g,
                                   tokens=toks if mode != dl.DL_MEAN else None, dtype=dtype)
        want = expected(mode, frag, arrivals, dtype, with_global)
        got = ei.value.status
        assert got in STATUSES
        assert got == (dl.DL_E_HIP if want is None else want), (got, want)
        for f in range(len(OFFS) - 1):
            assert dl.dl_round_participants(r, f) == []
            assert dl.dl_round_tokens(r, f) == 0
    finally:
        dl.dl_round_end(r)
