"""Round rules of the C ABI that need real device buffers: duplicate and
late calls after successful folds, pointer-range checks against the HIP
allocation, and an abandoned round leaving global, momentum and EMA
untouched."""
import numpy as np
import pytest
import torch

from checkpoint_averaging_amd import dlmerge as dl

pytestmark = pytest.mark.gpu


def expect(status, fn, *a, **k):
    with pytest.raises(dl.DLError) as ei:
        fn(*a, **k)
    assert ei.value.status == status, (ei.value.status, status)


def test_round_rules_after_folds():
    n = 8192
    dev = torch.device("cuda")
    acc = torch.empty(n, device=dev)
    out = torch.empty(n, device=dev)
    c = [torch.randn(n, device=dev) for _ in range(3)]
    r = dl.dl_round_begin(4, dl.DL_MEAN, n, [0, 4096, n], 2, 3, acc)
    dl.dl_fold_checkpoint(r, 0, 1, 4, c[1][:4096])
    expect(dl.DL_E_DUP, dl.dl_fold_checkpoint, r, 0, 1, 4, c[1][:4096])
    expect(dl.DL_E_QUORUM, dl.dl_finalize_mean, r, 0, out)
    dl.dl_fold_checkpoint(r, 0, 2, 4, c[2][:4096])
    dl.dl_fold_checkpoint(r, 1, 1, 4, c[1][4096:])       # same worker, other fragment
    dl.dl_finalize_mean(r, 0, out)
    expect(dl.DL_E_STATE, dl.dl_fold_checkpoint, r, 0, 0, 4, c[0][:4096])
    expect(dl.DL_E_STATE, dl.dl_finalize_mean, r, 0, out)
    expect(dl.DL_E_QUORUM, dl.dl_finalize_mean, r, 1, out)
    assert dl.dl_round_participants(r, 0) == [1, 2]
    assert dl.dl_round_participants(r, 1) == [1]
    dl.dl_round_end(r)
    torch.cuda.synchronize()
    want = (c[1][:4096] + c[2][:4096]) / 2
    assert torch.equal(out[:4096], want)


class RawAlloc:
    """A device allocation made with hipMalloc directly, so its end is the
    end of the HIP allocation (torch's caching allocator may place a tensor
    inside a larger segment)."""

    def __init__(self, nbytes):
        import ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ptr = ctypes.c_void_p()
        assert self.hip.hipMalloc(ctypes.byref(self.ptr), ctypes.c_size_t(nbytes)) == 0
        self.nbytes = nbytes

    @property
    def addr(self):
        return self.ptr.value

    @property
    def end(self):
        return self.ptr.value + self.nbytes

    def free(self):
        torch.cuda.synchronize()
        assert self.hip.hipFree(self.ptr) == 0


def test_pointer_ranges_checked_against_allocation():
    n = 4096
    dev = torch.device("cuda")
    acc = torch.empty(n, device=dev)
    raw = RawAlloc(1 << 20)
    try:
        r = dl.dl_round_begin(1, dl.DL_MEAN, n, [0, n], 1, 2, acc)
        # a checkpoint whose span runs past the end of its allocation
        expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 0, 1, raw.end - 4 * 100,
               dtype=dl.DL_F32)
        # a host pointer
        host = np.zeros(n, np.float32)
        expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 0, 1, host.ctypes.data,
               dtype=dl.DL_F32)
        dl.dl_fold_checkpoint(r, 0, 0, 1, torch.ones(n, device=dev))
        # an output too short for the fragment
        expect(dl.DL_E_INVAL, dl.dl_finalize_mean, r, 0, raw.end - 4 * 10)
        # output partly overlapping the accumulator
        expect(dl.DL_E_INVAL, dl.dl_finalize_mean, r, 0, acc.data_ptr() + 16)
        dl.dl_finalize_mean(r, 0, acc)
        dl.dl_round_end(r)
        torch.cuda.synchronize()
        assert torch.equal(acc, torch.ones(n, device=dev))
        # the stand-alone EMA checks its spans too
        expect(dl.DL_E_INVAL, dl.dl_ema_update, raw.end - 64, acc, n=n)
    finally:
        raw.free()


def test_accumulator_past_allocation_rejected():
    dev = torch.device("cuda")
    raw = RawAlloc(4 << 20)
    try:
        n = 2 << 20                                   # the accumulator holds only half
        r = dl.dl_round_begin(1, dl.DL_MEAN, n, [0, n], 1, 2, raw.addr)
        expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 0, 1, torch.ones(n, device=dev))
        dl.dl_round_end(r)
    finally:
        raw.free()


def test_delta_rules_and_abandoned_round():
    n = 6000
    dev = torch.device("cuda")
    acc = torch.empty(n, device=dev)
    theta = torch.randn(n, device=dev)
    other = theta.clone()
    m = torch.randn(n, device=dev)
    e = torch.randn(n, device=dev)
    snap = [theta.clone(), theta.clone(), m.clone(), e.clone()]
    c = theta + 1e-3 * torch.randn(n, device=dev)
    r = dl.dl_round_begin(2, dl.DL_DELTA_NESTEROV, n, [0, 3000, n], 1, 4, acc)
    dl.dl_fold_checkpoint(r, 0, 0, 2, c[:3000], theta, 100)
    # the deltas of one fragment must be taken against one global
    expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 1, 2, c[:3000], other, 100)
    expect(dl.DL_E_INVAL, dl.dl_outer_nesterov, r, 0, other, m)
    # token total would overflow int64
    expect(dl.DL_E_INVAL, dl.dl_fold_checkpoint, r, 0, 1, 2, c[:3000], theta, (1 << 63) - 1)
    # momentum overlapping the global
    expect(dl.DL_E_INVAL, dl.dl_outer_nesterov, r, 0, theta, theta.data_ptr() + 4)
    dl.dl_fold_checkpoint(r, 1, 3, 2, c[3000:], theta, 7)
    assert dl.dl_round_tokens(r, 0) == 100 and dl.dl_round_tokens(r, 1) == 7
    dl.dl_round_end(r)                                 # abandoned: nothing closed
    torch.cuda.synchronize()
    assert torch.equal(theta, snap[0]) and torch.equal(m, snap[2]) and torch.equal(e, snap[3])


def test_streams_are_respected():
    """All work of a round goes to the round's stream."""
    n = 1 << 22
    s = torch.cuda.Stream()
    dev = torch.device("cuda")
    acc = torch.empty(n, device=dev)
    out = torch.empty(n, device=dev)
    c = [torch.full((n,), float(i + 1), device=dev) for i in range(4)]
    torch.cuda.synchronize()
    r = dl.dl_round_begin(3, dl.DL_MEAN, n, [0, n], 4, 4, acc, stream=s)
    for i in range(4):
        dl.dl_fold_checkpoint(r, 0, i, 3, c[i])
    dl.dl_finalize_mean(r, 0, out)
    dl.dl_round_end(r)
    s.synchronize()
    assert torch.equal(out, torch.full((n,), 2.5, device=dev))


def test_pending_hip_error_is_reported_and_left_pending():
    """A HIP error left pending on the thread by earlier work is reported as
    DL_E_HIP before anything is launched: the library does not clear it, the
    handle is unchanged, and after the caller clears it the same call goes
    through.  The pending error comes from a harmless failed runtime call
    (selecting a device ordinal that does not exist); no kernel faults."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    n = 4096
    dev = torch.device("cuda")
    acc = torch.full((n,), 7.0, device=dev)
    ck = torch.ones(n, device=dev)
    torch.cuda.synchronize()
    r = dl.dl_round_begin(11, dl.DL_MEAN, n, [0, n], 1, 2, acc)
    hip.hipGetLastError()                                    # start from a clear state
    assert hip.hipSetDevice(1 << 20) != 0                    # leaves an error pending
    assert hip.hipPeekAtLastError() != 0
    lib = dl.raw_lib()
    st = lib.dl_fold_checkpoint(r.handle, 0, 0, 11, ck.data_ptr(), dl.DL_F32, None, 0)
    assert st == dl.DL_E_HIP
    assert hip.hipPeekAtLastError() != 0                     # still pending: not cleared
    assert hip.hipGetLastError() != 0                        # the caller clears it
    assert dl.dl_round_participants(r, 0) == []              # handle unchanged
    torch.cuda.synchronize()
    assert torch.all(acc == 7.0)                             # nothing launched
    assert lib.dl_fold_checkpoint(r.handle, 0, 0, 11, ck.data_ptr(), dl.DL_F32, None, 0) == 0
    dl.dl_finalize_mean(r, 0, acc)
    dl.dl_round_end(r)
    torch.cuda.synchronize()
    assert torch.all(acc == 1.0)
    # the stand-alone calls report it the same way
    e = torch.zeros(n, device=dev)
    torch.cuda.synchronize()
    assert hip.hipSetDevice(1 << 20) != 0
    assert lib.dl_ema_update(e.data_ptr(), ck.data_ptr(), n, 0.5, None) == dl.DL_E_HIP
    assert hip.hipGetLastError() != 0
    assert lib.dl_ema_update(e.data_ptr(), ck.data_ptr(), n, 0.5, None) == 0
    torch.cuda.synchronize()
    assert torch.all(e == 0.5)


def test_several_arrival_rules_on_device_buffers():
    """The several-arrival calls: a rejected call (a checkpoint past its
    allocation, a duplicate, a checkpoint under an output) folds nothing, and
    the arrivals a later call folds are recorded in array order, after the
    one-arrival folds before it."""
    n = 4096
    dev = torch.device("cuda")
    acc = torch.empty(n, device=dev)
    out = torch.empty(n, device=dev)
    c = [torch.randn(n, device=dev) for _ in range(4)]
    raw = RawAlloc(1 << 20)
    try:
        r = dl.dl_round_begin(6, dl.DL_MEAN, n, [0, n], 3, 4, acc)
        dl.dl_fold_checkpoint(r, 0, 2, 6, c[2])
        expect(dl.DL_E_INVAL, dl.dl_fold_checkpoints, r, 0, [0, 1], 6,
               [c[0], raw.end - 4 * 100], dtype=dl.DL_F32)            # past its allocation
        expect(dl.DL_E_DUP, dl.dl_fold_checkpoints, r, 0, [0, 2], 6, [c[0], c[2]])
        expect(dl.DL_E_INVAL, dl.dl_fold_checkpoints_and_finalize_mean, r, 0, [0, 1], 6,
               [c[0], c[1]], c[1])                                    # output over a checkpoint
        assert dl.dl_round_participants(r, 0) == [2]
        dl.dl_fold_checkpoints_and_finalize_mean(r, 0, [3, 0], 6, [c[3], c[0]], out)
        assert dl.dl_round_participants(r, 0) == [2, 3, 0]
        expect(dl.DL_E_STATE, dl.dl_fold_checkpoints, r, 0, [1], 6, [c[1]])
        dl.dl_round_end(r)
        torch.cuda.synchronize()
        h = [x.cpu().numpy() for x in c]
        want = ((h[2] + h[3]) + h[0]) / np.float32(3)         # binary32, IEEE division
        assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
    finally:
        raw.free()
