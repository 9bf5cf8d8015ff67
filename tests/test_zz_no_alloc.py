"""GPU test of the allocation-free decoder step (rlt_decoder_step_noalloc).

It is the same transition as rlt_decoder_step with the duplicate-row
counters kept in the library's fixed device array, so its results must equal
rlt_decoder_step's bit for bit (same kernels, same launch shapes): checked on
two calls in a row, the second with fewer rows, through the C ABI; then under
a caller's own graph capture (which fails on any device allocation), replayed
several times with eager work between the replays and every replay checked.
"""
import numpy as np
import pytest

import synth
from tests.gpu_common import GpuRun, require_gpu, torch

pytestmark = pytest.mark.gpu

WL = synth.SMALL.with_(B=8, T=24)


def _pair():
    a = GpuRun(WL)
    b = GpuRun(WL, raw=a.raw)
    a.init(poison=True)   # every cache slot defined (NaN until written)
    b.init(poison=True)
    torch.cuda.synchronize()  # later calls may run on other streams
    return a, b


def _outs(n):
    return dict(s_out=torch.empty((n, WL.d), device="cuda"), logits=torch.empty((n, WL.V), device="cuda"),
                argmax=torch.empty(n, dtype=torch.int32, device="cuda"))


def _same_state(a, b):
    """Bitwise (the unwritten cache slots hold the same NaN pattern)."""
    bits = lambda t: t.view(torch.int16)
    return (torch.equal(a.st.s, b.st.s) and torch.equal(a.st.pos, b.st.pos) and
            torch.equal(bits(a.st.ring("k")), bits(b.st.ring("k"))) and
            torch.equal(bits(a.st.ring("v")), bits(b.st.ring("v"))))


def test_noalloc_step_equals_decoder_step():
    require_gpu()
    a, b = _pair()
    for idx in (list(range(8)), [5, 2]):          # the second call is smaller
        rows = a.rows(idx)
        t = int(a.st.pos[idx[0]]) + 1
        e = a.Ed[torch.tensor(idx, device="cuda"), t - 1].contiguous()
        oa, ob = _outs(len(idx)), _outs(len(idx))
        assert a.dec.step(a.st, rows, e, a.mem, **oa) == 0
        assert b.dec.step(b.st, rows, e, b.mem, noalloc=True, **ob) == 0
        torch.cuda.synchronize()
        for k in oa:
            assert torch.equal(oa[k], ob[k]), (idx, k)
        assert _same_state(a, b), idx
    assert a.dec.sync_error() == 0 and b.dec.sync_error() == 0


def test_noalloc_step_limits_and_duplicate_rows():
    require_gpu()
    from stateful_sequence_model_amd import _abi as A
    a, b = _pair()
    rows = a.rows([1, 3, 1])
    e = a.Ed[[1, 3, 1], 0].contiguous()
    # duplicate rows: device-detected, those slots skipped, the others done
    assert b.dec.step(b.st, rows, e, b.mem, noalloc=True) == 0
    assert b.dec.sync_error() == A.RLT_EINVAL
    assert int(b.st.pos[1]) == 0 and int(b.st.pos[3]) == 1
    # the counters were cleared: the same rows once each succeed
    assert b.dec.step(b.st, b.rows([1]), e[:1], b.mem, noalloc=True) == 0
    assert b.dec.sync_error() == 0 and int(b.st.pos[1]) == 1
    # refused before anything is enqueued: the captured-graph flag, a state
    # beyond the fixed array (only the size field is changed; nothing runs)
    assert b.dec.step(b.st, b.rows([0]), e[:1], b.mem, noalloc=True, graph=True) == A.RLT_EINVAL
    io = A.rlt_step_io()
    io.n, io.rows, io.e, io.mem = 1, b.rows([0]).data_ptr(), e.data_ptr(), b.mem
    st = b.st.c()
    st.B_cap = A.RLT_NOALLOC_MAX_ROWS + 1
    assert A.rlt_decoder_step_noalloc(b.dec.ctx, st, io, torch.cuda.current_stream().cuda_stream) == A.RLT_ESHAPE
    torch.cuda.synchronize()
    assert int(b.st.pos[0]) == 0


def test_noalloc_step_inside_a_callers_graph_capture():
    """Captured by the caller (global capture mode: a device allocation
    during the capture would fail it), then replayed four times with eager
    work between replays; each replay equals an eager rlt_decoder_step."""
    require_gpu()
    a, b = _pair()
    idx = list(range(6))
    rows = a.rows(idx)
    e = a.Ed[torch.tensor(idx, device="cuda"), 0].contiguous()   # the same e each step
    ob = _outs(len(idx))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())  # rows and e were made on the default stream
    with torch.cuda.stream(stream):
        # one eager allocation-free step first (both states advance)
        assert b.dec.step(b.st, rows, e, b.mem, noalloc=True, **ob) == 0
    oa = _outs(len(idx))
    assert a.dec.step(a.st, rows, e, a.mem, **oa) == 0
    torch.cuda.synchronize()
    assert _same_state(a, b)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        rc = b.dec.step(b.st, rows, e, b.mem, noalloc=True, **ob)
    assert rc == 0
    torch.cuda.synchronize()
    for r in range(4):
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        g.replay()
        assert a.dec.step(a.st, rows, e, a.mem, **oa) == 0
        torch.cuda.synchronize()
        del junk
        for k in oa:
            assert torch.equal(oa[k], ob[k]), (r, k)
        assert _same_state(a, b), r
    assert a.dec.sync_error() == 0 and b.dec.sync_error() == 0
