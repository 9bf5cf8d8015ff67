"""GPU tests of the recurrence, the state bookkeeping and the readout.

Bit-exact where the same kernels see the same inputs in the same launch
shape (replay vs incremental steps, Prop. 3.1 split invariance, graph vs
direct launches, causality with NaN-poisoned unread data); within the float
tolerances of test_gpu_parity otherwise; exact for every integer result.
"""
import math

import numpy as np
import pytest

import synth
from oracle import Memory, Oracle, behaviour_logprobs, replay as oracle_replay
from tests.gpu_common import GpuRun, require_gpu, torch
from tests.helpers import memory_of, oracle_config, oracle_weights, rel_l2, widen

pytestmark = pytest.mark.gpu

SMALL = synth.SMALL.with_(B=6, T=48)


def _steps(run, idx, n, **kw):
    S, Z = run.run(n, idx, **kw)
    return S, Z


def test_replay_equals_incremental_steps_bitexact():
    """Replay from H_0 (App. A.4) gives bit-identical s_t, log-probs and
    final state to init + the same transitions issued one call per token."""
    require_gpu()
    run = GpuRun(SMALL)
    B, T = run.B, run.T
    tokens = torch.from_numpy(synth.make_tokens(SMALL, 0, B, T)).cuda()
    lens = np.full(B, T, dtype=np.int32)
    splits = np.full(B, 1, dtype=np.int32)
    logp = torch.full((B, T), float("nan"), device="cuda")
    s_trace = torch.zeros((B, T, SMALL.d), device="cuda")
    assert run.dec.replay(run.st, lens, splits, run.Ed, run.mem, tokens, logp, s_trace=s_trace) == 0
    torch.cuda.synchronize()
    ring_k = run.st.ring("k").clone()
    pend = run.st.pending.clone()
    # incremental
    run2 = GpuRun(SMALL)
    run2.init()
    s_out = torch.empty((B, SMALL.d), device="cuda")
    lp = torch.empty(B, device="cuda")
    for t in range(1, T):
        rc = run2.step(range(B), t, s_out=s_out, score_tok=tokens[:, t].contiguous(), logp=lp)
        assert rc == 0
        assert torch.equal(s_out, s_trace[:, t - 1]), t
        assert torch.equal(lp, logp[:, t]), t
    torch.cuda.synchronize()
    assert torch.equal(run2.st.ring("k"), ring_k)
    assert torch.equal(run.st.pos.cpu(), torch.full((B,), T - 1, dtype=torch.int32))
    assert torch.equal(pend.cpu(), tokens[:, T - 1].cpu())          # x_len left pending
    assert torch.isnan(logp[:, 0]).all()                            # t = 0 never scored


def test_replay_graph_runs_equal_direct_launches():
    """Replay on a side stream captures each run of ticks with one active set
    as a graph (the position advances on the device) and replays it; with
    capture off (every tick launched directly) or on for every run, the
    log-probs, the state trace and the final state are bit-identical. Ragged
    lengths give runs shorter and longer than the capture threshold."""
    require_gpu()
    wl = SMALL.with_(B=6, T=40)
    lens = np.array([40, 33, 33, 20, 9, 3], dtype=np.int32)
    splits = np.array([1, 5, 2, 1, 3, 1], dtype=np.int32)
    out = {}
    raw = None
    for name, gmin in (("direct", -1), ("default", 0), ("every", 1)):
        run = GpuRun(wl, raw=raw, launch={"replay_graph_min": gmin})
        raw = run.raw
        B, T = run.B, run.T
        tokens = torch.from_numpy(synth.make_tokens(wl, 0, B, T)).cuda()
        logp = torch.full((B, T), float("nan"), device="cuda")
        s_trace = torch.zeros((B, T, wl.d), device="cuda")
        run.st.ring_k.zero_()  # slots the short sequences never write: equal in every run
        run.st.ring_v.zero_()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            assert run.dec.replay(run.st, lens, splits, run.Ed, run.mem, tokens, logp, s_trace=s_trace,
                                  stream=side.cuda_stream) == 0
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert run.dec.sync_error() == 0
        out[name] = (logp.cpu(), s_trace.cpu(), run.st.pos.cpu(), run.st.pending.cpu(), run.st.ring("k").cpu(),
                     run.st.s.cpu())
        run.dec.close()
    ref = out["direct"]
    for name in ("default", "every"):
        for a, b in zip(out[name], ref):
            assert torch.equal(a.view(torch.int32) if a.is_floating_point() else a,
                               b.view(torch.int32) if b.is_floating_point() else b), name
    assert torch.equal(ref[2], torch.from_numpy(lens - 1))


def test_split_invariance_prop_3_1_bitexact():
    """Prop. 3.1: replaying a prefix then stepping equals replaying the
    whole history, for several split points."""
    require_gpu()
    B, T = 4, 40
    wl = SMALL.with_(B=B, T=T)
    tokens = torch.from_numpy(synth.make_tokens(wl, 0, B, T)).cuda()
    ref = GpuRun(wl)
    lp_full = torch.zeros((B, T), device="cuda")
    tr_full = torch.zeros((B, T, wl.d), device="cuda")
    ref.dec.replay(ref.st, np.full(B, T, np.int32), np.ones(B, np.int32), ref.Ed, ref.mem, tokens, lp_full,
                   s_trace=tr_full)
    torch.cuda.synchronize()
    for T0 in (2, 15, 16, 33):
        run = GpuRun(wl)
        lp = torch.zeros((B, T), device="cuda")
        run.dec.replay(run.st, np.full(B, T0 + 1, np.int32), np.ones(B, np.int32), run.Ed, run.mem, tokens, lp)
        s_out = torch.empty((B, wl.d), device="cuda")
        lpt = torch.empty(B, device="cuda")
        for t in range(T0 + 1, T):
            assert run.step(range(B), t, s_out=s_out, consume_tok=tokens[:, t - 1].contiguous(),
                            score_tok=tokens[:, t].contiguous(), logp=lpt) == 0
            assert torch.equal(s_out, tr_full[:, t - 1]), (T0, t)
            assert torch.equal(lpt, lp_full[:, t]), (T0, t)
        torch.cuda.synchronize()
        assert torch.equal(lp[:, 1:T0 + 1], lp_full[:, 1:T0 + 1])


def test_graph_replays_equal_direct_launches():
    """The captured step replayed many times (with eager work between the
    replays) gives the same states as direct launches."""
    require_gpu()
    wl = SMALL.with_(B=5, T=40)
    a, b = GpuRun(wl), GpuRun(wl)
    a.init()
    b.init()
    rows = a.rows()
    stream = torch.cuda.Stream()
    e_fixed = a.Ed[:, 0].contiguous()
    argmax_a = torch.empty(wl.B, dtype=torch.int32, device="cuda")
    argmax_b = torch.empty(wl.B, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        for i in range(12):
            assert a.dec.step(a.st, rows, e_fixed, a.mem, argmax=argmax_a, graph=True) == 0
            assert b.dec.step(b.st, rows, e_fixed, b.mem, argmax=argmax_b, graph=False) == 0
            stream.synchronize()
            junk = torch.randn(1000, device="cuda").sum()  # eager work between replays
            assert torch.equal(a.st.s, b.st.s), i
            assert torch.equal(argmax_a, argmax_b), i
    assert torch.equal(a.st.pos, b.st.pos) and int(a.st.pos[0]) == 12
    # slots 0..11 hold positions 1..12 (W-1 = 15 slots; the rest never written)
    assert torch.equal(a.st.ring("v")[:, :, :12], b.st.ring("v")[:, :, :12])
    assert torch.equal(a.st.ring("k")[:, :, :12], b.st.ring("k")[:, :, :12])


def test_causality_with_poisoned_unread_data():
    """Prop. B.1 / report §4.2: NaN in memory positions j > t, in e beyond
    the current token, and in every cache slot at H_0 (the ring before it is
    written) must not reach any output: all outputs finite and bit-identical
    to the unpoisoned run."""
    require_gpu()
    wl = SMALL.with_(B=3, T=40)
    nsteps = 30
    clean = GpuRun(wl)
    clean.init()
    S0, Z0 = clean.run(nsteps)
    dirty = GpuRun(wl)
    nan = torch.tensor(float("nan"), dtype=dirty.cfg.torch_dtype)
    dirty.mkd[:, :, nsteps:] = nan.cuda()
    dirty.mvd[:, :, nsteps:] = nan.cuda()
    dirty.Ed[:, nsteps:] = nan.cuda()
    dirty.init(poison=True)
    assert torch.isnan(dirty.st.ring("k")).all()
    S1, Z1 = dirty.run(nsteps)
    assert np.isfinite(S1).all() and np.isfinite(Z1).all()
    assert np.array_equal(S0, S1) and np.array_equal(Z0, Z1)


def test_batch_composition_independence():
    """A sequence's results do not depend on which other sequences share the
    call, or their order [RLT §3.1 Prop. 3.1, §4.1]: bit for bit within one
    context, since every reduction order is fixed by the config and the
    context's capacities, not by the call's row count."""
    require_gpu()
    wl = SMALL.with_(B=8, T=40)
    full = GpuRun(wl)
    full.init()
    S, Z = full.run(20)
    part = GpuRun(wl, raw=full.raw)
    part.init([5, 2])
    S2, Z2 = part.run(20, [5, 2])
    one = GpuRun(wl, raw=full.raw)
    one.init([6])
    S4, Z4 = one.run(20, [6])
    for j, b in enumerate((5, 2)):
        assert np.array_equal(S2[:, j], S[:, b]) and np.array_equal(Z2[:, j], Z[:, b]), b
    assert np.array_equal(S4[:, 0], S[:, 6]) and np.array_equal(Z4[:, 0], Z[:, 6])
    # same call size, permuted rows
    perm = GpuRun(wl, raw=full.raw)
    perm.init()
    order = [7, 3, 0, 1, 6, 2, 5, 4]
    S3, Z3 = perm.run(20, order)
    for j, b in enumerate(order):
        assert np.array_equal(S3[:, j], S[:, b]) and np.array_equal(Z3[:, j], Z[:, b])


@pytest.mark.timeout(600)
def test_batch_invariance_across_product_tiles():
    """Mid width (d=1024, 16x64 heads, W=128) in a 96-row context: calls of
    96, 40, 7 and 1 rows take different product tiles (64 x 2 pairs, 64 x 1,
    32 x 1), yet every row's states and logits are bit-identical to its
    results in the full call."""
    require_gpu()
    wl = synth.MID.with_(T=24, L=3)
    B, n = 96, 6
    full = GpuRun(wl, B=B, T=wl.T)
    full.init()
    S, Z = full.run(n)
    for sub in ([3, 50] + list(range(58, 96)), [10, 20, 30, 40, 50, 60, 70], [41]):
        part = GpuRun(wl, raw=full.raw, B=B, T=wl.T)
        part.init(sub)
        S2, Z2 = part.run(n, sub)
        for j, b in enumerate(sub):
            assert np.array_equal(S2[:, j], S[:, b]) and np.array_equal(Z2[:, j], Z[:, b]), (len(sub), b)
        part.dec.close()


def test_every_product_shape_bit_identical():
    """Mid width (K = 1024 and 2816: 16 and 44 chunks of 64, so stream groups
    of 2 to 44 chunks and every tail of the staged tile's unrolled loop) at 1,
    3, 8, 40 and 128 rows: each operand-order product shape the launcher can be
    told to take -- register tile of 32 or 64 rows x 1 or 2 column pairs with
    1-4 chunks in flight and the epilogue values loaded before or after the K
    loop; staged tile of 128 x 64 or 64 x 128 over 1, 2, 4 or 8 stream
    groups (with the combine kernel below 8 streams per group) -- gives
    states and logits
    bit-identical to the default shapes (at 1 row: the register tile with
    the activations staged in LDS): the stream tree fixes the summation
    order, the tile does not."""
    require_gpu()
    from stateful_sequence_model_amd import _abi
    wl = synth.MID.with_(T=24, L=2)
    raw = synth.make_weights(wl)
    shapes = [(1, 1, 0, 2, 0), (1, 1, 0, 2, 1), (1, 1, 0, 3, 0), (1, 1, 0, 3, 1), (1, 1, 0, 4, 0), (2, 1, 0, 1, 1),
              (2, 1, 0, 2, 0), (1, 2, 0, 1, 1), (1, 2, 0, 2, 0), (1, 1, 1, 1, 0), (1, 1, 2, 1, 0), (1, 1, 4, 1, 0),
              (1, 1, 8, 1, 0), (1, 4, 1, 1, 0), (1, 4, 2, 1, 0), (1, 4, 4, 1, 0), (1, 4, 8, 1, 0)]
    for B in (1, 3, 8, 40, 128):
        base = GpuRun(wl, raw=raw, B=B, T=wl.T)
        base.init()
        S, Z = base.run(3)
        base.dec.close()
        for sh in shapes:
            run = GpuRun(wl, raw=raw, B=B, T=wl.T)
            _abi.check(_abi.rlt_dbg_product_shape(run.dec.ctx, *sh), "product shape")
            run.init()
            S2, Z2 = run.run(3)
            assert run.dec.sync_error() == 0
            assert np.array_equal(S2, S) and np.array_equal(Z2, Z), (B, sh)
            run.dec.close()
        if B == 1:  # the one-row tile with 3 and 4 weight chunks in flight
            for pf in (3, 4):
                run = GpuRun(wl, raw=raw, B=B, T=wl.T, launch={"one_row_pf": pf})
                run.init()
                S2, Z2 = run.run(3)
                assert run.dec.sync_error() == 0
                assert np.array_equal(S2, S) and np.array_equal(Z2, Z), (B, "one_row_pf", pf)
                run.dec.close()


def test_staged_tile_copied_straight_into_lds_bit_identical():
    """The staged product tile of 64 rows x 4 column pairs with its chunks
    copied from memory straight into LDS (the default) gives the bits of the
    register-staged tile (launch option no_lt_dma): default shapes at 128 and
    96 rows (one and two stream groups), and forced shapes over 1, 2, 4 and 8
    groups (group lengths of 2 to 44 chunks, every tail of the four-chunk
    loop; at the small width, K of 256 and 704, groups of 0 and 1 chunks),
    two and one activation terms."""
    require_gpu()
    from stateful_sequence_model_amd import _abi
    for wl, sizes in ((synth.MID.with_(T=24, L=2), (96, 128)), (synth.SMALL.with_(T=24, B=128), (128,))):
        _copied_tile_case(_abi, wl, sizes)


def _copied_tile_case(_abi, wl, sizes):
    raw = synth.make_weights(wl)
    for one in (0, 1):
        for B in sizes:
            base = GpuRun(wl, raw=raw, B=B, T=wl.T, launch={"one_term": one, "no_lt_dma": 1})
            base.init()
            S, Z = base.run(3)
            base.dec.close()
            for sh in (None, (1, 4, 1, 1, 0), (1, 4, 2, 1, 0), (1, 4, 4, 1, 0), (1, 4, 8, 1, 0)):
                run = GpuRun(wl, raw=raw, B=B, T=wl.T, launch={"one_term": one})
                if sh:
                    _abi.check(_abi.rlt_dbg_product_shape(run.dec.ctx, *sh), "product shape")
                run.init()
                S2, Z2 = run.run(3)
                assert run.dec.sync_error() == 0
                assert np.array_equal(S2, S) and np.array_equal(Z2, Z), (one, B, sh)
                run.dec.close()


def test_one_term_activations_shapes_and_closeness():
    """The one-term activation mode (launch option one_term: the products'
    activations as one bf16 value, the kernels' single-term instantiations)
    at 1, 40 and 128 rows: bit-identical across product shapes, and close to
    the two-term results (relative L2 of the states and logits within 2e-2
    after 3 steps: only the activations' rounding differs)."""
    require_gpu()
    from stateful_sequence_model_amd import _abi
    wl = synth.MID.with_(T=24, L=2)
    raw = synth.make_weights(wl)
    shapes = [(1, 1, 0, 2, 0), (1, 1, 0, 3, 1), (1, 1, 2, 1, 0), (1, 1, 8, 1, 0), (1, 4, 1, 1, 0), (1, 4, 4, 1, 0)]
    for B in (1, 40, 128):
        two = GpuRun(wl, raw=raw, B=B, T=wl.T)
        two.init()
        S2, Z2 = two.run(3)
        two.dec.close()
        base = GpuRun(wl, raw=raw, B=B, T=wl.T, launch={"one_term": 1})
        base.init()
        S, Z = base.run(3)
        base.dec.close()
        assert rel_l2(S, S2) < 2e-2 and rel_l2(Z, Z2) < 2e-2, (B, rel_l2(S, S2), rel_l2(Z, Z2))
        assert not np.array_equal(S, S2)  # the mode is in effect
        for sh in shapes:
            run = GpuRun(wl, raw=raw, B=B, T=wl.T, launch={"one_term": 1})
            _abi.check(_abi.rlt_dbg_product_shape(run.dec.ctx, *sh), "product shape")
            run.init()
            S3, Z3 = run.run(3)
            assert run.dec.sync_error() == 0
            assert np.array_equal(S3, S) and np.array_equal(Z3, Z), (B, sh)
            run.dec.close()


def test_duplicate_rows_are_refused_on_device():
    """A decoder call naming one state row in two slots would let two
    workgroups update the same row: the library detects it on the device,
    skips those slots (their rows stay unchanged), processes the others and
    reports RLT_EINVAL on the next call; the detection leaves nothing behind
    (the following call is clean)."""
    require_gpu()
    from stateful_sequence_model_amd import _abi as A
    wl = SMALL.with_(B=4, T=16)
    run = GpuRun(wl)
    run.init()
    run.run(2)
    before_s = run.st.s.clone()
    before_pos = run.st.pos.clone()
    rows = torch.tensor([1, 3, 1], dtype=torch.int32, device="cuda")
    e = run.Ed[[1, 3, 1], 2].contiguous()
    assert run.dec.step(run.st, rows, e, run.mem) == 0
    assert run.dec.sync_error() == A.RLT_EINVAL
    assert torch.equal(run.st.s[1], before_s[1]) and int(run.st.pos[1]) == int(before_pos[1])
    assert int(run.st.pos[3]) == int(before_pos[3]) + 1 and not torch.equal(run.st.s[3], before_s[3])
    # the counters were cleared: a proper call of the same rows succeeds
    ok = run.rows([1, 0])
    assert run.dec.step(run.st, ok, run.Ed[[1, 0], 2].contiguous(), run.mem) == 0
    assert run.dec.sync_error() == 0
    assert int(run.st.pos[1]) == int(before_pos[1]) + 1


def test_memory_strides_other_layout_bit_exact():
    """The memory ABI takes explicit strides: the same entries laid out
    [B][G][T][d] (stride_b = G T d, stride_g = T d) instead of [G][B][T][d]
    give bit-identical states and logits (only the addressing differs)."""
    require_gpu()
    from stateful_sequence_model_amd import _abi as A
    wl = SMALL.with_(B=4, T=24)
    ref = GpuRun(wl)
    ref.init()
    S, Z = ref.run(12)
    alt = GpuRun(wl)
    alt.init()
    G, B, T, d = alt.mkd.shape
    mk = alt.mkd.permute(1, 0, 2, 3).contiguous()  # [B][G][T][d]
    mv = alt.mvd.permute(1, 0, 2, 3).contiguous()
    alt.mem = A.rlt_memory(mk.data_ptr(), mv.data_ptr(), T * d, G * T * d, d, alt.mem_len.data_ptr())
    S2, Z2 = alt.run(12)
    assert np.array_equal(S2, S) and np.array_equal(Z2, Z)
    del mk, mv


def test_call_shape_errors_leave_state_untouched():
    """Empty and oversized calls are refused on the host before any work:
    a step of 0 rows or of more than max_rows rows is RLT_ESHAPE, a replay of
    0 sequences is RLT_ESHAPE, a prefill with a length past T_cap is
    RLT_ESHAPE; the state (positions, s) is unchanged and the next step runs
    as if nothing had happened (bit-identical to an untouched run)."""
    require_gpu()
    from stateful_sequence_model_amd import _abi as A
    wl = SMALL.with_(B=4, T=16)
    run = GpuRun(wl)
    run.init()
    rows = run.rows()
    e0 = run.Ed[:, 0].contiguous()
    pos0, s0 = run.st.pos.clone(), run.st.s.clone()
    assert run.dec.step(run.st, rows[:0], e0[:0], run.mem) == A.RLT_ESHAPE
    five = torch.arange(5, dtype=torch.int32, device="cuda")
    e5 = torch.zeros((5, wl.d), dtype=e0.dtype, device="cuda")
    assert run.dec.step(run.st, five, e5, run.mem) == A.RLT_ESHAPE
    tok = torch.zeros((4, wl.T), dtype=torch.int32, device="cuda")
    logp = torch.zeros((4, wl.T), device="cuda")
    assert run.dec.replay(run.st, np.zeros(0, np.int32), np.zeros(0, np.int32), run.Ed, run.mem, tok,
                          logp) == A.RLT_ESHAPE
    torch.cuda.synchronize()
    assert torch.equal(run.st.pos, pos0) and torch.equal(run.st.s, s0)
    assert run.dec.sync_error() == 0
    S, Z = run.run(3)
    clean = GpuRun(wl)
    clean.init()
    S2, Z2 = clean.run(3)
    assert np.array_equal(S, S2) and np.array_equal(Z, Z2)
    # prefill length past the capacity
    from tests.test_gpu_memory import _setup
    dec, mw, _, K, V, mem_len, mem, _ = _setup(wl, 2, 8)
    Ed = run.Ed[:2, :8].contiguous()
    assert dec.memory_prefill(mw, mem, 8, np.array([8, 9], np.int32), Ed) == A.RLT_ESHAPE
    torch.cuda.synchronize()
    assert mem_len.cpu().tolist() == [0, 0] and not K.float().abs().sum().item()


def test_pending_token_bookkeeping_and_errors():
    """App. A.2: a deferred token is recorded as pending; consuming it clears
    it; consuming a different token is RLT_EPENDING and leaves that row's
    state untouched while the other rows advance."""
    require_gpu()
    from stateful_sequence_model_amd import _abi
    wl = SMALL.with_(B=3, T=40)
    run = GpuRun(wl)
    run.init()
    argmax = torch.empty(3, dtype=torch.int32, device="cuda")
    assert run.step(range(3), 1, argmax=argmax, defer=True) == 0
    torch.cuda.synchronize()
    assert torch.equal(run.st.pending, argmax)
    ok = argmax.clone()
    bad = argmax.clone()
    bad[1] = (bad[1] + 1) % wl.V
    s_before = run.st.s.clone()
    ring_before = run.st.ring("k")[:, 1].clone()
    assert run.step(range(3), 2, consume_tok=bad, argmax=argmax) == 0
    assert run.dec.sync_error() == _abi.RLT_EPENDING
    assert run.st.pos.tolist() == [2, 1, 2]
    assert torch.equal(run.st.s[1], s_before[1])
    # bitwise: slots not yet written hold arbitrary bits (possibly NaN patterns)
    assert torch.equal(run.st.ring("k")[:, 1].view(torch.int16), ring_before.view(torch.int16))
    assert run.st.pending.tolist() == [-1, int(ok[1]), -1]
    # consuming the recorded token works and clears it
    assert run.step([1], 2, consume_tok=ok[1:2].contiguous()) == 0
    assert run.dec.sync_error() == 0
    assert run.st.pos.tolist() == [2, 2, 2] and run.st.pending.tolist() == [-1, -1, -1]


def test_prefix_error_and_stale_state():
    """Memory shorter than the consumed position: RLT_EPREFIX, row skipped.
    A state built under another weights version: RLT_ESTALE before any work."""
    require_gpu()
    from stateful_sequence_model_amd import _abi
    wl = SMALL.with_(B=2, T=8)
    run = GpuRun(wl)
    run.init()
    run.mem_len[1] = 3
    for t in range(1, 4):
        assert run.step(range(2), t) == 0
    assert run.dec.sync_error() == 0
    assert run.step(range(2), 4) == 0
    assert run.dec.sync_error() == _abi.RLT_EPREFIX
    assert run.st.pos.tolist() == [4, 3]
    run.st.version = 99
    rows = run.rows()
    assert run.dec.step(run.st, rows, run.Ed[:, 0].contiguous(), run.mem) == _abi.RLT_ESTALE
    assert "version" in _abi.rlt_last_error()


def test_argmax_sampling_and_scoring_against_oracle_on_gpu_logits():
    """Readout integer results from the GPU's own logits: argmax (lowest id
    among ties) exact; sampled token = the oracle's inverse-CDF pick under
    temperature/top-k (or a boundary case the two precisions may resolve
    differently); log mu, log p and the ratio within float tolerance."""
    require_gpu()
    wl = synth.SMALL.with_(B=16, T=20)
    run = GpuRun(wl)
    run.init()
    B, V = wl.B, wl.V
    logits = torch.empty((B, V), device="cuda")
    argmax = torch.empty(B, dtype=torch.int32, device="cuda")
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    lmu = torch.empty(B, device="cuda")
    checked = 0
    for t in range(1, 12):
        u = torch.from_numpy(synth.uniform01(wl.seed, "u", B, start=t * B)).cuda()
        score = torch.from_numpy(synth.uniform_int(wl.seed, "score", B, 0, V - 1, start=t * B)).cuda()
        lp = torch.empty(B, device="cuda")
        assert run.step(range(B), t, logits=logits, argmax=argmax, uniform=u, temperature=0.7, top_k=50,
                        sample_tok=tok, sample_logmu=lmu, score_tok=score, logp=lp) == 0
        torch.cuda.synchronize()
        Zg = logits.cpu().numpy()
        for b in range(B):
            z = Zg[b]
            assert int(argmax[b]) == int(np.flatnonzero(z == z.max())[0])
            ids, lm = behaviour_logprobs(z.astype(np.float64), 0.7, 50)
            w = np.exp(lm - lm.max())
            cum = np.cumsum(w)
            target = float(u[b]) * cum[-1]
            i = int(np.searchsorted(cum, target, side="right"))
            g = list(ids).index(int(tok[b]))
            if g != i:  # only a boundary case may differ
                assert abs(cum[min(g, i)] - target) <= 1e-5 * cum[-1], (t, b)
            assert abs(float(lmu[b]) - lm[g]) < 1e-4
            zz = z.astype(np.float64)
            lse = zz.max() + math.log(np.exp(zz - zz.max()).sum())
            assert abs(float(lp[b]) - (zz[int(score[b])] - lse)) < 1e-4
            checked += 1
    assert checked == 11 * B
    # scoring API on the GPU states: raw log p, behaviour log mu, ratio
    s = run.st.s[:B].contiguous()
    toks = tok.clone()
    logp = torch.empty(B, device="cuda")
    logmu = torch.empty(B, device="cuda")
    ratio = torch.empty(B, device="cuda")
    assert run.dec.score(s, toks, logp, temperature=0.7, top_k=50, logmu=logmu, logmu_behaviour=lmu,
                         ratio=ratio) == 0
    torch.cuda.synchronize()
    orc = Oracle(oracle_config(wl), oracle_weights(run.raw))
    for b in range(B):
        zo = orc.logits(s[b].double().cpu().numpy())
        ids, lm = behaviour_logprobs(zo, 0.7, 50)
        lpo = Oracle.log_softmax(zo)[int(toks[b])]
        assert abs(float(logp[b]) - lpo) < 2e-2
        if int(toks[b]) in set(ids.tolist()):
            assert abs(float(logmu[b]) - lm[list(ids).index(int(toks[b]))]) < 2e-2
        assert abs(float(ratio[b]) - math.exp(float(logp[b]) - float(lmu[b]))) < 1e-4 * max(1, float(ratio[b]))


def test_persistent_step_equals_separate_kernels():
    """The persistent step (one kernel, grid barriers between the recorded
    phases; enabled per context by the fused_rows launch option) reproduces
    the separate kernels bit for bit: same bodies, launch shapes and
    reduction orders (the reference context runs the same narrow-tile
    products, no_packed, since the persistent step does not take the
    operand-order products). Covers plain steps, hipGraph-captured steps
    and a replay from H_0."""
    require_gpu()
    wl = SMALL.with_(B=8, T=40)
    ref = GpuRun(wl, launch=dict(no_packed=1))
    fz = GpuRun(wl, raw=ref.raw, launch=dict(no_packed=1, fused_rows=16))
    _persistent_vs_separate(wl, ref, fz)


def _persistent_vs_separate(wl, ref, fz, nsteps=10):
    for run in (ref, fz):
        run.init()
    S0, Z0 = ref.run(nsteps)
    S1, Z1 = fz.run(nsteps)
    assert np.array_equal(S0, S1) and np.array_equal(Z0, Z1)
    # captured steps
    stream = torch.cuda.Stream()
    rows = ref.rows()
    e_fixed = ref.Ed[:, 0].contiguous()
    am = [torch.empty(wl.B, dtype=torch.int32, device="cuda") for _ in range(2)]
    with torch.cuda.stream(stream):
        for i in range(3):
            for run, out in zip((ref, fz), am):
                assert run.dec.step(run.st, rows, e_fixed, run.mem, argmax=out, graph=True) == 0
            stream.synchronize()
            assert torch.equal(ref.st.s, fz.st.s) and torch.equal(am[0], am[1]), i
    # replay from H_0 with an active set that shrinks over the ticks
    lens = np.array([12, 9, 5, 12, 3, 7, 2, 10], dtype=np.int32)[:wl.B]
    splits = np.ones(wl.B, dtype=np.int32)
    tokens = torch.from_numpy(synth.make_tokens(wl, 0, wl.B, wl.T)).cuda()
    lp = [torch.full((wl.B, wl.T), float("nan"), device="cuda") for _ in range(2)]
    for run, out in zip((ref, fz), lp):
        assert run.dec.replay(run.st, lens, splits, run.Ed, run.mem, tokens, out) == 0
    torch.cuda.synchronize()
    assert torch.equal(lp[0].isnan(), lp[1].isnan())
    assert torch.equal(torch.nan_to_num(lp[0]), torch.nan_to_num(lp[1]))
    assert torch.equal(ref.st.s, fz.st.s)
    return S0, Z0


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cross_attention_many_chunks(dtype):
    """Cross-attention split into 16-position chunks up to t = 300 (up to 19
    chunks per row: the combine's all-at-once path for <= 16 chunks and its
    plain loop beyond), chunks merged inside the cross-attention launch
    (forced: the call has more workgroups than the in-launch merge is
    chosen for),
    against the oracle; the separate combine kernel and (bf16) the
    persistent step's combine phase against it bit for bit [RLT §2.5
    eq. (2.15), §4.2]."""
    require_gpu()
    T = 300
    wl = synth.SMALL.with_(B=2, T=T, L=2, G=2, dtype=dtype)
    sep = GpuRun(wl, launch=dict(xattn_chunk=16, no_packed=1, xattn_combine_kernel=2))
    sep.init()
    S, Z = sep.run(T)
    orc = Oracle(oracle_config(wl), oracle_weights(sep.raw))
    tol = 2e-2 if dtype == "bf16" else 1e-4
    worst = 0.0
    for b in range(wl.B):
        mem = memory_of(wl, b, T=T)
        st = orc.initial_state()
        for t in range(1, T + 1):
            st = orc.transition(st, widen(sep.E[b, t - 1]), mem)
            if t % 7 == 0 or t > T - 20 or t in (16, 17, 256, 257, 272, 273):
                es, ez = rel_l2(S[t - 1, b], st.s), rel_l2(Z[t - 1, b], orc.logits(st.s))
                worst = max(worst, es, ez)
                assert es < tol and ez < tol, (dtype, b, t, es, ez)
    print("many chunks %s: worst rel L2 %.2e" % (dtype, worst))
    k = GpuRun(wl, raw=sep.raw, launch=dict(xattn_chunk=16, no_packed=1, xattn_combine_kernel=1))
    k.init()
    Sk, Zk = k.run(T)
    assert np.array_equal(Sk, S) and np.array_equal(Zk, Z)
    # the library's own choice in one context: the two-row call merges with
    # the combine kernel, a one-row call inside the launch; same bits
    one = GpuRun(wl, raw=sep.raw, launch=dict(xattn_chunk=16, no_packed=1))
    one.init([1])
    S1, Z1 = one.run(T, [1])
    assert np.array_equal(S1[:, 0], S[:, 1]) and np.array_equal(Z1[:, 0], Z[:, 1])
    if dtype == "bf16":
        f = GpuRun(wl, raw=sep.raw, launch=dict(xattn_chunk=16, no_packed=1, fused_rows=16))
        f.init()
        Sf, Zf = f.run(T)
        assert np.array_equal(Sf, S) and np.array_equal(Zf, Z)


def test_snapshot_restore_resumes_bit_exact():
    """§6 exact prefix snapshot: rows saved after 12 transitions and restored
    into a fresh state continue bit for bit like the uninterrupted rows
    (same launch shape); the restored bytes re-snapshot identically; bad
    headers are rejected before anything is written."""
    require_gpu()
    from stateful_sequence_model_amd import _abi
    wl = synth.SMALL.with_(B=4, T=40)
    a = GpuRun(wl)
    a.init()
    a.run(12)
    rows = [1, 3]
    snap = a.dec.snapshot(a.st, rows)
    hdr = _abi.rlt_snapshot_header.from_buffer_copy(bytes(snap[0, :64]))
    assert hdr.magic == _abi.RLT_SNAPSHOT_MAGIC and hdr.pos == 12 and hdr.pending == -1
    SA, ZA = a.run(8, idx=rows)
    b = GpuRun(wl, raw=a.raw)
    b.init()
    assert b.dec.restore(b.st, rows, snap) == 0
    assert np.array_equal(b.dec.snapshot(b.st, rows), snap)
    SB, ZB = b.run(8, idx=rows)
    assert np.array_equal(SA, SB) and np.array_equal(ZA, ZB)
    assert torch.equal(a.st.s[rows], b.st.s[rows])
    # rejected headers leave the state untouched
    before = b.dec.snapshot(b.st, rows)
    for field, value, code in (("magic", 0, _abi.RLT_EINVAL), ("n_layers", wl.L + 1, _abi.RLT_ESHAPE),
                               ("weights_version", 99, _abi.RLT_ESTALE)):
        bad = snap.copy()
        h = _abi.rlt_snapshot_header.from_buffer(bad[1])
        setattr(h, field, value)
        assert b.dec.restore(b.st, rows, bad) == code, field
    assert np.array_equal(b.dec.snapshot(b.st, rows), before)


def test_refresh_weights_after_in_place_update():
    """bf16 contexts multiply an operand-order copy of the matrix weights
    made at creation: weights changed in place are not seen until
    rlt_refresh_weights, which rebuilds the copy and adopts a new weights
    version [RLT §5.4, App. A.4]: states of the old version are then refused
    (RLT_ESTALE) and, re-initialised under the new version, transition
    exactly like those of a context created with the new weights."""
    require_gpu()
    from stateful_sequence_model_amd import DecoderState, _abi as A
    wl = SMALL.with_(B=4, T=16)
    a = GpuRun(wl)
    a.init()
    S0, Z0 = a.run(3)
    # exact bf16 rescalings of matrices of the decoder, the readout and the merge
    a.dec.params["layer.0.wq"].mul_(2)
    a.dec.params["layer.1.w_down"].mul_(0.5)
    a.dec.params["out.w"].mul_(2)
    a.dec.params["merge.ws"].mul_(2)
    a.init()
    S1, Z1 = a.run(3)
    assert np.array_equal(S1, S0) and np.array_equal(Z1, Z0)  # the copy made at creation
    assert a.dec.refresh_weights(a.cfg.version) == A.RLT_EINVAL  # a refresh needs a new version
    old_version = a.st.version
    assert a.dec.refresh_weights(old_version + 1) == 0
    assert a.step(range(4), 4) == A.RLT_ESTALE                  # old states are stale
    a.st = DecoderState(a.cfg, wl.B)
    assert a.st.version == old_version + 1
    a.init()
    S2, Z2 = a.run(3)
    raw = dict(a.raw)
    for k in ("layer.0.wq", "layer.1.w_down", "out.w", "merge.ws"):
        raw[k] = a.dec.params[k].clone()
    b = GpuRun(wl, raw=raw)
    b.init()
    S3, Z3 = b.run(3)
    assert np.array_equal(S2, S3) and np.array_equal(Z2, Z3)
    assert not np.array_equal(S2, S0)
