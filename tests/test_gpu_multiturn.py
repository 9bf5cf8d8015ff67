"""Multi-turn spans ("Recurrent Looped Transformer" §6, App. A.2): a
conversation's later spans (a tool result, the next user message) update the
existing state; nothing is reset. Turn 1 replays the prompt x_1..x_a from H_0
(x_a stays pending); turn 2's span x_{a+1}..x_b then arrives, its memory
entries are appended position by position, and the decoder consumes
x_a .. x_{b-1} from the state it has, the pending token first.
"""
import numpy as np
import pytest

import synth
from oracle import Oracle, build_memory
from tests.gpu_common import model_config, require_gpu, torch
from tests.helpers import oracle_config, oracle_weights, rel_l2, widen

pytestmark = pytest.mark.gpu

A_LEN, B_LEN = 10, 16


def _setup(wl, B, T):
    from stateful_sequence_model_amd import Decoder, DecoderState
    raw = synth.make_weights(wl)
    cfg = model_config(wl)
    dec = Decoder(cfg, raw, max_rows=B, max_ctx=T)
    mw_raw = synth.make_memory_weights(wl)
    mw = dec.memory_weights(mw_raw)
    E = synth.make_e(wl, 0, B, T)
    Ed = torch.from_numpy(E.view(np.int16)).cuda().view(torch.bfloat16)
    tokens = np.random.default_rng(3).integers(0, wl.V, (B, T)).astype(np.int32)
    return dec, mw, mw_raw, raw, E, Ed, torch.from_numpy(tokens).cuda(), DecoderState


def _memory(dec, wl, B, T):
    from stateful_sequence_model_amd import Decoder
    K = torch.zeros((wl.G, B, T, wl.d), dtype=torch.bfloat16, device="cuda")
    V = torch.zeros_like(K)
    mem_len = torch.zeros(B, dtype=torch.int32, device="cuda")
    # the ABI struct holds raw pointers: the caller keeps K, V and mem_len alive
    return Decoder.memory(K, V, mem_len), mem_len, K, V


def _turn2(dec, st, rows, Ed, mem, tok, mw=None, B_cap=None, T_cap=None):
    """Consume x_a .. x_{b-1}; with mw, append memory position t before consuming x_t (t > a)."""
    out = []
    s = torch.empty((len(rows), dec.cfg.d), device="cuda")
    for t in range(A_LEN, B_LEN):
        if mw is not None and t > A_LEN:
            assert dec.memory_append(mw, mem, B_cap, T_cap, rows, Ed[:, t - 1].contiguous()) == 0
        assert dec.step(st, rows, Ed[:, t - 1].contiguous(), mem, consume_tok=tok[:, t - 1].contiguous(),
                        s_out=s) == 0
        out.append(s.clone())
    assert dec.sync_error() == 0
    return torch.stack(out)


def test_multi_turn_continues_like_one_replay():
    """Same memory buffer (prefilled to b): turn-1 replay + turn-2 steps equal
    a single replay of x_1..x_b bit for bit; the pending token of turn 1 is
    x_a and is cleared when consumed."""
    require_gpu()
    wl = synth.SMALL.with_(B=2, T=B_LEN)
    B, T = 2, B_LEN
    dec, mw, _, _, _, Ed, tok, DecoderState = _setup(wl, B, T)
    mem, mem_len, K, V = _memory(dec, wl, B, T)
    assert dec.memory_prefill(mw, mem, T, np.full(B, T, np.int32), Ed) == 0
    rows = torch.arange(B, dtype=torch.int32, device="cuda")
    # one replay over the whole history
    ref = DecoderState(dec.cfg, B)
    logp = torch.zeros((B, T), device="cuda")
    trace = torch.zeros((B, T, wl.d), device="cuda")
    assert dec.replay(ref, np.full(B, B_LEN, np.int32), np.ones(B, np.int32), Ed, mem, tok, logp,
                      s_trace=trace) == 0
    # turn 1, then turn 2 from the existing state
    st = DecoderState(dec.cfg, B)
    assert dec.replay(st, np.full(B, A_LEN, np.int32), np.ones(B, np.int32), Ed, mem, tok,
                      torch.zeros((B, T), device="cuda")) == 0
    torch.cuda.synchronize()
    assert st.pos.tolist() == [A_LEN - 1] * B
    assert st.pending.tolist() == tok[:, A_LEN - 1].tolist()
    S = _turn2(dec, st, rows, Ed, mem, tok)
    assert st.pos.tolist() == [B_LEN - 1] * B and st.pending.tolist() == [-1] * B
    for i, t in enumerate(range(A_LEN, B_LEN)):
        assert torch.equal(S[i], trace[:, t - 1]), t
    assert torch.equal(st.s[:B], ref.s[:B])


def test_multi_turn_with_appended_span_matches_oracle():
    """Turn 2's memory entries appended one position at a time while the
    decoder advances: the states against the oracle over the whole history
    (bf16 gate, relative L2 <= 2e-2 per row and step)."""
    require_gpu()
    wl = synth.SMALL.with_(B=2, T=B_LEN)
    B, T = 2, B_LEN
    dec, mw, mw_raw, raw, E, Ed, tok, DecoderState = _setup(wl, B, T)
    mem, mem_len, K, V = _memory(dec, wl, B, T)
    assert dec.memory_prefill(mw, mem, T, np.full(B, A_LEN, np.int32), Ed) == 0
    rows = torch.arange(B, dtype=torch.int32, device="cuda")
    st = DecoderState(dec.cfg, B)
    assert dec.replay(st, np.full(B, A_LEN, np.int32), np.ones(B, np.int32), Ed, mem, tok,
                      torch.zeros((B, T), device="cuda")) == 0
    S = _turn2(dec, st, rows, Ed, mem, tok, mw=mw, B_cap=B, T_cap=T).double().cpu().numpy()
    assert mem_len.tolist() == [B_LEN - 1] * B
    cfg = oracle_config(wl)
    orc = Oracle(cfg, oracle_weights(raw))
    omw = oracle_weights(mw_raw)
    for b in range(B):
        omem = build_memory(cfg, widen(E[b]), omw, n=B_LEN - 1)
        ost = orc.initial_state()
        for t in range(1, B_LEN):
            ost = orc.transition(ost, widen(E[b, t - 1]), omem)
            if t >= A_LEN:
                e = rel_l2(S[t - A_LEN, b], ost.s)
                assert e < 2e-2, (b, t, e)
