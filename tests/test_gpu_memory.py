"""GPU parity of the encoder-memory construction ("Recurrent Looped
Transformer" §2.2, eq. (2.2)): token-parallel prefill and per-step append
against the oracle's entry-by-entry definition, bookkeeping of mem_len
(exact), the capacity error, and a decoder run on GPU-built memory.

Tolerances: float32 mode 1e-5 relative L2 per entry vector; bf16 mode 1e-2
per entry vector (the GPU rounds e * gain and the stored entries to bf16,
each a relative 2^-9 per element, against the oracle's float64 on the same
bf16-valued inputs).
"""
import numpy as np
import pytest

import synth
from oracle import Memory, Oracle, build_memory, memory_entry
from tests.gpu_common import GpuRun, model_config, require_gpu, torch
from tests.helpers import oracle_config, oracle_weights, rel_l2, widen

pytestmark = pytest.mark.gpu


def _setup(wl, B, T_cap, launch=None):
    from stateful_sequence_model_amd import Decoder
    raw = synth.make_weights(wl)
    cfg = model_config(wl)
    dec = Decoder(cfg, raw, max_rows=max(B, 1), max_ctx=T_cap, launch=launch)
    mw_raw = synth.make_memory_weights(wl)
    mw = dec.memory_weights(mw_raw)
    tdt = cfg.torch_dtype
    K = torch.zeros((wl.G, B, T_cap, wl.d), dtype=tdt, device="cuda")
    V = torch.zeros_like(K)
    mem_len = torch.zeros(B, dtype=torch.int32, device="cuda")
    mem = Decoder.memory(K, V, mem_len)
    return dec, mw, mw_raw, K, V, mem_len, mem, raw


def _check_entries(wl, K, V, mw_raw, E, entries, tol):
    """entries: iterable of (b, t); compares every group's (k, v)."""
    cfg = oracle_config(wl)
    mw = oracle_weights(mw_raw)
    Kh = K.double().cpu().numpy() if K.dtype == torch.float32 else K.float().double().cpu().numpy()
    Vh = V.double().cpu().numpy() if V.dtype == torch.float32 else V.float().double().cpu().numpy()
    worst = 0.0
    for b, t in entries:
        for g in range(wl.G):
            k, v = memory_entry(cfg, widen(E[b, t - 1]), t, mw["memory.%d.norm_e" % g], mw["memory.%d.wk" % g],
                                mw["memory.%d.wv" % g])
            ek, ev = rel_l2(Kh[g, b, t - 1], k), rel_l2(Vh[g, b, t - 1], v)
            worst = max(worst, ek, ev)
            assert ek < tol and ev < tol, (b, t, g, ek, ev)
    return worst


def test_prefill_unaligned_buffers_and_decoder_alignment_check():
    """bf16 small workload with e and the memory buffers starting 2 bytes past
    a 16-byte boundary: the prefill takes its element-wise gather and
    epilogue (the 16-byte ones need aligned runs), every entry against the
    oracle; a decoder step on that memory is refused on the host (RLT_EINVAL:
    the attention kernels read 16-byte runs)."""
    require_gpu()
    from stateful_sequence_model_amd import Decoder, DecoderState
    from stateful_sequence_model_amd._abi import RLT_EINVAL
    wl = synth.SMALL
    B, T_cap = 4, 40
    dec, mw, mw_raw, K0, V0, mem_len, _, _ = _setup(wl, B, T_cap)
    n = K0.numel()
    kbuf = torch.zeros(n + 8, dtype=K0.dtype, device="cuda")
    vbuf = torch.zeros_like(kbuf)
    K, V = kbuf[1:n + 1].view(K0.shape), vbuf[1:n + 1].view(V0.shape)
    assert K.data_ptr() % 16 and V.data_ptr() % 16
    mem = Decoder.memory(K, V, mem_len)
    E = synth.make_e(wl, 0, B, T_cap)
    flat = torch.from_numpy(E.view(np.int16)).cuda().view(torch.bfloat16).reshape(-1)
    ebuf = torch.zeros(flat.numel() + 8, dtype=torch.bfloat16, device="cuda")
    ebuf[1:flat.numel() + 1] = flat
    Ed = ebuf[1:flat.numel() + 1].view(B, T_cap, wl.d)
    assert Ed.data_ptr() % 16
    lens = np.array([40, 17, 1, 33], dtype=np.int32)
    assert dec.memory_prefill(mw, mem, T_cap, lens, Ed) == 0
    torch.cuda.synchronize()
    assert dec.sync_error() == 0
    assert mem_len.cpu().tolist() == lens.tolist()
    worst = _check_entries(wl, K, V, mw_raw, E, [(b, t) for b in range(B) for t in range(1, lens[b] + 1)], 1e-2)
    print("unaligned prefill: worst entry rel L2 %.2e" % worst)
    st = DecoderState(dec.cfg, B)
    rows = torch.arange(B, dtype=torch.int32, device="cuda")
    dec.init_state(st, rows)
    assert dec.step(st, rows, Ed[:, 0].contiguous(), mem) == RLT_EINVAL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_matches_oracle(dtype):
    """Small workload (G = 4 groups, d = 256): ragged lengths; every entry
    against the oracle; untouched positions stay zero; mem_len = len."""
    require_gpu()
    wl = synth.SMALL.with_(dtype=dtype)
    B, T_cap = 4, 40
    dec, mw, mw_raw, K, V, mem_len, mem, _ = _setup(wl, B, T_cap)
    E = synth.make_e(wl, 0, B, T_cap)
    Ed = torch.from_numpy(E.view(np.int16) if E.dtype == np.uint16 else E).cuda()
    if dtype == "bf16":
        Ed = Ed.view(torch.bfloat16)
    lens = np.array([40, 17, 1, 33], dtype=np.int32)
    assert dec.memory_prefill(mw, mem, T_cap, lens, Ed) == 0
    torch.cuda.synchronize()
    assert dec.sync_error() == 0
    assert mem_len.cpu().tolist() == lens.tolist()
    tol = 1e-2 if dtype == "bf16" else 1e-5
    worst = _check_entries(wl, K, V, mw_raw, E, [(b, t) for b in range(B) for t in range(1, lens[b] + 1)], tol)
    print("prefill %s: worst entry rel L2 %.2e" % (dtype, worst))
    for b in range(B):
        assert not K[:, b, lens[b]:].float().abs().sum().item()
        assert not V[:, b, lens[b]:].float().abs().sum().item()


def test_append_matches_oracle_and_prefill():
    """Per-step append of a subset of rows in a scattered order: entries
    against the oracle, mem_len advancing by one per call, untouched rows
    unchanged; the same entries as the prefill within the bf16 tolerance."""
    require_gpu()
    wl = synth.SMALL
    B, T_cap = 5, 24
    dec, mw, mw_raw, K, V, mem_len, mem, _ = _setup(wl, B, T_cap)
    E = synth.make_e(wl, 0, B, T_cap)
    Ed = torch.from_numpy(E.view(np.int16)).cuda().view(torch.bfloat16)
    rows = [3, 0, 4]
    rows_d = torch.tensor(rows, dtype=torch.int32, device="cuda")
    for t in range(1, T_cap + 1):
        e = Ed[rows_d.long(), t - 1].contiguous()
        assert dec.memory_append(mw, mem, B, T_cap, rows_d, e) == 0
    torch.cuda.synchronize()
    assert dec.sync_error() == 0
    assert mem_len.cpu().tolist() == [T_cap, 0, 0, T_cap, T_cap]
    assert not K[:, 1].float().abs().sum().item() and not K[:, 2].float().abs().sum().item()
    _check_entries(wl, K, V, mw_raw, E, [(b, t) for b in rows for t in range(1, T_cap + 1)], 1e-2)
    # prefill of the same rows into fresh buffers
    dec2, mw2, _, K2, V2, len2, mem2, _ = _setup(wl, B, T_cap)
    assert dec2.memory_prefill(mw2, mem2, T_cap, np.full(B, T_cap, np.int32), Ed) == 0
    torch.cuda.synchronize()
    for b in rows:
        for g in range(wl.G):
            for t in range(T_cap):
                assert rel_l2(K[g, b, t].double().cpu().numpy(), K2[g, b, t].double().cpu().numpy()) < 1e-2
                assert rel_l2(V[g, b, t].double().cpu().numpy(), V2[g, b, t].double().cpu().numpy()) < 1e-2


def test_append_at_capacity_raises_prefix_error():
    """A row already holding T_cap entries is left unchanged and the call
    reports a device-detected RLT_EPREFIX; other rows of the call proceed."""
    require_gpu()
    from stateful_sequence_model_amd import _abi
    wl = synth.SMALL
    B, T_cap = 2, 3
    dec, mw, _, K, V, mem_len, mem, _ = _setup(wl, B, T_cap)
    mem_len.copy_(torch.tensor([T_cap, 1], dtype=torch.int32))
    K_before = K.clone()
    e = torch.randn((2, wl.d), device="cuda").to(torch.bfloat16)
    assert dec.memory_append(mw, mem, B, T_cap, torch.tensor([0, 1], dtype=torch.int32, device="cuda"), e) == 0
    assert dec.sync_error() == _abi.RLT_EPREFIX
    assert mem_len.cpu().tolist() == [T_cap, 2]
    assert torch.equal(K[:, 0], K_before[:, 0])
    assert K[:, 1, 1].float().abs().sum().item() > 0


def test_prefill_across_chunks_mid_width():
    """Mid width (d = 1024, 16 x 64 heads): more entries than one chunk of
    the prefill schedule (8192), so the wide-tile product and the chunked
    (sequence, position) mapping are exercised; sampled entries against the
    oracle, mem_len exact."""
    require_gpu()
    wl = synth.MID
    B, T_cap = 5, 2048
    dec, mw, mw_raw, K, V, mem_len, mem, _ = _setup(wl, B, T_cap)
    E = synth.make_e(wl, 0, B, T_cap)
    Ed = torch.from_numpy(E.view(np.int16)).cuda().view(torch.bfloat16)
    lens = np.array([2048, 1500, 2048, 2048, 848], dtype=np.int32)  # 8492 entries
    assert dec.memory_prefill(mw, mem, T_cap, lens, Ed) == 0
    torch.cuda.synchronize()
    assert dec.sync_error() == 0
    assert mem_len.cpu().tolist() == lens.tolist()
    offs = np.concatenate([[0], np.cumsum(lens)])
    b_edge = int(np.searchsorted(offs, 8192, side="right") - 1)
    t_edge = 8192 - int(offs[b_edge]) + 1
    assert (b_edge, t_edge) == (4, 549)  # the second chunk starts inside sequence 4
    sample = [(0, 1), (0, 2048), (1, 1500), (2, 777), (3, 2048), (4, 1), (4, 848),
              (b_edge, t_edge - 1), (b_edge, t_edge)]
    worst = _check_entries(wl, K, V, mw_raw, E, sample, 1e-2)
    print("mid prefill: worst sampled entry rel L2 %.2e" % worst)


def test_decoder_on_gpu_built_memory():
    """Small workload: memory built on the GPU (prefill), then 10 decoder
    steps; the oracle builds its own memory from the same weights and runs
    the same steps (bf16 gates of the decoder: rel L2 <= 2e-2, top-1)."""
    require_gpu()
    from stateful_sequence_model_amd import Decoder, DecoderState
    wl = synth.SMALL.with_(B=3, T=16)
    B, T = 3, 16
    dec, mw, mw_raw, K, V, mem_len, mem, raw = _setup(wl, B, T)
    E = synth.make_e(wl, 0, B, T)
    Ed = torch.from_numpy(E.view(np.int16)).cuda().view(torch.bfloat16)
    assert dec.memory_prefill(mw, mem, T, np.full(B, T, np.int32), Ed) == 0
    st = DecoderState(dec.cfg, B)
    rows = torch.arange(B, dtype=torch.int32, device="cuda")
    dec.init_state(st, rows)
    s_out = torch.empty((B, wl.d), device="cuda")
    logits = torch.empty((B, wl.V), device="cuda")
    S, Z = [], []
    for t in range(1, 11):
        assert dec.step(st, rows, Ed[:, t - 1].contiguous(), mem, s_out=s_out, logits=logits) == 0
        S.append(s_out.double().cpu().numpy())
        Z.append(logits.double().cpu().numpy())
    assert dec.sync_error() == 0
    cfg = oracle_config(wl)
    orc = Oracle(cfg, oracle_weights(raw))
    omw = oracle_weights(mw_raw)
    for b in range(B):
        omem = build_memory(cfg, widen(E[b]), omw, n=10)
        ost = orc.initial_state()
        for t in range(1, 11):
            ost = orc.transition(ost, widen(E[b, t - 1]), omem)
            assert rel_l2(S[t - 1][b], ost.s) < 2e-2, (b, t)
            zo = orc.logits(ost.s)
            assert rel_l2(Z[t - 1][b], zo) < 2e-2, (b, t)


@pytest.mark.timeout(900)
def test_prefill_reference_width_and_decoder_on_it():
    """Reference width (d = 2048, 16 x 128 heads, the width the memory
    prefill benchmark times): 10,861 entries over two chunks of the prefill
    schedule, with the 16-byte rotary/scatter epilogue (aligned bf16
    buffers); sampled entries against the oracle (incl. both sides of the
    chunk edge and each sequence's first and last position), mem_len exact;
    then four decoder steps from H_0 of two rows reading that memory,
    against the oracle on its own memory built from the same weights
    [RLT §2.2 eq. (2.2), §2.5 eq. (2.15)]."""
    require_gpu()
    from stateful_sequence_model_amd import DecoderState
    wl = synth.REF
    B, T_cap = 5, 4096
    dec, mw, mw_raw, K, V, mem_len, mem, raw = _setup(wl, B, T_cap)
    E = synth.make_e(wl, 0, B, T_cap)
    Ed = torch.from_numpy(E.view(np.int16)).cuda().view(torch.bfloat16)
    lens = np.array([4096, 3000, 1200, 2048, 517], dtype=np.int32)
    assert dec.memory_prefill(mw, mem, T_cap, lens, Ed) == 0
    torch.cuda.synchronize()
    assert dec.sync_error() == 0
    assert mem_len.cpu().tolist() == lens.tolist()
    offs = np.concatenate([[0], np.cumsum(lens)])
    b_edge = int(np.searchsorted(offs, 8192, side="right") - 1)
    t_edge = 8192 - int(offs[b_edge]) + 1
    assert (b_edge, t_edge) == (2, 1097)  # the second chunk starts inside sequence 2
    sample = [(0, 1), (0, 4096), (0, 2049), (1, 1), (1, 3000), (2, 600), (2, 1200), (3, 1), (3, 2048),
              (b_edge, t_edge - 1), (b_edge, t_edge), (4, 1), (4, 517)]
    worst = _check_entries(wl, K, V, mw_raw, E, sample, 1e-2)
    print("reference-width prefill: worst sampled entry rel L2 %.2e" % worst)
    # decoder steps on the GPU-built memory
    st = DecoderState(dec.cfg, B)
    rows = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    dec.init_state(st, rows)
    s_out = torch.empty((2, wl.d), device="cuda")
    logits = torch.empty((2, wl.V), device="cuda")
    S, Z = [], []
    for t in range(1, 5):
        assert dec.step(st, rows, Ed[rows.long(), t - 1].contiguous(), mem, s_out=s_out, logits=logits) == 0
        S.append(s_out.double().cpu().numpy())
        Z.append(logits.double().cpu().numpy())
    assert dec.sync_error() == 0
    del K, V
    cfg = oracle_config(wl)
    orc = Oracle(cfg, oracle_weights(raw))
    omw = oracle_weights(mw_raw)
    for j, b in enumerate((0, 4)):
        omem = build_memory(cfg, widen(E[b]), omw, n=4)
        ost = orc.initial_state()
        for t in range(1, 5):
            ost = orc.transition(ost, widen(E[b, t - 1]), omem)
            assert rel_l2(S[t - 1][j], ost.s) < 2e-2, (b, t)
            assert rel_l2(Z[t - 1][j], orc.logits(ost.s)) < 2e-2, (b, t)


def test_prefill_big_tile_equals_lds_tile():
    """Reference width (d = 2048, 16 x 128 heads), 2,333 entries (nine full
    256-row tiles and a ragged tenth): the K/V product on the 256 x 256 tile
    writes exactly the entries of the 128 x 128 tile (launch option
    no_big_tile): both add every entry's products in the same order (K in
    stages of 64, 16-wide MFMA steps in order, one accumulator per 32 x 32
    block), and a few of them match the oracle."""
    require_gpu()
    wl = synth.REF.with_(L=2)
    B, T_cap = 3, 1500
    lens = np.array([1500, 700, 133], dtype=np.int32)
    out = []
    for launch in (None, {"no_big_tile": 1}):
        dec, mw, mw_raw, K, V, mem_len, mem, _ = _setup(wl, B, T_cap, launch=launch)
        E = synth.make_e(wl, 0, B, T_cap)
        Ed = torch.from_numpy(E.view(np.int16)).cuda().view(torch.bfloat16)
        assert dec.memory_prefill(mw, mem, T_cap, lens, Ed) == 0
        torch.cuda.synchronize()
        assert dec.sync_error() == 0
        assert mem_len.cpu().tolist() == lens.tolist()
        out.append((K.clone(), V.clone()))
        if launch is None:
            _check_entries(wl, K, V, mw_raw, E, [(0, 1), (0, 1500), (1, 700), (2, 1), (2, 133)], 1e-2)
        dec.close()
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])
