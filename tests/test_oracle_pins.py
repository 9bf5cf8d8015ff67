"""Pins of the CPU oracle against facts fixed outside it.

Each test ties one part of the oracle to a library routine, a closed form, an
independent formulation or an invariant stated in "Recurrent Looped
Transformer" (Zhang, 2026), so that a dropped term, a wrong sign or index, or
a transposed operand in the oracle fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import synth
from oracle import (Config, Memory, Oracle, attend, behaviour_logprobs, importance_ratio, replay,
                    retained_positions, ring_slot, rms_norm, rope, sample, state_from_ring,
                    state_to_ring, topk_order, window_positions)
from tests.helpers import e_of, make_oracle, memory_of, oracle_config, rel_l2

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(**kw):
    base = synth.TINY.with_(dtype="f32", **kw)
    return base


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# building blocks against library routines / independent formulations
# ---------------------------------------------------------------------------

def test_rms_norm_matches_torch():
    x = _rand((5, 64), 0)
    g = 1 + 0.1 * _rand(64, 1)
    ref = Fn.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)


def test_rope_equals_complex_rotation():
    """Rotate-half RoPE == multiplying z_i = x_i + i x_{i+dh/2} by exp(i t w_i)."""
    H, dh, theta = 4, 16, 10000.0
    x = _rand(H * dh, 2)
    for t in (1, 7, 4096):
        y = rope(x, t, H, dh, theta).reshape(H, dh)
        xh = x.reshape(H, dh)
        w = theta ** (-np.arange(dh // 2) * 2.0 / dh)
        z = (xh[:, : dh // 2] + 1j * xh[:, dh // 2:]) * np.exp(1j * t * w)
        assert np.allclose(y[:, : dh // 2], z.real, atol=1e-12)
        assert np.allclose(y[:, dh // 2:], z.imag, atol=1e-12)


def test_rope_relative_position():
    """<RoPE(q,t1), RoPE(k,t2)> depends only on t1 - t2 (the scores in SWA
    depend on the offset, not on the absolute origin)."""
    H, dh = 2, 32
    q, k = _rand(H * dh, 3), _rand(H * dh, 4)
    d1 = rope(q, 10, H, dh, 1e4) @ rope(k, 3, H, dh, 1e4)
    d2 = rope(q, 1010, H, dh, 1e4) @ rope(k, 1003, H, dh, 1e4)
    assert abs(d1 - d2) < 1e-9
    assert np.allclose(rope(q, 0, H, dh, 1e4), q)


def test_attend_matches_sdpa():
    H, dh, n = 4, 16, 9
    q, K, V = _rand(H * dh, 5), _rand((n, H * dh), 6), _rand((n, H * dh), 7)
    tq = torch.from_numpy(q).view(1, H, 1, dh)
    tk = torch.from_numpy(K).view(n, H, dh).transpose(0, 1).unsqueeze(0)
    tv = torch.from_numpy(V).view(n, H, dh).transpose(0, 1).unsqueeze(0)
    ref = Fn.scaled_dot_product_attention(tq, tk, tv).reshape(-1).numpy()
    assert np.allclose(attend(q, K, V, H, dh), ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# merge [RLT §2.5 eqs. (2.9)-(2.11)] closed forms
# ---------------------------------------------------------------------------

def test_convex_merge_zero_gate_is_midpoint():
    wl = _tiny(merge="convex")
    raw = synth.make_weights(wl)
    raw["merge.wg"][:] = 0
    raw["merge.bg"][:] = 0
    orc = make_oracle(wl, raw)
    e, s = _rand(64, 8), _rand(64, 9)
    assert np.array_equal(orc.merge(e, s), (e + s) / 2)


def test_gated_merge_alpha_zero_is_identity_in_e():
    wl = _tiny(merge="gated")
    orc = make_oracle(wl, alpha=0.0)
    e, s = _rand(64, 10), _rand(64, 11)
    assert np.array_equal(orc.merge(e, s), e)


def test_gated_merge_half_gate_identity_projection():
    """W_g = 0, b_g = 0, W_s = I  =>  u = e + alpha/2 * RMSNorm_s(s)."""
    wl = _tiny(merge="gated")
    raw = synth.make_weights(wl)
    raw["merge.wg"][:] = 0
    raw["merge.bg"][:] = 0
    raw["merge.ws"][:] = np.eye(64, dtype=np.float32)
    orc = make_oracle(wl, raw, alpha=0.7)
    e, s = _rand(64, 12), _rand(64, 13)
    g = torch.from_numpy(orc.w["merge.norm"])
    ref = e + 0.35 * Fn.rms_norm(torch.from_numpy(s), (64,), weight=g, eps=wl.eps).numpy()
    assert np.allclose(orc.merge(e, s), ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# SWA window and cache [RLT §2.5 eq. (2.14) and the retention rule after (2.16)]
# ---------------------------------------------------------------------------

def _read_retention_fixture():
    path = os.path.join(GOLDEN, "swa_retention_W4.txt")
    rows = {}
    with open(path) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            t, window, kept = line.split("|")
            rows[int(t)] = ([int(x) for x in window.split()], [int(x) for x in kept.split()])
    return rows


def test_retention_fixture_and_oracle_cache():
    """Golden table: window read and positions kept at W = 4 for t = 1..9."""
    rows = _read_retention_fixture()
    assert sorted(rows) == list(range(1, 10))
    for t, (win, kept) in rows.items():
        assert window_positions(t, 4) == win
        assert retained_positions(t, 4) == kept
    wl = _tiny(W=4, T=12)
    orc = make_oracle(wl)
    st = orc.initial_state()
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    for t in range(1, 10):
        st = orc.transition(st, E[t - 1], mem)
        for l in range(wl.L):
            assert sorted(st.hist[l]) == rows[t][1]


def test_occupancy_and_slots_closed_form():
    for W in (2, 3, 4, 16, 17):
        for t in range(0, 3 * W):
            kept = retained_positions(t, W) if t > 0 else []
            assert len(kept) == min(t, W - 1)
            slots = [ring_slot(j, W) for j in kept]
            assert len(set(slots)) == len(slots)  # no two retained positions share a slot
            # the slot evicted at t+1 is the one holding the oldest position of the window
            if t >= W - 1:
                assert ring_slot(t + 1, W) == ring_slot(t + 1 - (W - 1), W)
    assert retained_positions(5, 1) == []


def test_w1_is_self_only():
    """W = 1: the window is {t}, so the SWA sublayer adds W_O v_t exactly."""
    wl = _tiny(W=1, T=6)
    orc = make_oracle(wl)
    st = orc.initial_state()
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    for t in range(1, 6):
        tr = {}
        st = orc.transition(st, E[t - 1], mem, trace=tr)
        for l in range(wl.L):
            z_in = tr["u"] if l == 0 else tr["z"][l - 1]
            b = tr["b"][l]
            wo = orc.w["layer.%d.wo" % l]
            assert np.allclose(b - z_in, wo @ tr["v"][l], rtol=1e-12, atol=1e-12)
            assert st.hist[l] == {}


def test_uniform_query_averages_exact_window():
    """W_Q = 0 makes every SWA score 0, so o = mean of exactly min(t, W)
    window values (an off-by-one in the window shows as a wrong mean)."""
    wl = _tiny(W=4, T=10, pos="none")
    raw = synth.make_weights(wl)
    for l in range(wl.L):
        raw["layer.%d.wq" % l][:] = 0
    orc = make_oracle(wl, raw)
    st = orc.initial_state()
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    vs = [[] for _ in range(wl.L)]
    for t in range(1, 10):
        tr = {}
        st = orc.transition(st, E[t - 1], mem, trace=tr)
        for l in range(wl.L):
            vs[l].append(tr["v"][l])
            win = vs[l][max(0, t - 4):t]
            assert len(win) == min(t, 4)
            assert np.allclose(tr["o_swa"][l], np.mean(win, axis=0), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# cross-attention to M_{<=t} [RLT §2.5 eq. (2.15), §4.2]
# ---------------------------------------------------------------------------

def test_cross_attention_first_position_returns_v1():
    wl = _tiny()
    orc = make_oracle(wl)
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    tr = {}
    orc.transition(orc.initial_state(), E[0], mem, trace=tr)
    for l in range(wl.L):
        assert np.allclose(tr["o_mem"][l], mem.v[wl.group_of(l)][0], rtol=1e-12, atol=1e-12)


def test_cross_attention_uniform_query_is_prefix_mean():
    wl = _tiny(T=12)
    raw = synth.make_weights(wl)
    for l in range(wl.L):
        raw["layer.%d.wqm" % l][:] = 0
    orc = make_oracle(wl, raw)
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    st = orc.initial_state()
    for t in range(1, 12):
        tr = {}
        st = orc.transition(st, E[t - 1], mem, trace=tr)
        for l in range(wl.L):
            ref = np.mean(mem.v[wl.group_of(l)][:t], axis=0)
            assert np.allclose(tr["o_mem"][l], ref, rtol=1e-12, atol=1e-12)


def test_causality_future_memory_and_inputs_unused():
    """Prop. B.1: H_t depends only on the prefix. NaN in memory rows j > t and
    in future e leaves every state up to t finite and unchanged."""
    wl = _tiny(T=16, G=2)
    orc = make_oracle(wl)
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    st = orc.initial_state()
    ref = []
    for t in range(1, 16):
        st = orc.transition(st, E[t - 1], mem)
        ref.append(st.s)
    st = orc.initial_state()
    for t in range(1, 16):
        mk = [m.copy() for m in mem.k]
        mv = [m.copy() for m in mem.v]
        for g in range(wl.G):
            mk[g][t:] = np.nan
            mv[g][t:] = np.nan
        Ep = E.copy()
        Ep[t:] = np.nan
        st = orc.transition(st, Ep[t - 1], Memory(mk, mv))
        assert np.all(np.isfinite(st.s))
        assert np.array_equal(st.s, ref[t - 1])


# ---------------------------------------------------------------------------
# whole decoder: alpha = 0 equals an independent parallel teacher-forced pass
# ---------------------------------------------------------------------------

def _complex_rope(x, positions, H, dh, theta):
    """RoPE written as complex multiplication (independent of the oracle's
    rotate-half code): x [T, d] at positions [T]."""
    T = x.shape[0]
    xh = x.reshape(T, H, dh)
    w = theta ** (-np.arange(dh // 2) * 2.0 / dh)
    z = (xh[..., : dh // 2] + 1j * xh[..., dh // 2:]) * np.exp(1j * np.outer(positions, w))[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1).reshape(T, H * dh)


def _parallel_pass(orc: Oracle, E: np.ndarray, mem: Memory, T: int) -> np.ndarray:
    """Teacher-forced pass over positions 1..T with banded-causal SWA masks
    and prefix masks on memory, using library SDPA / rms_norm / silu in
    float64. Valid only when the merge ignores s (gated, alpha = 0)."""
    c, w = orc.cfg, orc.w
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    pos = np.arange(1, T + 1)
    jj, ii = np.meshgrid(pos, pos)  # ii = query position, jj = key position
    band = tt((jj <= ii) & (jj >= ii - c.W + 1))
    prefix = tt(jj <= ii)

    def heads(x):
        return tt(x).view(T, c.H, c.dh).transpose(0, 1)

    def rp(x):
        return _complex_rope(x, pos, c.H, c.dh, c.rope_theta) if c.pos == "rope" else x

    Z = E[:T].copy()
    for l in range(c.L):
        p = "layer.%d." % l
        Hn = Fn.rms_norm(tt(Z), (c.d,), weight=tt(w[p + "norm_s"]), eps=c.eps).numpy()
        Q, K, Vv = rp(Hn @ w[p + "wq"].T), rp(Hn @ w[p + "wk"].T), Hn @ w[p + "wv"].T
        O = Fn.scaled_dot_product_attention(heads(Q), heads(K), heads(Vv), attn_mask=band)
        Bm = Z + O.transpose(0, 1).reshape(T, c.d).numpy() @ w[p + "wo"].T
        Hm = Fn.rms_norm(tt(Bm), (c.d,), weight=tt(w[p + "norm_m"]), eps=c.eps).numpy()
        g = c.group_of(l)
        Om = Fn.scaled_dot_product_attention(heads(rp(Hm @ w[p + "wqm"].T)), heads(mem.k[g][:T]),
                                             heads(mem.v[g][:T]), attn_mask=prefix)
        A = Bm + Om.transpose(0, 1).reshape(T, c.d).numpy() @ w[p + "wom"].T
        Hd = Fn.rms_norm(tt(A), (c.d,), weight=tt(w[p + "norm_d"]), eps=c.eps)
        act = Fn.silu(Hd @ tt(w[p + "w_gate"]).T) * (Hd @ tt(w[p + "w_up"]).T)
        Z = A + (act @ tt(w[p + "w_down"]).T).numpy()
    return Z


@pytest.mark.parametrize("W,G,pos", [(4, 1, "rope"), (3, 2, "none"), (40, 2, "rope"), (1, 1, "rope")])
def test_alpha_zero_equals_parallel_pass(W, G, pos):
    """With alpha = 0 the decoder input is e_t and no state feeds back, so the
    recurrence must equal a banded-causal parallel pass (W >= T gives plain
    causal attention, W = 1 self-only)."""
    T = 20
    wl = _tiny(W=W, G=G, T=T, merge="gated", pos=pos)
    orc = make_oracle(wl, alpha=0.0)
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    Z = _parallel_pass(orc, E, mem, T)
    st = orc.initial_state()
    for t in range(1, T + 1):
        st = orc.transition(st, E[t - 1], mem)
        assert rel_l2(st.s, Z[t - 1]) < 1e-12


def test_feedback_breaks_parallel_equivalence():
    """alpha != 0: a parallel SWA pass is not the recurrence (report §2.4)."""
    T = 12
    wl = _tiny(W=4, T=T, merge="gated")
    orc = make_oracle(wl, alpha=0.5)
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    Z = _parallel_pass(Oracle(orc.cfg, orc.w), E, mem, T)  # pretends u_t = e_t
    st = orc.initial_state()
    diffs = []
    for t in range(1, T + 1):
        st = orc.transition(st, E[t - 1], mem)
        diffs.append(rel_l2(st.s, Z[t - 1]))
    assert min(diffs) > 1e-3


# ---------------------------------------------------------------------------
# recurrence-level properties
# ---------------------------------------------------------------------------

def test_split_invariance_and_state_roundtrip():
    """Prop. 3.1: stopping at any T0 and continuing gives the same states;
    a state exported to the ring layout and re-imported continues identically."""
    wl = _tiny(W=4, T=14)
    orc = make_oracle(wl)
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    full, ss = orc.run(orc.initial_state(), E, mem, 13)
    for T0 in (1, 3, 4, 9):
        mid, _ = orc.run(orc.initial_state(), E, mem, T0)
        rk, rv = state_to_ring(orc.cfg, mid)
        mid2 = state_from_ring(orc.cfg, mid.s, mid.pos, rk, rv)
        end, _ = orc.run(mid2, E[T0:], mem, 13 - T0)
        assert np.array_equal(end.s, full.s)
        assert end.pos == full.pos == 13


def test_path_depth_counts():
    """After t tokens the state path has traversed t * L_D decoder blocks
    (report §3.3; 48t for the 48-layer configuration)."""
    wl = _tiny(T=6)
    orc = make_oracle(wl)
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    st, _ = orc.run(orc.initial_state(), E, mem, 5)
    assert st.blocks == 5 * wl.L
    cfg48 = oracle_config(synth.REF)
    assert cfg48.L * 7 == 48 * 7


def test_fp32_drift_is_far_below_fp32_gate():
    """The fp32 gate (rel. L2 1e-4 over all steps) is meaningful only if the
    oracle's own fp32-vs-fp64 drift is far below it."""
    wl = synth.TINY
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    o64 = make_oracle(wl)
    o32 = make_oracle(wl, dtype=np.float32)
    _, s64 = o64.run(o64.initial_state(), E, mem, wl.T - 1)
    mem32 = Memory([m.astype(np.float32) for m in mem.k], [m.astype(np.float32) for m in mem.v])
    _, s32 = o32.run(o32.initial_state(), E.astype(np.float32), mem32, wl.T - 1)
    drift = max(rel_l2(a, b) for a, b in zip(s32, s64))
    assert drift < 1e-5


# ---------------------------------------------------------------------------
# readout and behaviour distribution [RLT §2.3 eq. (2.6), §5.3 eq. (5.5)]
# ---------------------------------------------------------------------------

def test_log_softmax_normalises_and_matches_torch():
    z = _rand(300, 14, 5.0)
    lp = Oracle.log_softmax(z)
    assert abs(np.sum(np.exp(lp)) - 1.0) < 1e-12
    assert np.allclose(lp, torch.log_softmax(torch.from_numpy(z), 0).numpy(), atol=1e-12)


def test_behaviour_equals_raw_policy_without_transforms():
    """tau = 1 and k = V: mu = p, so every ratio r_i is 1."""
    z = _rand(100, 15, 3.0)
    ids, lmu = behaviour_logprobs(z, 1.0, 0)
    lp = Oracle.log_softmax(z)
    assert np.allclose(lmu, lp[ids], atol=1e-12)
    assert all(abs(importance_ratio(lp[i], m) - 1.0) < 1e-12 for i, m in zip(ids, lmu))


def test_topk_order_ties_and_truncation():
    z = np.array([1.0, 3.0, 3.0, 0.5, 3.0, 2.0])
    assert list(topk_order(z, 4)) == [1, 2, 4, 5]
    ids, lmu = behaviour_logprobs(z, 0.5, 2)
    assert list(ids) == [1, 2]
    assert np.allclose(np.exp(lmu), [0.5, 0.5])
    z2 = _rand(1000, 16)
    assert topk_order(z2, 1)[0] == int(np.argmax(z2))
    ids, lmu = behaviour_logprobs(z2, 0.7, 50)
    assert abs(np.sum(np.exp(lmu)) - 1.0) < 1e-12
    assert set(ids) == set(np.argsort(-z2)[:50])


def test_sampler_inverse_cdf_counts():
    """Over a fine grid of uniforms the sampler's picks reproduce mu."""
    z = np.array([0.0, np.log(2.0), np.log(5.0), -50.0])
    ids, lmu = behaviour_logprobs(z, 1.0, 3)   # mu = (5, 2, 1) / 8 over ids 2, 1, 0
    N = 8000
    counts = {}
    for i in range(N):
        tok, lm = sample(z, 1.0, 3, (i + 0.5) / N)
        counts[tok] = counts.get(tok, 0) + 1
        assert abs(lm - lmu[list(ids).index(tok)]) < 1e-12
    assert counts == {2: 5000, 1: 2000, 0: 1000}


def test_convex_merge_saturated_gate_selects_each_input():
    """b = +-40 saturates g: u -> e for g = 1 and u -> s for g = 0 (an e/s
    swap in the convex form fails here)."""
    wl = _tiny(merge="convex")
    raw = synth.make_weights(wl)
    raw["merge.wg"][:] = 0
    e, s = _rand(64, 17), _rand(64, 18)
    raw["merge.bg"][:] = 40.0
    assert np.allclose(make_oracle(wl, raw).merge(e, s), e, atol=1e-12)
    raw["merge.bg"][:] = -40.0
    assert np.allclose(make_oracle(wl, raw).merge(e, s), s, atol=1e-12)


def test_gated_merge_concatenation_order():
    """Only the e-half of W_g non-zero and W_s = I:
    u = e + alpha * sigmoid(W_g[:, :d] e + b_g) * RMSNorm_s(s)."""
    wl = _tiny(merge="gated")
    raw = synth.make_weights(wl)
    raw["merge.wg"][:, 64:] = 0
    raw["merge.ws"][:] = np.eye(64, dtype=np.float32)
    orc = make_oracle(wl, raw, alpha=0.5)
    e, s = _rand(64, 19), _rand(64, 20)
    w = orc.w
    g = torch.sigmoid(Fn.linear(torch.from_numpy(e), torch.from_numpy(w["merge.wg"][:, :64]),
                                torch.from_numpy(w["merge.bg"])))
    r = Fn.rms_norm(torch.from_numpy(s), (64,), weight=torch.from_numpy(w["merge.norm"]), eps=wl.eps)
    ref = e + 0.5 * (g * r).numpy()
    assert np.allclose(orc.merge(e, s), ref, rtol=1e-13, atol=1e-13)


def test_readout_is_linear_of_rms_norm():
    """logits = W_o RMSNorm_o(s_t), composed from library linear and rms_norm."""
    wl = _tiny()
    orc = make_oracle(wl)
    s = _rand(64, 21, 3.0)
    w = orc.w
    ref = Fn.linear(Fn.rms_norm(torch.from_numpy(s), (64,), weight=torch.from_numpy(w["out.norm"]),
                                eps=wl.eps), torch.from_numpy(w["out.w"])).numpy()
    assert np.allclose(orc.logits(s), ref, rtol=1e-12, atol=1e-12)
    assert abs(orc.log_prob(s, 5) - torch.log_softmax(torch.from_numpy(ref), 0)[5].item()) < 1e-12


def test_temperature_closed_form():
    """mu proportional to exp(z / tau): z = (log 4, 0), tau = 2 -> mu = (2/3, 1/3)."""
    z = np.array([0.0, np.log(4.0)])
    ids, lmu = behaviour_logprobs(z, 2.0, 0)
    assert list(ids) == [1, 0]
    assert np.allclose(np.exp(lmu), [2.0 / 3.0, 1.0 / 3.0], atol=1e-14)


def test_sampler_boundary_rule():
    """The pick is the first id whose cumulative weight strictly exceeds
    u * total: with two equal weights, u = 0.5 lands on the boundary and picks
    the second id; u = 0 picks the first."""
    z = np.array([0.0, 0.0])
    assert sample(z, 1.0, 0, 0.5)[0] == 1
    assert sample(z, 1.0, 0, 0.0)[0] == 0
    assert sample(z, 1.0, 0, 0.4999)[0] == 0


# ---------------------------------------------------------------------------
# encoder-memory construction [RLT §2.2, eq. (2.2)]
# ---------------------------------------------------------------------------

def _mem_cfg(**kw):
    base = dict(L=1, d=32, H=2, dh=16, W=4, G=1, F=64, V=16)
    base.update(kw)
    return Config(**base)


def test_memory_entry_basis_vector_closed_form():
    """W_K = I, W_V = 2 I, unit gain, e = c * u_i: v is twice the normalised
    basis vector c / sqrt(c^2/d + eps) u_i and k puts the normalised value on
    the rotary pair of coordinate i at the angle t * theta^(-2 i'/dh) (i' = i
    within the head, i' < dh/2: cos on i, sin on i + dh/2) -- written out,
    not through rope()."""
    from oracle import memory_entry
    cfg = _mem_cfg()
    d, dh, I = cfg.d, cfg.dh, np.eye(cfg.d)
    c = 3.0
    for i, t in ((0, 1), (5, 9), (dh + 3, 4096)):
        e = np.zeros(d)
        e[i] = c
        k, v = memory_entry(cfg, e, t, np.ones(d), I, 2.0 * I)
        mag = c / math.sqrt(c * c / d + cfg.eps)
        ev = np.zeros(d)
        ev[i] = 2.0 * mag
        assert np.allclose(v, ev, atol=1e-12)
        h, ii = divmod(i, dh)
        ang = t * cfg.rope_theta ** (-2.0 * ii / dh)
        ek = np.zeros(d)
        ek[h * dh + ii] = mag * math.cos(ang)
        ek[h * dh + ii + dh // 2] = mag * math.sin(ang)
        assert np.allclose(k, ek, atol=1e-12), (i, t)


def test_memory_entry_scale_and_norm_invariants():
    """RMSNorm_E removes the scale of e (up to eps); the rotary transform
    keeps the norm of W_K RMSNorm_E(e); the gain scales the columns."""
    from oracle import memory_entry
    cfg = _mem_cfg()
    d = cfg.d
    e = _rand(d, 11)
    wk, wv = _rand((d, d), 12, 0.2), _rand((d, d), 13, 0.2)
    g = 1 + 0.1 * _rand(d, 14)
    k1, v1 = memory_entry(cfg, e, 17, g, wk, wv)
    k2, v2 = memory_entry(cfg, 7.0 * e, 17, g, wk, wv)
    assert rel_l2(k2, k1) < 1e-6 and rel_l2(v2, v1) < 1e-6
    h = e / np.sqrt(np.mean(e * e) + cfg.eps) * g
    assert abs(np.linalg.norm(k1) - np.linalg.norm(wk @ h)) < 1e-10 * np.linalg.norm(k1)
    # without the positional transform the key is the plain projection
    k0, _ = memory_entry(_mem_cfg(pos="none"), e, 17, g, wk, wv)
    assert np.allclose(k0, wk @ h, atol=1e-12)


def test_memory_keys_relative_position_with_decoder_query():
    """A decoder query rotated at s against a memory key built at t: the score
    depends on s - t only (same rotary form on both sides)."""
    from oracle import memory_entry
    cfg = _mem_cfg()
    d, H, dh = cfg.d, cfg.H, cfg.dh
    e = _rand(d, 21)
    wk, wv = _rand((d, d), 22, 0.3), _rand((d, d), 23, 0.3)
    q = _rand(d, 24)
    for s, t, delta in ((9, 4, 100), (30, 30, 7), (2, 50, 1000)):
        ka, _ = memory_entry(cfg, e, t, np.ones(d), wk, wv)
        kb, _ = memory_entry(cfg, e, t + delta, np.ones(d), wk, wv)
        qa = rope(q, s, H, dh, cfg.rope_theta).reshape(H, dh)
        qb = rope(q, s + delta, H, dh, cfg.rope_theta).reshape(H, dh)
        sa = (qa * ka.reshape(H, dh)).sum(-1)
        sb = (qb * kb.reshape(H, dh)).sum(-1)
        assert np.allclose(sa, sb, rtol=1e-9, atol=1e-9)


def test_build_memory_groups_and_positions():
    """build_memory: group g uses its own weights; row t-1 holds position t."""
    from oracle import build_memory, memory_entry
    cfg = _mem_cfg(G=2)
    d = cfg.d
    E = _rand((6, d), 31)
    mw = {}
    for g in range(2):
        mw["memory.%d.norm_e" % g] = 1 + 0.1 * _rand(d, 40 + g)
        mw["memory.%d.wk" % g] = _rand((d, d), 50 + g, 0.2)
        mw["memory.%d.wv" % g] = _rand((d, d), 60 + g, 0.2)
    mem = build_memory(cfg, E, mw)
    for g in range(2):
        for t in (1, 4, 6):
            k, v = memory_entry(cfg, E[t - 1], t, mw["memory.%d.norm_e" % g], mw["memory.%d.wk" % g],
                                mw["memory.%d.wv" % g])
            assert np.array_equal(mem.k[g][t - 1], k) and np.array_equal(mem.v[g][t - 1], v)
    assert not np.allclose(mem.v[0], mem.v[1])


# ---------------------------------------------------------------------------
# variants: merge gate / rank [RLT §2.5], sublayer order, top-p and the
# trajectory weight [RLT §5.3]
# ---------------------------------------------------------------------------

def _variant_oracle(wl, raw):
    from tests.helpers import oracle_config, oracle_weights
    return Oracle(oracle_config(wl), oracle_weights(raw))


def test_scalar_gate_equals_constant_vector_gate():
    """A scalar gate with w_g = 0, b_g = beta is the vector gate with W_g = 0
    and b_g = beta in every channel (both give sigmoid(beta) everywhere)."""
    wl_v = synth.SMALL.with_(L=1, d=64, H=2, dh=32, F=128, V=64, G=1, dtype="f32")
    wl_s = wl_v.with_(gate="scalar")
    rv, rs = synth.make_weights(wl_v), synth.make_weights(wl_s)
    beta = 0.37
    rv["merge.wg"][:] = 0
    rv["merge.bg"][:] = beta
    rs["merge.wg"][:] = 0
    rs["merge.bg"][:] = beta
    for k in rv:
        if k not in ("merge.wg", "merge.bg"):
            rs[k] = rv[k]
    ov, os_ = _variant_oracle(wl_v, rv), _variant_oracle(wl_s, rs)
    e, s = _rand(64, 71), _rand(64, 72)
    assert np.allclose(ov.merge(e, s), os_.merge(e, s), rtol=1e-13, atol=1e-13)
    # and the scalar really is one value: scaling one channel of W_s r
    # scales that channel's feedback only
    u0 = os_.merge(e, s) - e
    rs2 = dict(rs)
    rs2["merge.ws"] = rs["merge.ws"].copy()
    rs2["merge.ws"][5] *= 2
    u1 = _variant_oracle(wl_s, rs2).merge(e, s) - e
    assert np.allclose(u1[5], 2 * u0[5]) and np.allclose(np.delete(u1, 5), np.delete(u0, 5))


def test_low_rank_ws_equals_full_product():
    """W_s = U V given as factors equals the full matrix U @ V (the full path
    is pinned by the merge tests above)."""
    wl_f = synth.SMALL.with_(L=1, d=64, H=2, dh=32, F=128, V=64, G=1, dtype="f32")
    wl_r = wl_f.with_(ws_rank=32)
    rf, rr = synth.make_weights(wl_f), synth.make_weights(wl_r)
    for k in rf:
        if k != "merge.ws":
            rr[k] = rf[k]
    rf["merge.ws"] = (rr["merge.ws_u"].astype(np.float64) @ rr["merge.ws_v"].astype(np.float64)).astype(np.float32)
    e, s = _rand(64, 81), _rand(64, 82)
    a = _variant_oracle(wl_f, rf).merge(e, s)
    b = _variant_oracle(wl_r, rr).merge(e, s)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-7)


def _run_steps(orc, wl, n=5):
    mem = memory_of(wl, 0, T=n)
    st = orc.initial_state()
    out = []
    for t in range(1, n + 1):
        st = orc.transition(st, e_of(wl, 0, T=n)[t - 1], mem)
        out.append(st.s)
    return np.array(out)


def test_sublayer_order_with_identity_sublayers():
    """With the FFN switched off (W_down = 0) the FFN sublayer is the
    identity, so "sfx" equals "sxf"; with the cross-attention output
    projection zero, "xsf" equals "sxf". Orders whose non-trivial sublayers
    are permuted differ."""
    wl = synth.SMALL.with_(L=2, d=64, H=2, dh=32, F=128, V=64, G=1, W=4, dtype="f32")
    raw = synth.make_weights(wl)
    no_ffn = dict(raw)
    no_x = dict(raw)
    for l in range(wl.L):
        no_ffn["layer.%d.w_down" % l] = np.zeros_like(raw["layer.%d.w_down" % l])
        no_x["layer.%d.wom" % l] = np.zeros_like(raw["layer.%d.wom" % l])
    ref_f = _run_steps(_variant_oracle(wl, no_ffn), wl)
    assert np.allclose(_run_steps(_variant_oracle(wl.with_(order="sfx"), no_ffn), wl), ref_f, rtol=1e-12, atol=1e-12)
    ref_x = _run_steps(_variant_oracle(wl, no_x), wl)
    assert np.allclose(_run_steps(_variant_oracle(wl.with_(order="xsf"), no_x), wl), ref_x, rtol=1e-12, atol=1e-12)
    full = _run_steps(_variant_oracle(wl, raw), wl)
    assert rel_l2(_run_steps(_variant_oracle(wl.with_(order="fxs"), raw), wl), full) > 1e-4


def test_top_p_closed_forms():
    """Uniform logits: the nucleus at p = 1/2 is the first V/2 ids (id order)
    with mu = 2/V each; p -> 0 keeps the argmax only (mu = 1); p = 1 is no
    nucleus; p is applied after top-k (mass renormalised over the top-k)."""
    V = 16
    ids, lmu = behaviour_logprobs(np.zeros(V), 1.0, 0, 0.5)
    assert ids.tolist() == list(range(V // 2)) and np.allclose(lmu, math.log(2.0 / V))
    z = _rand(V, 91)
    ids, lmu = behaviour_logprobs(z, 0.7, 0, 1e-9)
    assert ids.tolist() == [int(np.argmax(z))] and abs(lmu[0]) < 1e-15
    a = behaviour_logprobs(z, 0.7, 5, 1.0)
    b = behaviour_logprobs(z, 0.7, 5)
    assert np.array_equal(a[0], b[0]) and np.allclose(a[1], b[1])
    # explicit: logits 3, 2, 1, 0 at tau = 1 -> p = e^3, e^2, e^1, 1 over S
    z4 = np.array([0.0, 3.0, 1.0, 2.0])
    w = np.exp([3.0, 2.0, 1.0, 0.0])
    P = w / w.sum()                        # ordered ids 1, 3, 2, 0
    ids, lmu = behaviour_logprobs(z4, 1.0, 0, P[0] + P[1] - 1e-12)
    assert ids.tolist() == [1, 3] and np.allclose(np.exp(lmu), w[:2] / w[:2].sum())
    ids, lmu = behaviour_logprobs(z4, 1.0, 3, 0.999)  # top-3 first, then all 3 needed
    assert ids.tolist() == [1, 3, 2]


def test_trajectory_log_ratio_is_log_of_product():
    from oracle import trajectory_log_ratio
    lp = _rand(7, 101) - 3
    lm = _rand(7, 102) - 3
    prod = 1.0
    for a, b in zip(lp, lm):
        prod *= importance_ratio(a, b)
    assert math.isclose(math.exp(trajectory_log_ratio(lp, lm)), prod, rel_tol=1e-12)
    assert trajectory_log_ratio([], []) == 0.0


# ---------------------------------------------------------------------------
# replay scoring index ("Recurrent Looped Transformer" App. A.4 and App. A.2)
# ---------------------------------------------------------------------------

# A hand-written token table: x_1 .. x_5 (1-based as in the report). The
# literals below are the ids each scored position must use, written out
# rather than indexed from the table, so that an off-by-one in the replay's
# token index (scoring x_t instead of x_{t+1}) changes every expected value.
REPLAY_X = [7, 11, 22, 33, 44]
REPLAY_EXPECT = {2: 22, 3: 33, 4: 44}   # split = 2, length = 5: t -> x_{t+1}


def _replay_fixture():
    wl = _tiny(T=8)
    orc = make_oracle(wl)
    mem, E = memory_of(wl, 0), e_of(wl, 0)
    return wl, orc, mem, E


def test_replay_scores_next_token_before_consuming_it():
    """App. A.4: after consuming x_t (t >= split) the replay reads
    log p(x_{t+1} | x_{1:t}) from s_t, before x_{t+1} is consumed; x_len is
    never consumed (App. A.2, pending). The states come from explicit
    transitions, the scored ids from the literal table above."""
    wl, orc, mem, E = _replay_fixture()
    final, logp, ss = replay(orc, E, mem, np.array(REPLAY_X), 5, 2)
    assert sorted(logp) == [2, 3, 4]
    st = orc.initial_state()
    states = {}
    for t in (1, 2, 3, 4):
        st = orc.transition(st, E[t - 1], mem)
        states[t] = st.s
    for t, tok in REPLAY_EXPECT.items():
        assert logp[t] == orc.log_prob(states[t], tok), t
        # a neighbouring id scores differently (the pin can see an index slip)
        assert logp[t] != orc.log_prob(states[t], REPLAY_X[t - 1])
    assert final.pos == 4 and np.array_equal(final.s, states[4])
    assert len(ss) == 4 and np.array_equal(ss[1], states[2])


def test_gradient_twin_scores_next_token():
    """The autograd twin of the replay scores the same literal ids."""
    from oracle.rlt_grad import replay_loss
    import torch as _t
    wl, orc, mem, E = _replay_fixture()
    cfg = orc.cfg
    w = {k: _t.tensor(np.asarray(v, dtype=np.float64)) for k, v in orc.w.items()}
    seq = dict(E=_t.tensor(E), mem_k=[_t.tensor(m) for m in mem.k], mem_v=[_t.tensor(m) for m in mem.v],
               tokens=np.array(REPLAY_X), length=5, split=2, w=np.ones(5))
    _, lps = replay_loss(cfg, w, [seq])
    st = orc.initial_state()
    for t in (1, 2, 3, 4):
        st = orc.transition(st, E[t - 1], mem)
        if t in REPLAY_EXPECT:
            assert abs(float(lps[0][t]) - orc.log_prob(st.s, REPLAY_EXPECT[t])) < 1e-10, t
    assert sorted(lps[0]) == [2, 3, 4]
