"""Pins of the gradient oracle (``oracle.rlt_grad``), CPU only.

The float64 autograd twin must (1) replay the same log-probabilities as the
pinned NumPy oracle and (2) give, for every parameter tensor, for e_t and for
the memory entries, directional derivatives equal to central finite
differences of the NumPy oracle's loss ("Recurrent Looped Transformer" §5.4,
App. B: full BPTT through s_t, the decoder cache and the memory). A dropped
path (for example through the decoder keys/values of earlier positions) or a
wrong sign in any tensor's gradient fails (2).
"""
import numpy as np
import pytest

import synth
from oracle import Memory, Oracle, replay
from oracle.rlt_grad import replay_grads
from tests.helpers import oracle_config, oracle_weights, rel_l2

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _problem(merge, G, lens=(7, 5), splits=(2, 1), seed=3):
    wl = synth.TINY.with_(dtype="f32", merge=merge, G=G, W=3)
    cfg = oracle_config(wl)
    w = oracle_weights(synth.make_weights(wl))
    rng = np.random.default_rng(seed)
    seqs = []
    for b, (n, sp) in enumerate(zip(lens, splits)):
        seqs.append(dict(E=rng.standard_normal((n, wl.d)),
                         mem_k=[rng.standard_normal((n, wl.d)) for _ in range(G)],
                         mem_v=[rng.standard_normal((n, wl.d)) for _ in range(G)],
                         tokens=rng.integers(0, wl.V, n), length=n, split=sp,
                         w=rng.standard_normal(n)))
    return cfg, w, seqs


def _np_loss(cfg, w, seqs):
    orc = Oracle(cfg, w)
    tot = 0.0
    lps = []
    for sq in seqs:
        _, lp, _ = replay(orc, sq["E"], Memory(sq["mem_k"], sq["mem_v"]), sq["tokens"], sq["length"], sq["split"])
        tot += sum(sq["w"][t] * v for t, v in lp.items())
        lps.append(lp)
    return tot, lps


@pytest.mark.parametrize("merge,G", [("gated", 1), ("convex", 2)])
def test_twin_replays_the_oracle_log_probs(merge, G):
    cfg, w, seqs = _problem(merge, G)
    L, lps, *_ = replay_grads(cfg, w, seqs)
    L_np, lps_np = _np_loss(cfg, w, seqs)
    assert abs(L - L_np) <= 1e-11 * max(1.0, abs(L_np))
    for a, b in zip(lps, lps_np):
        assert a.keys() == b.keys()
        for t in a:
            assert abs(a[t] - b[t]) < 1e-11


def _fd(f, x, d, eps=1e-5):
    return (f(x + eps * d) - f(x - eps * d)) / (2 * eps)


@pytest.mark.parametrize("merge,G", [("gated", 1), ("convex", 2)])
def test_parameter_gradients_match_finite_differences(merge, G):
    cfg, w, seqs = _problem(merge, G)
    _, _, grads, _, _, _ = replay_grads(cfg, w, seqs)
    rng = np.random.default_rng(11)
    for name in sorted(w):
        d = rng.standard_normal(w[name].shape)

        def f(x, name=name):
            ww = dict(w)
            ww[name] = x
            return _np_loss(cfg, ww, seqs)[0]

        fd = _fd(f, w[name], d)
        an = float(np.sum(grads[name] * d))
        assert abs(fd - an) <= 1e-6 * max(1e-3, abs(fd)), (name, fd, an)


@pytest.mark.parametrize("merge,G", [("gated", 1), ("convex", 2)])
def test_input_and_memory_gradients_match_finite_differences(merge, G):
    cfg, w, seqs = _problem(merge, G)
    _, _, _, dE, dK, dV = replay_grads(cfg, w, seqs)
    rng = np.random.default_rng(12)
    for b in range(len(seqs)):
        def fe(x, b=b):
            ss = [dict(s) for s in seqs]
            ss[b]["E"] = x
            return _np_loss(cfg, w, ss)[0]

        d = rng.standard_normal(seqs[b]["E"].shape)
        assert abs(_fd(fe, seqs[b]["E"], d) - np.sum(dE[b] * d)) <= 1e-6 * max(1e-3, abs(np.sum(dE[b] * d)))
        for g in range(G):
            for which, grad in (("mem_k", dK), ("mem_v", dV)):
                def fm(x, b=b, g=g, which=which):
                    ss = [dict(s) for s in seqs]
                    ss[b][which] = list(ss[b][which])
                    ss[b][which][g] = x
                    return _np_loss(cfg, w, ss)[0]

                d = rng.standard_normal(seqs[b][which][g].shape)
                an = float(np.sum(grad[b][g] * d))
                assert abs(_fd(fm, seqs[b][which][g], d) - an) <= 1e-6 * max(1e-3, abs(an)), (b, g, which)


def test_unread_positions_get_no_gradient():
    """Memory positions past a sequence's last consumed token and e_len (x_len
    is never consumed) take no part in the loss (Prop. B.1)."""
    cfg, w, seqs = _problem("gated", 1, lens=(6,), splits=(3,))
    seqs[0]["mem_k"] = [np.vstack([seqs[0]["mem_k"][0], np.ones((3, cfg.d))])]
    seqs[0]["mem_v"] = [np.vstack([seqs[0]["mem_v"][0], np.ones((3, cfg.d))])]
    _, _, _, dE, dK, dV = replay_grads(cfg, w, seqs)
    assert np.all(dE[0][5:] == 0)
    assert np.all(dK[0][0][5:] == 0) and np.all(dV[0][0][5:] == 0)
    assert np.any(dK[0][0][:5] != 0)


def test_cache_path_carries_gradient():
    """The decoder-cache path of the state Jacobian (App. B, eq. (B.3)) is
    live: the gradient of W_k of layer 0 changes when the window widens."""
    cfg, w, seqs = _problem("gated", 1)
    _, _, g3, _, _, _ = replay_grads(cfg, w, seqs)
    cfg1 = cfg.__class__(**{**cfg.__dict__, "W": 1})
    _, _, g1, _, _, _ = replay_grads(cfg1, w, seqs)
    assert rel_l2(g1["layer.0.wk"], g3["layer.0.wk"]) > 1e-3
