"""GPU replay backward against the gradient oracle ("Recurrent Looped
Transformer" §5.4, App. B): full BPTT of L = sum_b sum_t w[b,t] log p(x_{t+1})
through s_t, the decoder keys/values (also after they leave the window) and
the memory, on ragged sequences replayed from H_0.

Gate: every gradient tensor (each parameter, e_t, the memory keys and values)
within relative L2 1e-4 of the float64 oracle, computed on the same
parameter values (bf16 parameters widened exactly), since the backward
computes in float32 throughout; log-probabilities of the replay within 1e-5.
"""
import numpy as np
import pytest

import synth
from oracle.rlt_grad import replay_grads
from tests.gpu_common import GpuRun, require_gpu, torch
from tests.helpers import oracle_config, oracle_weights, rel_l2, widen

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _case(wl, lens, splits, seed=7, launch=None, raw=None):
    run = GpuRun(wl, B=len(lens), T=max(lens), launch=launch, raw=raw)
    rng = np.random.default_rng(seed)
    B, T = len(lens), max(lens)
    tokens = rng.integers(0, wl.V, (B, T)).astype(np.int32)
    w = rng.standard_normal((B, T)).astype(np.float32)
    return run, tokens, w


def _gpu_backward(run, lens, splits, tokens, w):
    B, T, d, G = len(lens), max(lens), run.wl.d, run.wl.G
    grads = run.dec.grad_buffers()
    logp = torch.zeros((B, T), device="cuda")
    de = torch.zeros((B, T, d), device="cuda")
    dmk = torch.zeros((G, B, T, d), device="cuda")
    dmv = torch.zeros((G, B, T, d), device="cuda")
    rc = run.dec.replay_backward(grads, np.array(lens), np.array(splits), run.Ed, run.mem,
                                 torch.from_numpy(tokens).cuda(), torch.from_numpy(w).cuda(), logp=logp, de=de,
                                 dmem_k=dmk, dmem_v=dmv)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return ({k: v.double().cpu().numpy() for k, v in grads.items()}, logp.double().cpu().numpy(),
            de.double().cpu().numpy(), dmk.double().cpu().numpy(), dmv.double().cpu().numpy())


def _oracle(run, lens, splits, tokens, w):
    wl = run.wl
    cfg = oracle_config(wl)
    seqs = []
    for b, (n, sp) in enumerate(zip(lens, splits)):
        seqs.append(dict(E=widen(run.E[b, :n]), mem_k=[widen(run.mk[g, b, :n]) for g in range(wl.G)],
                         mem_v=[widen(run.mv[g, b, :n]) for g in range(wl.G)], tokens=tokens[b, :n], length=n,
                         split=sp, w=w[b, :n].astype(np.float64)))
    return replay_grads(cfg, oracle_weights(run.raw), seqs)


def _check(run, lens, splits, tokens, w):
    g_gpu, logp, de, dmk, dmv = _gpu_backward(run, lens, splits, tokens, w)
    _, lps, g_ref, dE, dK, dV = _oracle(run, lens, splits, tokens, w)
    worst = 0.0
    for name, ref in g_ref.items():
        if name not in g_gpu:
            continue
        e = rel_l2(g_gpu[name].reshape(ref.shape), ref)
        worst = max(worst, e)
        assert e <= TOL, (name, e)
    for b, n in enumerate(lens):
        for t, v in lps[b].items():
            assert abs(logp[b, t] - v) < 1e-5, (b, t)
        # e_t of the consumed tokens; e_len and later positions take no part
        e = rel_l2(de[b, : n - 1], dE[b][: n - 1])
        worst = max(worst, e)
        assert e <= TOL, ("de", b, e)
        assert np.all(de[b, n - 1:] == 0)
        for g in range(run.wl.G):
            for got, ref, nm in ((dmk, dK, "dmem_k"), (dmv, dV, "dmem_v")):
                e = rel_l2(got[g, b, : n - 1], ref[b][g][: n - 1])
                worst = max(worst, e)
                assert e <= TOL, (nm, b, g, e)
                assert np.all(got[g, b, n - 1:] == 0)
    return worst


@pytest.mark.parametrize("merge,G", [("gated", 1), ("convex", 2)])
def test_backward_tiny_f32(merge, G):
    require_gpu()
    wl = synth.TINY.with_(dtype="f32", merge=merge, G=G, W=3)
    lens, splits = [9, 6, 2], [2, 1, 1]
    run, tokens, w = _case(wl, lens, splits)
    worst = _check(run, lens, splits, tokens, w)
    print("tiny f32 %s G=%d: worst rel L2 %.2e" % (merge, G, worst))


def test_backward_small_bf16_parameters():
    """bf16 parameters, e and memory (widened exactly on both sides), G = L
    (one memory group per layer), window 16 wider than the sequences."""
    require_gpu()
    wl = synth.SMALL
    lens, splits = [12, 7, 10], [3, 1, 9]
    run, tokens, w = _case(wl, lens, splits)
    worst = _check(run, lens, splits, tokens, w)
    print("small bf16: worst rel L2 %.2e" % worst)


def test_backward_window_eviction_and_determinism():
    """Window 2 on 14 steps: every key leaves the window one step after it is
    written; gradients of earlier steps still flow through the states that
    read it. A repeated call gives bit-identical gradients, and a call into
    filled buffers adds to them."""
    require_gpu()
    wl = synth.SMALL.with_(W=2, G=1, dtype="f32")
    lens, splits = [15, 11], [4, 2]
    run, tokens, w = _case(wl, lens, splits, seed=9)
    _check(run, lens, splits, tokens, w)
    g1, g2 = run.dec.grad_buffers(), run.dec.grad_buffers()
    args = (np.array(lens), np.array(splits), run.Ed, run.mem, torch.from_numpy(tokens).cuda(),
            torch.from_numpy(w).cuda())
    assert run.dec.replay_backward(g1, *args) == 0
    assert run.dec.replay_backward(g2, *args) == 0
    g3 = {k: v.clone() for k, v in g1.items()}
    assert run.dec.replay_backward(g3, *args) == 0
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
        assert rel_l2(g3[k].double().cpu().numpy(), 2 * g1[k].double().cpu().numpy()) < 1e-6, k


def test_backward_logp_matches_replay_sequence():
    """The backward's replay (float32 configuration) gives the log-probs of
    rlt_replay_sequence up to summation order."""
    require_gpu()
    wl = synth.SMALL.with_(dtype="f32", B=3)
    lens, splits = [10, 8, 3], [1, 2, 1]
    run, tokens, w = _case(wl, lens, splits)
    g_gpu, logp, *_ = _gpu_backward(run, lens, splits, tokens, w)
    run.init()
    ref = torch.zeros((3, max(lens)), device="cuda")
    assert run.dec.replay(run.st, np.array(lens), np.array(splits), run.Ed, run.mem,
                          torch.from_numpy(tokens).cuda(), ref) == 0
    torch.cuda.synchronize()
    ref = ref.double().cpu().numpy()
    for b, (n, sp) in enumerate(zip(lens, splits)):
        assert np.allclose(logp[b, sp:n], ref[b, sp:n], atol=2e-5, rtol=0), b


def test_backward_kept_and_recomputed_activations():
    """Activations kept from the forward pass (the choice when they fit) and
    recomputed per step (per-step checkpointing) [RLT §5.4, App. C]: the
    recompute runs the same kernels on the same inputs, so log-probabilities,
    e and memory gradients are the same bits; the parameter gradients differ
    only in summation order (one product or column sum over every step's rows
    when kept, step by step otherwise)."""
    require_gpu()
    wl = synth.SMALL
    lens, splits = [12, 7, 10, 3], [3, 1, 9, 2]
    outs = []
    raw = None
    for mode in (1, 2):
        run, tokens, w = _case(wl, lens, splits, seed=11, launch={"bwd_activations": mode}, raw=raw)
        raw = run.raw
        outs.append(_gpu_backward(run, lens, splits, tokens, w))
        run.dec.close()
    (g1, *r1), (g2, *r2) = outs
    for k in g1:
        assert rel_l2(g2[k], g1[k]) < 1e-6, k
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)


def test_backward_rejects_unsupported_variants():
    require_gpu()
    from stateful_sequence_model_amd import _abi
    wl = synth.SMALL.with_(gate="scalar")
    run, tokens, w = _case(wl, [4], [1])
    rc = run.dec.replay_backward(run.dec.grad_buffers(), np.array([4]), np.array([1]), run.Ed, run.mem,
                                 torch.from_numpy(tokens).cuda(), torch.from_numpy(w).cuda())
    assert rc == _abi.RLT_EUNSUPPORTED
