"""GPU parity of the variants ("Recurrent Looped Transformer" §2.5 text
after eqs. (2.11) and (2.16), §5.3): scalar merge gate, low-rank W_s,
sublayer orders, top-p behaviour sampling and the trajectory weight.

Gates: bf16 relative L2 <= 2e-2 per (row, step) on s_t and logits with
top-1 agreement outside near-ties; float32 1e-4; sampling re-derived by the
oracle from the GPU's own logits (the token exactly, up to a boundary case
the two precisions may resolve differently).
"""
import math

import numpy as np
import pytest

import synth
from oracle import Oracle, behaviour_logprobs, trajectory_log_ratio
from tests.gpu_common import GpuRun, require_gpu, torch
from tests.helpers import memory_of, oracle_config, oracle_weights, rel_l2, widen

pytestmark = pytest.mark.gpu

BASE = synth.SMALL.with_(B=4, T=16)


def _run_vs_oracle(wl, nsteps, tol):
    run = GpuRun(wl)
    run.init()
    S, Z = run.run(nsteps)
    orc = Oracle(oracle_config(wl), oracle_weights(run.raw))
    worst = 0.0
    for b in range(wl.B):
        mem = memory_of(wl, b, T=wl.T)
        st = orc.initial_state()
        for t in range(1, nsteps + 1):
            st = orc.transition(st, widen(run.E[b, t - 1]), mem)
            zo = orc.logits(st.s)
            es, ez = rel_l2(S[t - 1, b], st.s), rel_l2(Z[t - 1, b], zo)
            worst = max(worst, es, ez)
            assert es < tol and ez < tol, (wl.gate, wl.ws_rank, wl.order, b, t, es, ez)
            if np.argmax(Z[t - 1, b]) != np.argmax(zo):
                top2 = np.sort(zo)[-2:]
                assert top2[1] - top2[0] <= np.abs(Z[t - 1, b] - zo).max(), (b, t)
    return worst


@pytest.mark.parametrize("over", [
    dict(gate="scalar"),
    dict(ws_rank=64),
    dict(order="xsf"),
    dict(order="fxs"),
    dict(gate="scalar", ws_rank=32, order="sfx"),
], ids=["scalar-gate", "rank64", "order-xsf", "order-fxs", "combined"])
def test_variant_bf16(over):
    require_gpu()
    wl = BASE.with_(**over)
    worst = _run_vs_oracle(wl, 8, 2e-2)
    print("variant %s: worst rel L2 %.2e" % (over, worst))


def test_variant_combined_f32():
    require_gpu()
    wl = BASE.with_(dtype="f32", gate="scalar", ws_rank=32, order="xfs")
    worst = _run_vs_oracle(wl, 8, 1e-4)
    print("variant f32 combined: worst rel L2 %.2e" % worst)


def test_top_p_sampling_and_scoring_on_gpu_logits():
    """Temperature 0.8, top-k 64, nucleus 0.9: the sampled token and its log
    mu against the oracle on the GPU's logits; the scoring API's log mu of
    the argmax (in every nucleus) and of the argmin (-inf, outside) against
    the oracle's logits of the same states."""
    require_gpu()
    wl = synth.SMALL.with_(B=16, T=12)
    run = GpuRun(wl)
    run.init()
    B, V = wl.B, wl.V
    tau, k, p = 0.8, 64, 0.9
    logits = torch.empty((B, V), device="cuda")
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    lmu = torch.empty(B, device="cuda")
    outside = 0
    for t in range(1, 9):
        u = torch.from_numpy(synth.uniform01(wl.seed, "u_p", B, start=t * B)).cuda()
        assert run.step(range(B), t, logits=logits, uniform=u, temperature=tau, top_k=k, top_p=p,
                        sample_tok=tok, sample_logmu=lmu) == 0
        torch.cuda.synchronize()
        Zg = logits.cpu().numpy().astype(np.float64)
        for b in range(B):
            ids, lm = behaviour_logprobs(Zg[b], tau, k, p)
            w = np.exp(lm - lm.max())
            cum = np.cumsum(w)
            target = float(u[b]) * cum[-1]
            i = int(np.searchsorted(cum, target, side="right"))
            assert int(tok[b]) in ids.tolist(), (t, b)
            g = list(ids).index(int(tok[b]))
            if g != i:
                assert abs(cum[min(g, i)] - target) <= 1e-5 * cum[-1], (t, b)
            assert abs(float(lmu[b]) - lm[g]) < 1e-4
        # scoring API (its own logits from s) on every row's argmax (rank 0,
        # always in the nucleus) and argmin (never in it), against the oracle's
        # float64 logits of the same states
        s = run.st.s[:B].contiguous()
        orc = Oracle(oracle_config(wl), oracle_weights(run.raw))
        Zo = [orc.logits(s[b].double().cpu().numpy()) for b in range(B)]
        for pick, inside in ((np.argmax, True), (np.argmin, False)):
            toks = torch.tensor([int(pick(Zo[b])) for b in range(B)], dtype=torch.int32, device="cuda")
            logp = torch.empty(B, device="cuda")
            logmu = torch.empty(B, device="cuda")
            assert run.dec.score(s, toks, logp, temperature=tau, top_k=k, top_p=p, logmu=logmu) == 0
            torch.cuda.synchronize()
            for b in range(B):
                ids, lm = behaviour_logprobs(Zo[b], tau, k, p)
                if inside:
                    assert abs(float(logmu[b]) - lm[0]) < 2e-2
                else:
                    assert float(logmu[b]) == -math.inf
                    outside += 1
    assert outside == 8 * B


def test_trajectory_log_ratio_matches_oracle():
    """Sum of log p - log mu over each sequence's scored positions (float32
    on the GPU) against the oracle's float64 sum; an empty range gives 0."""
    require_gpu()
    wl = synth.SMALL.with_(B=5, T=300)
    run = GpuRun(wl, T=8)
    rng = np.random.default_rng(5)
    lens = np.array([300, 17, 2, 255, 128], dtype=np.int32)
    splits = np.array([1, 16, 1, 100, 128], dtype=np.int32)
    lp = (rng.standard_normal((5, 300)) - 3).astype(np.float32)
    lm = (rng.standard_normal((5, 300)) - 3).astype(np.float32)
    out = torch.empty(5, device="cuda")
    assert run.dec.trajectory_log_ratio(lens, splits, torch.from_numpy(lp).cuda(), torch.from_numpy(lm).cuda(),
                                        out) == 0
    torch.cuda.synchronize()
    for b in range(5):
        ref = trajectory_log_ratio(lp[b, splits[b]:lens[b]], lm[b, splits[b]:lens[b]])
        assert abs(float(out[b]) - ref) <= 1e-5 * max(1.0, abs(ref)), (b, float(out[b]), ref)
