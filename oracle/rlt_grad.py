"""Gradient oracle of the replayed decoder recurrence (full BPTT).

TEST INFRASTRUCTURE ONLY, like ``rlt_oracle``: the product path never
imports it.

Source: "Recurrent Looped Transformer" (Y. Zhang, technical report, 2026).
The training computation differentiates the full-history replay through the
recurrent outputs s_t, the decoder SWA keys/values and the encoder memory
[RLT §5.4]; the state-to-state Jacobian has cross terms through the decoder
cache, so no path is detached [RLT App. B, eqs. (B.1)-(B.5)]. The loss used
here is linear in the replayed log-probabilities,

    L = sum_b sum_{t = split_b}^{len_b - 1} w_b[t] * log p(x_{t+1} | x_{1:t}),

which covers next-token likelihood (w = -1) and score-function surrogates
(w = advantages) [RLT §5.3, eq. (5.4)].

This module is a float64 PyTorch twin of ``rlt_oracle``'s transition (the
default variants: vector gate, full-rank W_s, sublayer order SWA, cross,
FFN) whose gradients come from autograd. It is pinned to the NumPy oracle by
equal log-probabilities and, per parameter tensor, by central finite
differences of the NumPy oracle's loss.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np
import torch

from .rlt_oracle import Config, rope_angles, window_positions


def _rms(x: torch.Tensor, gain: torch.Tensor, eps: float) -> torch.Tensor:
    return x / torch.sqrt(torch.mean(x * x) + eps) * gain


def _rope(x: torch.Tensor, t: int, cfg: Config) -> torch.Tensor:
    if cfg.pos != "rope":
        return x
    c, s = rope_angles(t, cfg.dh, cfg.rope_theta)
    c = torch.from_numpy(c)
    s = torch.from_numpy(s)
    xh = x.reshape(cfg.H, cfg.dh)
    a, b = xh[:, : cfg.dh // 2], xh[:, cfg.dh // 2:]
    return torch.cat([a * c - b * s, b * c + a * s], dim=1).reshape(-1)


def _attend(q: torch.Tensor, keys: torch.Tensor, values: torch.Tensor, cfg: Config) -> torch.Tensor:
    qh = q.reshape(cfg.H, cfg.dh)
    kh = keys.reshape(keys.shape[0], cfg.H, cfg.dh)
    vh = values.reshape(values.shape[0], cfg.H, cfg.dh)
    out = []
    for h in range(cfg.H):
        p = torch.softmax(kh[:, h, :] @ qh[h] / math.sqrt(cfg.dh), dim=0)
        out.append(p @ vh[:, h, :])
    return torch.cat(out)


def _transition(cfg: Config, w: Dict[str, torch.Tensor], s_prev: torch.Tensor, e: torch.Tensor, t: int,
                hist: List[Dict[int, Tuple[torch.Tensor, torch.Tensor]]], mk: Sequence[torch.Tensor],
                mv: Sequence[torch.Tensor]) -> torch.Tensor:
    """s_t from s_{t-1}, e_t, the decoder cache and the memory prefix, as
    ``rlt_oracle.Oracle.transition`` [RLT §2.3 eqs. (2.4)-(2.5), §2.5]."""
    if cfg.merge == "gated":
        r = _rms(s_prev, w["merge.norm"], cfg.eps)
        g = torch.sigmoid(w["merge.wg"] @ torch.cat([e, r]) + w["merge.bg"])
        z = e + cfg.alpha * g * (w["merge.ws"] @ r)
    else:
        g = torch.sigmoid(w["merge.wg"] @ torch.cat([e, s_prev]) + w["merge.bg"])
        z = g * e + (1.0 - g) * s_prev
    for l in range(cfg.L):
        p = "layer.%d." % l
        h = _rms(z, w[p + "norm_s"], cfg.eps)
        q = _rope(w[p + "wq"] @ h, t, cfg)
        k = _rope(w[p + "wk"] @ h, t, cfg)
        v = w[p + "wv"] @ h
        win = window_positions(t, cfg.W)
        keys = torch.stack([hist[l][j][0] for j in win[:-1]] + [k])
        vals = torch.stack([hist[l][j][1] for j in win[:-1]] + [v])
        z = z + w[p + "wo"] @ _attend(q, keys, vals, cfg)
        hist[l][t] = (k, v)  # kept whole: BPTT needs every entry a later window read
        gi = cfg.group_of(l)
        qm = _rope(w[p + "wqm"] @ _rms(z, w[p + "norm_m"], cfg.eps), t, cfg)
        z = z + w[p + "wom"] @ _attend(qm, mk[gi][:t], mv[gi][:t], cfg)
        hd = _rms(z, w[p + "norm_d"], cfg.eps)
        z = z + w[p + "w_down"] @ (torch.nn.functional.silu(w[p + "w_gate"] @ hd) * (w[p + "w_up"] @ hd))
    return z


def _log_prob(cfg: Config, w: Dict[str, torch.Tensor], s: torch.Tensor, token: int) -> torch.Tensor:
    z = w["out.w"] @ _rms(s, w["out.norm"], cfg.eps)
    return torch.log_softmax(z, dim=0)[token]


def check_supported(cfg: Config) -> None:
    if cfg.gate != "vector" or cfg.ws_rank != 0 or cfg.order != "sxf":
        raise ValueError("the gradient oracle covers the vector gate, full-rank W_s and order sxf")


def replay_loss(cfg: Config, w: Dict[str, torch.Tensor], seqs: Sequence[dict]):
    """Loss L and the log-probabilities of each sequence's replay from H_0
    [RLT App. A.4]. A sequence dict holds E [len, d], mem_k / mem_v
    (lists over groups of [>= len, d]), tokens [len], length, split and
    w [len] (w[t] weights log p(x_{t+1} | x_{1:t}))."""
    check_supported(cfg)
    loss = torch.zeros((), dtype=torch.float64)
    logps = []
    for sq in seqs:
        s = w["s_star"]
        hist = [dict() for _ in range(cfg.L)]
        lp = {}
        for t in range(1, sq["length"]):
            s = _transition(cfg, w, s, sq["E"][t - 1], t, hist, sq["mem_k"], sq["mem_v"])
            if t >= sq["split"]:
                lp[t] = _log_prob(cfg, w, s, int(sq["tokens"][t]))
                loss = loss + float(sq["w"][t]) * lp[t]
        logps.append(lp)
    return loss, logps


def replay_grads(cfg: Config, weights: Dict[str, np.ndarray], seqs: Sequence[dict]):
    """Full-BPTT gradients of L [RLT §5.4, App. B] with respect to every
    parameter, every sequence's e_t and every memory entry.

    Returns (L, [ {t: log p} per sequence ], {name: dL/dparam},
    [dL/dE per sequence], [[dL/dmem_k per group] per sequence],
    [[dL/dmem_v per group] per sequence])."""
    w = {k: torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True) for k, v in weights.items()}
    tseqs = []
    for sq in seqs:
        tq = dict(sq)
        tq["E"] = torch.tensor(np.asarray(sq["E"], dtype=np.float64), requires_grad=True)
        tq["mem_k"] = [torch.tensor(np.asarray(m, dtype=np.float64), requires_grad=True) for m in sq["mem_k"]]
        tq["mem_v"] = [torch.tensor(np.asarray(m, dtype=np.float64), requires_grad=True) for m in sq["mem_v"]]
        tseqs.append(tq)
    loss, logps = replay_loss(cfg, w, tseqs)
    leaves = list(w.values())
    for tq in tseqs:
        leaves += [tq["E"]] + tq["mem_k"] + tq["mem_v"]
    grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    out = {}
    it = iter(grads)
    for k, v in w.items():
        gk = next(it)
        out[k] = np.zeros(v.shape) if gk is None else gk.numpy()
    dE, dK, dV = [], [], []
    G = cfg.G
    for tq in tseqs:
        gE = next(it)
        dE.append(np.zeros(tq["E"].shape) if gE is None else gE.numpy())
        ks = [next(it) for _ in range(G)]
        vs = [next(it) for _ in range(G)]
        dK.append([np.zeros(m.shape) if gk is None else gk.numpy() for m, gk in zip(tq["mem_k"], ks)])
        dV.append([np.zeros(m.shape) if gv is None else gv.numpy() for m, gv in zip(tq["mem_v"], vs)])
    lp_np = [{t: float(v.detach()) for t, v in lp.items()} for lp in logps]
    return float(loss.detach()), lp_np, out, dE, dK, dV
