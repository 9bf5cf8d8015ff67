"""CPU oracle of the Recurrent Looped Transformer decoder state transition.

TEST INFRASTRUCTURE ONLY. This module is the correctness reference for the
GPU library. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run it; the product path never does, and the
oracle shares no code with the GPU path (inputs come from the separate
seeded generator module ``synth``).

Source: "Recurrent Looped Transformer" (Y. Zhang, technical report, 2026),
cited below as [RLT §x, eq. (y)]; its project page is cited as
[RLT project page]. Everything is plain NumPy in float64 unless a caller asks
for float32; matrices are the natural [out, in] layout and vectors are
column vectors, as in the report.

Readings where the report leaves a step open (each one is a convention the
report does not fix, so these parts are "parity unpinned" by the report
itself and are fixed here as a specification):
  * RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gain.
  * One pre-norm RMSNorm_{S,l} feeds the SWA query, key and value maps; the
    cross-attention query has its own RMSNorm_{M,l}.
  * The positional transform inside the query/key maps is rotary (RoPE,
    rotate-half pairing (i, i + dh/2), angle t * theta^(-2i/dh), t 1-based)
    on the SWA query and key and on the cross-attention query. Memory keys
    are inputs that already carry their own transform.
  * Multi-head attention: head h uses columns [h*dh, (h+1)*dh), scores
    q.k / sqrt(dh), softmax, output projection applied after concatenation.
  * FFN is SwiGLU: W_down (silu(W_gate h) * (W_up h)).
  * Projections carry no bias; the merge gate carries b_g.
  * Memory group of layer l (0-based): floor(l * G / L_D).
  * Merge variants [RLT §2.5, text after eq. (2.11)]: a scalar gate is one
    gate value per token, sigmoid(w_g . [e; r] + b_g) with w_g a single row,
    shared by every channel; a low-rank W_s is the product U V (U [d, k],
    V [k, d]), applied as U (V r).
  * Sublayer orders [RLT §2.5, text after eq. (2.16)]: a block applies its
    SWA ("s"), cross-attention ("x") and FFN ("f") sublayers, each a pre-norm
    residual update with its own RMSNorm, in the order of a permutation
    string; "sxf" is eqs. (2.14)-(2.16). The SWA key/value of the current
    token are formed from the SWA sublayer's own input.
  * Top-p behaviour sampling [RLT §5.3]: temperature first, then top-k, then
    the nucleus: the shortest prefix of the (logit desc, id asc) order whose
    renormalised probability mass reaches p; mu renormalises over it.
  * Memory construction [RLT §2.2, eq. (2.2)]: one RMSNorm_E per group g
    (gain norm_e^g) feeds both maps; the key map is W_K^g followed by the
    same rotary transform as the decoder queries, at the entry's own
    position t, so cross-attention scores depend on the query and key
    positions only through their difference.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# elementwise building blocks
# ----------------------------------------------------------------------------

def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gain."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gain


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def silu(x: np.ndarray) -> np.ndarray:
    return x * sigmoid(x)


def rope_angles(t: int, dh: int, theta: float, dtype=np.float64) -> Tuple[np.ndarray, np.ndarray]:
    """cos/sin of t * theta^(-2i/dh), i = 0 .. dh/2-1 (computed in float64)."""
    i = np.arange(dh // 2, dtype=np.float64)
    ang = float(t) * theta ** (-2.0 * i / dh)
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x: np.ndarray, t: int, n_heads: int, dh: int, theta: float) -> np.ndarray:
    """Rotary transform at 1-based position t, applied per head (rotate-half)."""
    c, s = rope_angles(t, dh, theta, x.dtype)
    xh = x.reshape(x.shape[:-1] + (n_heads, dh))
    a, b = xh[..., : dh // 2], xh[..., dh // 2:]
    out = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    return out.reshape(x.shape)


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, n_heads: int, dh: int) -> np.ndarray:
    """Multi-head softmax attention of one query over n keys.

    q [d], keys/values [n, d] -> concatenated head outputs [d] (before the
    output projection). Per head: p = softmax(K_h q_h / sqrt(dh)), o_h = p V_h.
    """
    qh = q.reshape(n_heads, dh)
    kh = keys.reshape(keys.shape[0], n_heads, dh)
    vh = values.reshape(values.shape[0], n_heads, dh)
    out = np.empty((n_heads, dh), dtype=q.dtype)
    for h in range(n_heads):
        scores = kh[:, h, :] @ qh[h] / math.sqrt(dh)
        scores = scores - np.max(scores)
        p = np.exp(scores)
        p = p / np.sum(p)
        out[h] = p @ vh[:, h, :]
    return out.reshape(-1)


# ----------------------------------------------------------------------------
# configuration, parameters, state
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    L: int
    d: int
    H: int
    dh: int
    W: int
    G: int
    F: int
    V: int
    merge: str = "gated"       # "gated" [RLT §2.5 eqs. (2.9)-(2.11)] or "convex"
    alpha: float = 0.5
    eps: float = 1e-6
    rope_theta: float = 10000.0
    pos: str = "rope"          # "rope" or "none"
    gate: str = "vector"       # merge gate: "vector" [eq. (2.10)] or "scalar"
    ws_rank: int = 0           # 0: full W_s; k > 0: W_s = U V of rank k
    order: str = "sxf"         # sublayer order of a block

    def group_of(self, layer: int) -> int:
        return (layer * self.G) // self.L


@dataclass
class State:
    """Complete decoder state H_t = (s_t, C_t^D) [RLT §2.1] plus its position.

    ``hist[l]`` maps an absolute 1-based position j to the layer-l decoder
    (k_j, v_j) retained for the next update.
    """
    s: np.ndarray
    pos: int
    hist: List[Dict[int, Tuple[np.ndarray, np.ndarray]]]
    blocks: int = 0            # decoder block evaluations along this state's path

    def copy(self) -> "State":
        return State(self.s.copy(), self.pos, [dict(h) for h in self.hist], self.blocks)


@dataclass
class Memory:
    """Encoder memory of one sequence: per group g, keys/values [T, d] for
    positions 1..T [RLT §2.2, eq. (2.2)]. Row j-1 holds position j."""
    k: Sequence[np.ndarray]
    v: Sequence[np.ndarray]


def memory_entry(cfg: Config, e: np.ndarray, t: int, norm_e: np.ndarray, wk: np.ndarray,
                 wv: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """One memory entry of one group at 1-based position t [RLT §2.2, eq. (2.2)]:
    k_t = P_K(e_t, t) = RoPE(W_K RMSNorm_E(e_t), t), v_t = W_V RMSNorm_E(e_t)."""
    h = rms_norm(e, norm_e, cfg.eps)
    k = wk @ h
    if cfg.pos == "rope":
        k = rope(k, t, cfg.H, cfg.dh, cfg.rope_theta)
    return k, wv @ h


def build_memory(cfg: Config, E: np.ndarray, mw: Dict[str, np.ndarray], n: Optional[int] = None) -> Memory:
    """Memory of one sequence for positions 1..n from its encoder
    representations E [T, d] and the memory weights ``mw`` keyed
    "memory.{g}.norm_e" / ".wk" / ".wv" [RLT §2.2, eq. (2.2)]: every group,
    every position, one entry at a time (the token-parallel form computes
    the same values, each position being independent of the others)."""
    n = E.shape[0] if n is None else n
    ks, vs = [], []
    for g in range(cfg.G):
        k = np.empty((n, cfg.d))
        v = np.empty((n, cfg.d))
        for t in range(1, n + 1):
            k[t - 1], v[t - 1] = memory_entry(cfg, np.asarray(E[t - 1], dtype=np.float64), t,
                                              mw["memory.%d.norm_e" % g], mw["memory.%d.wk" % g],
                                              mw["memory.%d.wv" % g])
        ks.append(k)
        vs.append(v)
    return Memory(ks, vs)


def retained_positions(t: int, W: int) -> List[int]:
    """Positions kept in C_t^D after the update at t: max(1, t-W+2) .. t,
    empty for W = 1 [RLT §2.5, text after eq. (2.16)]."""
    if W == 1:
        return []
    return list(range(max(1, t - W + 2), t + 1))


def window_positions(t: int, W: int) -> List[int]:
    """Positions read by SWA at t: max(1, t-W+1) .. t [RLT §2.5, eq. (2.14)]."""
    return list(range(max(1, t - W + 1), t + 1))


def ring_slot(j: int, W: int) -> int:
    """Ring-buffer slot of retained position j (a layout convention of the
    GPU state, W-1 slots): (j - 1) mod (W - 1)."""
    return (j - 1) % (W - 1)


class Oracle:
    """Step-by-step decoder transition, readout and sampler.

    weights: natural-layout parameters keyed as in ``synth.weight_shapes``
    (already widened to float; bf16 inputs are widened exactly).
    """

    def __init__(self, cfg: Config, weights: Dict[str, np.ndarray], dtype=np.float64):
        self.cfg = cfg
        self.dtype = dtype
        self.w = {k: np.asarray(v, dtype=dtype) for k, v in weights.items()}

    # -- H_0 ------------------------------------------------------------
    def initial_state(self) -> State:
        """H_0 = (s_star, empty cache) [RLT §2.3, eq. (2.3)]."""
        return State(self.w["s_star"].copy(), 0, [dict() for _ in range(self.cfg.L)])

    # -- merge --------------------------------------------------------------
    def merge(self, e: np.ndarray, s_prev: np.ndarray) -> np.ndarray:
        """u_t = Merge(e_t, s_{t-1}) [RLT §2.3, eq. (2.4)].

        gated [RLT §2.5, eqs. (2.9)-(2.11)]:
            r = RMSNorm_s(s_{t-1}); g = sigmoid(W_g [e; r] + b_g);
            u = e + alpha * g * (W_s r)
        convex (alternative merge used by the tiny workload):
            g = sigmoid(W_g [e; s] + b); u = g * e + (1 - g) * s
        """
        c, w = self.cfg, self.w
        if c.merge == "gated":
            r = rms_norm(s_prev, w["merge.norm"], c.eps)
            g = self._gate(np.concatenate([e, r]))
            proj = w["merge.ws"] @ r if c.ws_rank == 0 else w["merge.ws_u"] @ (w["merge.ws_v"] @ r)
            return e + c.alpha * g * proj
        if c.merge == "convex":
            g = self._gate(np.concatenate([e, s_prev]))
            return g * e + (1.0 - g) * s_prev
        raise ValueError(c.merge)

    def _gate(self, x: np.ndarray):
        """sigmoid(W_g x + b_g): a vector [d], or one scalar for the scalar gate."""
        w = self.w
        if self.cfg.gate == "scalar":
            return float(sigmoid(np.reshape(w["merge.wg"], -1) @ x + float(np.reshape(w["merge.bg"], -1)[0])))
        return sigmoid(w["merge.wg"] @ x + w["merge.bg"])

    def _pos(self, x: np.ndarray, t: int) -> np.ndarray:
        c = self.cfg
        return rope(x, t, c.H, c.dh, c.rope_theta) if c.pos == "rope" else x

    # -- one decoder block ---------------------------------------------------
    def block(self, l: int, z: np.ndarray, t: int, hist: Dict[int, Tuple[np.ndarray, np.ndarray]],
              mem: Memory, trace: Optional[dict] = None) -> np.ndarray:
        """Decoder block l at position t: SWA, then cross-attention, then FFN
        [RLT §2.5, eqs. (2.12)-(2.16)], or the sublayers in the configured
        order. Updates ``hist`` (the layer's cache)."""
        if self.cfg.order != "sxf":
            for kind in self.cfg.order:
                if kind == "s":
                    z = self._swa(l, z, t, hist)
                elif kind == "x":
                    z = self._cross(l, z, t, mem)
                else:
                    z = self._ffn(l, z)
            return z
        c, w = self.cfg, self.w
        p = "layer.%d." % l
        # (2.12)-(2.13): current KV formed first, from the layer input
        h = rms_norm(z, w[p + "norm_s"], c.eps)
        q = self._pos(w[p + "wq"] @ h, t)
        k = self._pos(w[p + "wk"] @ h, t)
        v = w[p + "wv"] @ h
        # (2.14): window max(1, t-W+1) .. t; history from C_{t-1}^D
        win = window_positions(t, c.W)
        keys = np.stack([hist[j][0] for j in win[:-1]] + [k])
        vals = np.stack([hist[j][1] for j in win[:-1]] + [v])
        o = attend(q, keys, vals, c.H, c.dh)
        b = z + w[p + "wo"] @ o
        # cache update: keep max(1, t-W+2) .. t
        hist[t] = (k, v)
        keep = set(retained_positions(t, c.W))
        for j in list(hist.keys()):
            if j not in keep:
                del hist[j]
        # (2.15): cross-attention to the prefix M_{<=t} of group g(l)
        g = c.group_of(l)
        hm = rms_norm(b, w[p + "norm_m"], c.eps)
        qm = self._pos(w[p + "wqm"] @ hm, t)
        om = attend(qm, np.asarray(mem.k[g][:t], dtype=self.dtype),
                    np.asarray(mem.v[g][:t], dtype=self.dtype), c.H, c.dh)
        a = b + w[p + "wom"] @ om
        # (2.16): FFN on RMSNorm_{D,l}
        hd = rms_norm(a, w[p + "norm_d"], c.eps)
        z_out = a + w[p + "w_down"] @ (silu(w[p + "w_gate"] @ hd) * (w[p + "w_up"] @ hd))
        if trace is not None:
            trace.setdefault("q", []).append(q)
            trace.setdefault("k", []).append(k)
            trace.setdefault("v", []).append(v)
            trace.setdefault("o_swa", []).append(o)
            trace.setdefault("b", []).append(b)
            trace.setdefault("qm", []).append(qm)
            trace.setdefault("o_mem", []).append(om)
            trace.setdefault("a", []).append(a)
            trace.setdefault("z", []).append(z_out)
        return z_out

    # sublayers (each a pre-norm residual update) for the other orders
    def _swa(self, l: int, z: np.ndarray, t: int, hist) -> np.ndarray:
        c, w = self.cfg, self.w
        p = "layer.%d." % l
        h = rms_norm(z, w[p + "norm_s"], c.eps)
        q, k, v = self._pos(w[p + "wq"] @ h, t), self._pos(w[p + "wk"] @ h, t), w[p + "wv"] @ h
        win = window_positions(t, c.W)
        o = attend(q, np.stack([hist[j][0] for j in win[:-1]] + [k]),
                   np.stack([hist[j][1] for j in win[:-1]] + [v]), c.H, c.dh)
        hist[t] = (k, v)
        keep = set(retained_positions(t, c.W))
        for j in list(hist.keys()):
            if j not in keep:
                del hist[j]
        return z + w[p + "wo"] @ o

    def _cross(self, l: int, z: np.ndarray, t: int, mem: Memory) -> np.ndarray:
        c, w = self.cfg, self.w
        p = "layer.%d." % l
        g = c.group_of(l)
        qm = self._pos(w[p + "wqm"] @ rms_norm(z, w[p + "norm_m"], c.eps), t)
        om = attend(qm, np.asarray(mem.k[g][:t], dtype=self.dtype), np.asarray(mem.v[g][:t], dtype=self.dtype),
                    c.H, c.dh)
        return z + w[p + "wom"] @ om

    def _ffn(self, l: int, z: np.ndarray) -> np.ndarray:
        c, w = self.cfg, self.w
        p = "layer.%d." % l
        hd = rms_norm(z, w[p + "norm_d"], c.eps)
        return z + w[p + "w_down"] @ (silu(w[p + "w_gate"] @ hd) * (w[p + "w_up"] @ hd))

    # -- F_t --------------------------------------------------------------
    def transition(self, state: State, e: np.ndarray, mem: Memory,
                   trace: Optional[dict] = None) -> State:
        """H_t = F_t(H_{t-1}) = D(Merge(e_t, s_{t-1}); M_{<=t}, C_{t-1}^D, t)
        [RLT §2.3, eqs. (2.4)-(2.5)], t = state.pos + 1. Returns a new state;
        the argument is left unchanged."""
        c = self.cfg
        t = state.pos + 1
        for g in range(c.G):
            if len(mem.k[g]) < t:
                raise ValueError("memory holds %d < t = %d positions" % (len(mem.k[g]), t))
        new = state.copy()
        e = np.asarray(e, dtype=self.dtype)
        z = self.merge(e, state.s)
        if trace is not None:
            trace["u"] = z
        for l in range(c.L):
            z = self.block(l, z, t, new.hist[l], mem, trace)
        new.s = z
        new.pos = t
        new.blocks += c.L
        return new

    def run(self, state: State, E: np.ndarray, mem: Memory, n: int) -> Tuple[State, List[np.ndarray]]:
        """Apply n transitions (eq. (2.7)): E[i] is e at position state.pos+1+i.
        Returns the final state and s_t after each transition."""
        ss = []
        for i in range(n):
            state = self.transition(state, E[i], mem)
            ss.append(state.s)
        return state, ss

    # -- readout [RLT §2.3, eq. (2.6)] ------------------------------------------
    def logits(self, s: np.ndarray) -> np.ndarray:
        """W_o RMSNorm_o(s_t)."""
        return self.w["out.w"] @ rms_norm(np.asarray(s, dtype=self.dtype), self.w["out.norm"], self.cfg.eps)

    @staticmethod
    def log_softmax(z: np.ndarray) -> np.ndarray:
        m = np.max(z)
        return z - (m + np.log(np.sum(np.exp(z - m))))

    def log_prob(self, s: np.ndarray, token: int) -> float:
        """log p(x_{t+1} = token | x_{1:t}) read from s_t."""
        return float(self.log_softmax(self.logits(s))[token])


# ----------------------------------------------------------------------------
# behaviour distribution of a temperature / top-k sampler [RLT §5.3]
# ----------------------------------------------------------------------------

def topk_order(z: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest logits, ordered by (logit descending, id ascending)."""
    ids = np.lexsort((np.arange(z.shape[0]), -z.astype(np.float64)))
    return ids[:k]


def behaviour_logprobs(z: np.ndarray, tau: float, k: int, p: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """mu over the truncated support: temperature tau, top-k truncation,
    optional nucleus (top-p) truncation, renormalisation (all of them enter
    the behaviour probability, [RLT §5.3]). p outside (0, 1) means no
    nucleus.

    Returns (support ids in (logit desc, id asc) order, log mu of each)."""
    V = z.shape[0]
    k = V if (k <= 0 or k > V) else k
    ids = topk_order(z, k)
    zz = z[ids].astype(np.float64) / tau
    m = np.max(zz)
    lse = m + np.log(np.sum(np.exp(zz - m)))
    if 0.0 < p < 1.0:
        mass = np.cumsum(np.exp(zz - lse))
        n = int(np.searchsorted(mass, p, side="left")) + 1   # shortest prefix with mass >= p
        n = min(n, len(ids))
        ids, zz = ids[:n], zz[:n]
        lse = m + np.log(np.sum(np.exp(zz - m)))
    return ids, zz - lse


def sample(z: np.ndarray, tau: float, k: int, u: float, p: float = 1.0) -> Tuple[int, float]:
    """Inverse-CDF draw from mu with a given uniform u in [0, 1): the first
    support id (in support order) whose cumulative unnormalised weight
    exceeds u times the total. Returns (token, log mu(token))."""
    ids, lmu = behaviour_logprobs(z, tau, k, p)
    w = np.exp(lmu - np.max(lmu))
    cum = np.cumsum(w)
    i = int(np.searchsorted(cum, u * cum[-1], side="right"))
    i = min(i, len(ids) - 1)
    return int(ids[i]), float(lmu[i])


def importance_ratio(logp: float, logmu: float) -> float:
    """r_i = exp(log p_Theta(y_i|.) - log mu(y_i|.)) [RLT §5.3, eq. (5.5)]."""
    return math.exp(logp - logmu)


def trajectory_log_ratio(logp: Sequence[float], logmu: Sequence[float]) -> float:
    """log of the trajectory importance weight prod_i r_i over a response
    [RLT §5.3]: sum_i (log p_i - log mu_i), in response order."""
    acc = 0.0
    for a, b in zip(logp, logmu):
        acc += float(a) - float(b)
    return acc


# ----------------------------------------------------------------------------
# batch helpers (sequences are independent: each keeps its own state [RLT §4.1])
# ----------------------------------------------------------------------------

def replay(orc: Oracle, E: np.ndarray, mem: Memory, tokens: np.ndarray, length: int, split: int):
    """Current-policy replay of one sequence from H_0 [RLT App. A.4]:
    consume x_1 .. x_{len-1}; after consuming x_t (t >= split) read
    log p(x_{t+1}) from s_t before consuming x_{t+1}. x_len is left pending.

    Returns (final state, {t: log p(x_{t+1} | x_{1:t})}, [s_1 .. s_{len-1}])."""
    st = orc.initial_state()
    logp = {}
    ss = []
    for t in range(1, length):
        st = orc.transition(st, E[t - 1], mem)
        ss.append(st.s)
        if t >= split:
            logp[t] = orc.log_prob(st.s, int(tokens[t]))
    return st, logp, ss


def state_from_ring(cfg: Config, s: np.ndarray, pos: int, ring_k: np.ndarray, ring_v: np.ndarray,
                    dtype=np.float64) -> State:
    """Build an oracle state at position ``pos`` from ring-buffer contents
    ring_k/ring_v [L, W-1, d] laid out with slot(j) = (j-1) mod (W-1)."""
    hist = []
    for l in range(cfg.L):
        h = {}
        for j in retained_positions(pos, cfg.W) if pos > 0 else []:
            sl = ring_slot(j, cfg.W)
            h[j] = (np.asarray(ring_k[l, sl], dtype=dtype), np.asarray(ring_v[l, sl], dtype=dtype))
        hist.append(h)
    return State(np.asarray(s, dtype=dtype).copy(), pos, hist)


def state_to_ring(cfg: Config, st: State) -> Tuple[np.ndarray, np.ndarray]:
    """Inverse of state_from_ring: [L, W-1, d] arrays, NaN in unused slots."""
    n = max(cfg.W - 1, 0)
    rk = np.full((cfg.L, n, cfg.d), np.nan)
    rv = np.full((cfg.L, n, cfg.d), np.nan)
    for l in range(cfg.L):
        for j, (k, v) in st.hist[l].items():
            rk[l, ring_slot(j, cfg.W)] = k
            rv[l, ring_slot(j, cfg.W)] = v
    return rk, rv
