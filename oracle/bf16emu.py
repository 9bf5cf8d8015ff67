"""Rounding-emulation variant of the CPU oracle (a DIAGNOSTIC).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it; it shares
no code with the GPU path.

The plain oracle (``rlt_oracle.Oracle``) is the definition of the transition
("Recurrent Looped Transformer" §2.3 eqs. (2.4)-(2.6), §2.5 eqs.
(2.9)-(2.16)) in float64 on the given (bf16-valued) weights and inputs. The
bf16 mode of the GPU library additionally rounds at fixed points of the
computation (the rounding contract, a convention of this implementation
that the report leaves open):

  * every matrix-product input ("act"): the merge input [e; r] with
    r = RMSNorm_s(s_{t-1}) (convex merge: [e; s]), the low-rank intermediate
    V r, the attention outputs before their output projections, the SwiGLU
    product silu(W_gate h) * (W_up h). The bf16 products of the operand-order
    path take it as two bf16 terms, x rounded and then the remainder rounded
    (``two_term``); the other bf16 tiles as one rounded term (``bf16_round``);
  * the normalised inputs of the products that follow an RMSNorm are carried
    as act(z * gain) and the factor 1 / sqrt(mean(z^2) + eps) multiplies the
    product's result (RMSNorm(z) W^T = rstd * ((z * gain) W^T));
  * the SWA key and value of the current token when they are stored ("kv"),
    always one bf16 rounding (the cache is bf16).

Everything else (accumulation, softmax, residual stream, the state s_t)
stays unrounded, here in float64. ``RoundingOracle`` applies exactly those
roundings; with identities for act and kv it is the plain oracle rearranged
(pinned in the tests to 1e-12). Comparing the GPU with it separates what the
rounding contract itself does (for example an argmax flipped by a near-tie)
from what the kernels add.
"""
from __future__ import annotations

from typing import Callable, Dict, Optional

import numpy as np

from .rlt_oracle import Config, Memory, Oracle, attend, retained_positions, silu, window_positions


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16, ties to even, through float32 (the GPU
    rounds float32 values): float64 -> float32 (nearest) -> keep the upper 16
    bits of the float32 pattern, rounded to nearest with ties to even.
    Returns float64. Finite inputs only."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def two_term(x: np.ndarray) -> np.ndarray:
    """The value two bf16 terms carry: hi = x rounded, lo = (x - hi) rounded,
    hi + lo (about 16 significant bits of x)."""
    x = np.asarray(x, dtype=np.float64)
    hi = bf16_round(x)
    return hi + bf16_round(x - hi)


class RoundingOracle(Oracle):
    """The transition with the bf16 rounding contract applied (float64
    elsewhere). ``act`` maps a matrix-product input to the value the product
    sees, ``kv`` a produced SWA key or value to its stored value."""

    def __init__(self, cfg: Config, weights: Dict[str, np.ndarray],
                 act: Callable[[np.ndarray], np.ndarray] = two_term,
                 kv: Callable[[np.ndarray], np.ndarray] = bf16_round):
        super().__init__(cfg, weights, dtype=np.float64)
        self.rnd = act
        self.kv = kv

    # rstd * (W @ rnd(x * gain)) == W @ RMSNorm(x) before rounding
    def _rstd(self, x: np.ndarray) -> float:
        return 1.0 / np.sqrt(np.mean(x * x) + self.cfg.eps)

    def _normed(self, W: np.ndarray, x: np.ndarray, gain: np.ndarray) -> np.ndarray:
        return self._rstd(x) * (W @ self.rnd(x * gain))

    def merge(self, e: np.ndarray, s_prev: np.ndarray) -> np.ndarray:
        """Eqs. (2.9)-(2.11) with r (or s, convex) rounded as a product input."""
        c, w = self.cfg, self.w
        if c.merge == "gated":
            r = self.rnd(s_prev * self._rstd(s_prev) * w["merge.norm"])
            g = self._gate(np.concatenate([e, r]))
            if c.ws_rank == 0:
                proj = w["merge.ws"] @ r
            else:
                proj = w["merge.ws_u"] @ self.rnd(w["merge.ws_v"] @ r)
            return e + c.alpha * g * proj
        if c.merge == "convex":
            g = self._gate(np.concatenate([e, self.rnd(s_prev)]))
            return g * e + (1.0 - g) * s_prev
        raise ValueError(c.merge)

    def block(self, l: int, z: np.ndarray, t: int, hist, mem: Memory, trace: Optional[dict] = None) -> np.ndarray:
        for kind in self.cfg.order:
            if kind == "s":
                z = self._swa(l, z, t, hist)
            elif kind == "x":
                z = self._cross(l, z, t, mem)
            else:
                z = self._ffn(l, z)
        return z

    def _swa(self, l: int, z: np.ndarray, t: int, hist) -> np.ndarray:
        c, w = self.cfg, self.w
        p = "layer.%d." % l
        gain = w[p + "norm_s"]
        q = self._pos(self._normed(w[p + "wq"], z, gain), t)
        k = self.kv(self._pos(self._normed(w[p + "wk"], z, gain), t))
        v = self.kv(self._normed(w[p + "wv"], z, gain))
        win = window_positions(t, c.W)
        o = attend(q, np.stack([hist[j][0] for j in win[:-1]] + [k]),
                   np.stack([hist[j][1] for j in win[:-1]] + [v]), c.H, c.dh)
        hist[t] = (k, v)
        keep = set(retained_positions(t, c.W))
        for j in list(hist.keys()):
            if j not in keep:
                del hist[j]
        return z + w[p + "wo"] @ self.rnd(o)

    def _cross(self, l: int, z: np.ndarray, t: int, mem: Memory) -> np.ndarray:
        c, w = self.cfg, self.w
        p = "layer.%d." % l
        g = c.group_of(l)
        qm = self._pos(self._normed(w[p + "wqm"], z, w[p + "norm_m"]), t)
        om = attend(qm, np.asarray(mem.k[g][:t], dtype=np.float64), np.asarray(mem.v[g][:t], dtype=np.float64),
                    c.H, c.dh)
        return z + w[p + "wom"] @ self.rnd(om)

    def _ffn(self, l: int, z: np.ndarray) -> np.ndarray:
        w = self.w
        p = "layer.%d." % l
        gain = w[p + "norm_d"]
        act = silu(self._normed(w[p + "w_gate"], z, gain)) * self._normed(w[p + "w_up"], z, gain)
        return z + w[p + "w_down"] @ self.rnd(act)

    def logits(self, s: np.ndarray) -> np.ndarray:
        """W_o RMSNorm_o(s_t) with the normalised input rounded (eq. (2.6))."""
        s = np.asarray(s, dtype=np.float64)
        return self._normed(self.w["out.w"], s, self.w["out.norm"])
