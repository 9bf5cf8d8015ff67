"""Shared test helpers: build oracle inputs from the seeded workload presets.

Only the seeded generator (``synth``) and the oracle are used here; nothing in
this file touches the GPU library.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

import synth
from oracle import Config, Memory, Oracle


def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 -> float64, exactly."""
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def oracle_config(wl: synth.Workload, **over) -> Config:
    kw = dict(L=wl.L, d=wl.d, H=wl.H, dh=wl.dh, W=wl.W, G=wl.G, F=wl.F, V=wl.V, merge=wl.merge,
              alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos, gate=wl.gate,
              ws_rank=wl.ws_rank, order=wl.order)
    kw.update(over)
    return Config(**kw)


def oracle_weights(raw: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    return {k: widen(v) for k, v in raw.items()}


def make_oracle(wl: synth.Workload, raw: Optional[Dict[str, np.ndarray]] = None, dtype=np.float64,
                **over) -> Oracle:
    raw = synth.make_weights(wl) if raw is None else raw
    return Oracle(oracle_config(wl, **over), oracle_weights(raw), dtype=dtype)


def memory_of(wl: synth.Workload, b: int, T: Optional[int] = None) -> Memory:
    """Memory of sequence b, all groups, positions 1..T (float64)."""
    ks = [widen(synth.make_memory(wl, "k", g, b0=b, nb=1, T=T)[0]) for g in range(wl.G)]
    vs = [widen(synth.make_memory(wl, "v", g, b0=b, nb=1, T=T)[0]) for g in range(wl.G)]
    return Memory(ks, vs)


def e_of(wl: synth.Workload, b: int, T: Optional[int] = None) -> np.ndarray:
    return widen(synth.make_e(wl, b0=b, nb=1, T=T)[0])


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))
