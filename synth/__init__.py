"""Seeded synthetic inputs for the recurrent decoder transition.

This module is shared by the CPU oracle side (tests) and the GPU side (tests,
bench). It holds the workload presets (shapes, dtypes, value recipes) and a
counter-based generator (``synth.c``); it holds none of the transition's
arithmetic. Every tensor is addressed by (seed, stream name, flat index), so
any sub-block (one sequence's memory, one layer's weight) can be regenerated
on its own and matches the corresponding slice of the full tensor bit for bit.

Value recipe (a stated stand-in for the Gaussian draws the workloads name):
``normal`` = Irwin-Hall(4) sum of the four 16-bit lanes of one SplitMix64
draw, centred and scaled to unit variance, times sigma (+ offset), rounded
once to fp32 and, for bf16 tensors, once more to bf16 (nearest even).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the generator with gcc (host code only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64 = ctypes.c_uint64, ctypes.c_int64
        lib.synth_normal.argtypes = [u64, u64, u64, u64, ctypes.c_float, ctypes.c_float,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        lib.synth_normal.restype = None
        lib.synth_uniform_int.argtypes = [u64, u64, u64, u64, i64, i64, ctypes.c_void_p]
        lib.synth_uniform_int.restype = None
        lib.synth_uniform01.argtypes = [u64, u64, u64, u64, ctypes.c_void_p]
        lib.synth_uniform01.restype = None
        _lib = lib
    return _lib


def stream_id(name: str) -> int:
    """FNV-1a 64-bit hash of a tensor name: its generator stream."""
    h = 0xCBF29CE484222325
    for b in name.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def _threads() -> int:
    try:
        return max(1, min(16, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))))
    except ValueError:
        return 1


def normal(seed: int, name: str, shape, sigma: float = 1.0, offset: float = 0.0,
           dtype: str = "f32", start: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Fill ``shape`` with the stream's values [start, start+size).

    dtype "f32" -> float32 array; "bf16" -> uint16 array of bf16 bit patterns.
    """
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    if out is None:
        out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    assert out.flags["C_CONTIGUOUS"] and out.size == n
    kind = 0 if dtype == "f32" else 1
    assert out.dtype == (np.float32 if kind == 0 else np.uint16)
    lib.synth_normal(seed, stream_id(name), start, n, float(sigma), float(offset), kind,
                     out.ctypes.data, _threads())
    return out


def uniform_int(seed: int, name: str, n: int, lo: int, hi: int, start: int = 0) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.int32)
    lib.synth_uniform_int(seed, stream_id(name), start, n, lo, hi, out.ctypes.data)
    return out


def uniform01(seed: int, name: str, n: int, start: int = 0) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.float32)
    lib.synth_uniform01(seed, stream_id(name), start, n, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Workload presets
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    L: int            # decoder depth L_D
    d: int            # residual width
    H: int            # heads
    dh: int           # head width, d = H * dh
    W: int            # SWA window (includes the current token)
    G: int            # encoder-memory groups: 1 (shared) or L (per layer)
    F: int            # SwiGLU hidden width
    V: int            # vocabulary
    B: int            # sequences
    T: int            # tokens per sequence (max length for ragged)
    dtype: str        # "f32" or "bf16": weights, KV ring, memory, e
    merge: str        # "gated" (paper eqs 2.9-2.11) or "convex"
    w_std: float      # projection weight std
    alpha: float = 0.5
    eps: float = 1e-6
    rope_theta: float = 10000.0
    pos: str = "rope"
    seed: int = 1
    ragged: bool = False
    len_lo: int = 0
    len_hi: int = 0
    split_lo: int = 16
    temperature: float = 1.0
    top_k: int = 0
    gain_std: float = 0.1  # norm gains are 1 + gain_std * normal
    gate: str = "vector"   # merge gate: "vector" (eq 2.10) or "scalar"
    ws_rank: int = 0       # 0: full W_s; k > 0: W_s = U V of rank k
    order: str = "sxf"     # sublayer order of a block
    top_p: float = 1.0     # nucleus of the behaviour sampler (1 = none)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def group_of(self, layer: int) -> int:
        """0-based memory group read by 0-based decoder layer (contiguous blocks)."""
        return (layer * self.G) // self.L


TINY = Workload("tiny_fp32", L=2, d=64, H=4, dh=16, W=4, G=1, F=128, V=256, B=1, T=32,
                dtype="f32", merge="convex", w_std=0.02, seed=1)
SMALL = Workload("small_batched", L=4, d=256, H=8, dh=32, W=16, G=4, F=704, V=4096, B=16, T=256,
                 dtype="bf16", merge="gated", w_std=0.02, seed=2)
MID = Workload("mid", L=12, d=1024, H=16, dh=64, W=128, G=1, F=2816, V=32000, B=64, T=2048,
               dtype="bf16", merge="gated", w_std=0.02, seed=3)
REF = Workload("reference_depth", L=48, d=2048, H=16, dh=128, W=256, G=1, F=5504, V=32000, B=128,
               T=4096, dtype="bf16", merge="gated", w_std=0.02 / (2 * 48) ** 0.5, seed=4)
RAGGED = Workload("ragged_rl_replay", L=24, d=1536, H=12, dh=128, W=512, G=24, F=4096, V=32000,
                  B=256, T=8192, dtype="bf16", merge="gated", w_std=0.02, seed=5, ragged=True,
                  len_lo=64, len_hi=8192, split_lo=16, temperature=0.7, top_k=50)

PRESETS = {w.name: w for w in (TINY, SMALL, MID, REF, RAGGED)}


def weight_shapes(wl: Workload) -> Dict[str, tuple]:
    """Natural ([out, in]) shapes of every parameter, keyed by name."""
    d, F, V = wl.d, wl.F, wl.V
    gw = 1 if wl.gate == "scalar" else d
    shapes = {"s_star": (d,), "merge.wg": (gw, 2 * d), "merge.bg": (gw,)}
    if wl.merge == "gated":
        shapes["merge.norm"] = (d,)
        if wl.ws_rank:
            shapes["merge.ws_u"] = (d, wl.ws_rank)
            shapes["merge.ws_v"] = (wl.ws_rank, d)
        else:
            shapes["merge.ws"] = (d, d)
    for l in range(wl.L):
        p = "layer.%d." % l
        shapes.update({p + "norm_s": (d,), p + "wq": (d, d), p + "wk": (d, d), p + "wv": (d, d),
                       p + "wo": (d, d), p + "norm_m": (d,), p + "wqm": (d, d), p + "wom": (d, d),
                       p + "norm_d": (d,), p + "w_gate": (F, d), p + "w_up": (F, d),
                       p + "w_down": (d, F)})
    shapes["out.norm"] = (d,)
    shapes["out.w"] = (V, d)
    return shapes


def is_matrix(name: str) -> bool:
    return name.split(".")[-1] in ("wg", "ws", "ws_u", "ws_v", "wq", "wk", "wv", "wo", "wqm", "wom",
                                   "w_gate", "w_up", "w_down", "w")


def make_weight(wl: Workload, name: str, shape) -> np.ndarray:
    """One parameter. Matrices in the workload dtype (bf16 -> uint16 bits), vectors fp32."""
    if is_matrix(name):
        return normal(wl.seed, name, shape, sigma=wl.w_std, dtype=wl.dtype)
    if name == "s_star":
        return normal(wl.seed, name, shape, sigma=1.0)
    if name == "merge.bg":
        return normal(wl.seed, name, shape, sigma=0.02)
    # normalization gains
    return normal(wl.seed, name, shape, sigma=wl.gain_std, offset=1.0)


def make_weights(wl: Workload) -> Dict[str, np.ndarray]:
    return {n: make_weight(wl, n, s) for n, s in weight_shapes(wl).items()}


def memory_weight_shapes(wl: Workload) -> Dict[str, tuple]:
    """Parameters of the encoder-memory maps, per group g: the RMSNorm_E gain
    and the key / value projections ([out, in])."""
    d = wl.d
    shapes = {}
    for g in range(wl.G):
        shapes.update({"memory.%d.norm_e" % g: (d,), "memory.%d.wk" % g: (d, d), "memory.%d.wv" % g: (d, d)})
    return shapes


def make_memory_weights(wl: Workload) -> Dict[str, np.ndarray]:
    """Memory-map weights: matrices N(0, w_std) in the workload dtype, gains
    1 + gain_std * N(0, 1) in fp32 (same recipe as the decoder weights)."""
    return {n: make_weight(wl, n, s) for n, s in memory_weight_shapes(wl).items()}


def make_e(wl: Workload, b0: int = 0, nb: Optional[int] = None, T: Optional[int] = None) -> np.ndarray:
    """Encoder representations e[b][t][d] for sequences b0..b0+nb-1, positions 1..T.

    Element (b, t, c) is index (b * wl.T + t) * d + c of stream "e": any
    sub-block is the same slice of the full tensor.
    """
    nb = wl.B if nb is None else nb
    T = wl.T if T is None else T
    out = np.empty((nb, T, wl.d), dtype=np.float32 if wl.dtype == "f32" else np.uint16)
    for i in range(nb):
        normal(wl.seed, "e", (T, wl.d), dtype=wl.dtype, start=(b0 + i) * wl.T * wl.d, out=out[i])
    return out


def make_memory(wl: Workload, which: str, g: int, b0: int = 0, nb: Optional[int] = None,
                T: Optional[int] = None) -> np.ndarray:
    """Encoder memory keys ("k") or values ("v") of group g: [nb][T][d]."""
    nb = wl.B if nb is None else nb
    T = wl.T if T is None else T
    out = np.empty((nb, T, wl.d), dtype=np.float32 if wl.dtype == "f32" else np.uint16)
    name = "mem_%s.%d" % (which, g)
    for i in range(nb):
        normal(wl.seed, name, (T, wl.d), dtype=wl.dtype, start=(b0 + i) * wl.T * wl.d, out=out[i])
    return out


def make_lengths(wl: Workload):
    """Ragged lengths (tokens incl. BOS) and first scored positions."""
    if not wl.ragged:
        L = np.full(wl.B, wl.T, dtype=np.int32)
        return L, np.ones(wl.B, dtype=np.int32)
    lens = uniform_int(wl.seed, "len", wl.B, wl.len_lo, wl.len_hi)
    splits = np.empty(wl.B, dtype=np.int32)
    for b in range(wl.B):
        splits[b] = uniform_int(wl.seed, "split", 1, wl.split_lo, int(lens[b]) - 1, start=b)[0]
    return lens, splits


def make_tokens(wl: Workload, b0: int = 0, nb: Optional[int] = None, T: Optional[int] = None) -> np.ndarray:
    """Token ids x_1..x_T per sequence (x_1 = BOS = 0)."""
    nb = wl.B if nb is None else nb
    T = wl.T if T is None else T
    out = np.empty((nb, T), dtype=np.int32)
    for i in range(nb):
        out[i] = uniform_int(wl.seed, "tokens", T, 0, wl.V - 1, start=(b0 + i) * wl.T)
        out[i, 0] = 0
    return out


def make_ring_prefill(wl: Workload, which: str, layer: int, b0: int, nb: int) -> np.ndarray:
    """Synthetic SWA history (for benchmarks / sampled parity from a pre-filled
    state): values for ring slots of layer `layer`, rows b0.., [nb][W-1][d]."""
    n = max(wl.W - 1, 0)
    out = np.empty((nb, n, wl.d), dtype=np.float32 if wl.dtype == "f32" else np.uint16)
    name = "ring_%s.%d" % (which, layer)
    for i in range(nb):
        normal(wl.seed, name, (n, wl.d), sigma=1.0, dtype=wl.dtype,
               start=(b0 + i) * n * wl.d, out=out[i])
    return out
