"""GPU-side test plumbing: build the library context from a workload preset
and run sequences through the C ABI. Inputs come from ``synth`` only; the
oracle side of each comparison lives in the tests themselves."""
from __future__ import annotations

import os
import sys
from typing import Dict, Optional

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from stateful_sequence_model_amd import _abi
    _abi.lib()  # raises loudly when the HIP library is missing


def model_config(wl: synth.Workload, **over):
    from stateful_sequence_model_amd import ModelConfig
    kw = dict(L=wl.L, d=wl.d, H=wl.H, dh=wl.dh, W=wl.W, G=wl.G, F=wl.F, V=wl.V, dtype=wl.dtype,
              merge=wl.merge, alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos, gate=wl.gate,
              ws_rank=wl.ws_rank, order=wl.order)
    kw.update(over)
    return ModelConfig(**kw)


class GpuRun:
    """A context, a state of B rows and device copies of e / memory."""

    def __init__(self, wl: synth.Workload, raw: Optional[Dict[str, np.ndarray]] = None, B: Optional[int] = None,
                 T: Optional[int] = None, max_rows: Optional[int] = None, b0: int = 0,
                 launch: Optional[Dict[str, int]] = None, **over):
        from stateful_sequence_model_amd import Decoder, DecoderState, to_device
        self.wl = wl
        self.B = wl.B if B is None else B
        self.T = wl.T if T is None else T
        self.raw = synth.make_weights(wl) if raw is None else raw
        self.cfg = model_config(wl, **over)
        self.dec = Decoder(self.cfg, self.raw, max_rows=max_rows or max(self.B, 1), max_ctx=self.T, launch=launch)
        self.st = DecoderState(self.cfg, self.B)
        self.E = synth.make_e(wl, b0, self.B, self.T)
        self.mk = np.stack([synth.make_memory(wl, "k", g, b0, self.B, self.T) for g in range(wl.G)])
        self.mv = np.stack([synth.make_memory(wl, "v", g, b0, self.B, self.T) for g in range(wl.G)])
        self.Ed = to_device(self.E, self.cfg.dtype)
        self.mkd = to_device(self.mk, self.cfg.dtype)
        self.mvd = to_device(self.mv, self.cfg.dtype)
        self.mem_len = torch.full((self.B,), self.T, dtype=torch.int32, device="cuda")
        self.mem = Decoder.memory(self.mkd, self.mvd, self.mem_len)

    def rows(self, idx=None):
        idx = range(self.B) if idx is None else idx
        return torch.tensor(list(idx), dtype=torch.int32, device="cuda")

    def init(self, idx=None, poison=False):
        self.dec.init_state(self.st, self.rows(idx), poison=poison)

    def step(self, idx, t: int, **kw):
        """One transition for rows idx (each at position t), returns the code."""
        rows = self.rows(idx)
        e = self.Ed[torch.tensor(list(idx), device="cuda"), t - 1].contiguous()
        return self.dec.step(self.st, rows, e, self.mem, **kw)

    def run(self, nsteps: int, idx=None, **kw):
        """nsteps transitions of rows idx from their current state; returns
        s [nsteps, n, d] and logits [nsteps, n, V] as float64 numpy."""
        idx = list(range(self.B)) if idx is None else list(idx)
        n = len(idx)
        S = np.empty((nsteps, n, self.wl.d))
        Z = np.empty((nsteps, n, self.wl.V))
        s_out = torch.empty((n, self.wl.d), device="cuda")
        logits = torch.empty((n, self.wl.V), device="cuda")
        t0 = int(self.st.pos[idx[0]].item())
        for i in range(nsteps):
            rc = self.step(idx, t0 + i + 1, s_out=s_out, logits=logits, **kw)
            assert rc == 0, "decoder step returned %d" % rc
            S[i] = s_out.double().cpu().numpy()
            Z[i] = logits.double().cpu().numpy()
        torch.cuda.synchronize()
        return S, Z


def widen(a):
    from tests.helpers import widen as w
    return w(a)
