"""Device-memory plumbing around the C ABI.

PyTorch provides device buffers and the stream handle; every step of the
decoder transition runs in ``librlt.so``. Nothing here computes any part of
the method.

Parameter names (natural [out, in] layout):
  s_star [d]; merge.norm [d] (gated); merge.wg [d, 2d]; merge.bg [d];
  merge.ws [d, d] (gated); layer.{l}.{norm_s, wq, wk, wv, wo, norm_m, wqm, wom,
  norm_d, w_gate, w_up, w_down}; out.norm [d]; out.w [V, d].
Matrices are float32 (dtype "f32") or bfloat16 ("bf16"); vectors float32.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import _abi as A

_MATRICES = ("wq", "wk", "wv", "wo", "wqm", "wom", "w_gate", "w_up", "w_down")
_LAYER_VECS = ("norm_s", "norm_m", "norm_d")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def to_device(a, dtype: str, device="cuda") -> torch.Tensor:
    """numpy (float32, or uint16 bf16 bit patterns) or tensor -> device tensor."""
    if isinstance(a, torch.Tensor):
        return a.to(device)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to(device)
    raise TypeError("unsupported array dtype %s" % a.dtype)


def current_stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclass
class ModelConfig:
    L: int
    d: int
    H: int
    dh: int
    W: int
    G: int
    F: int
    V: int
    dtype: str = "bf16"
    merge: str = "gated"
    alpha: float = 0.5
    eps: float = 1e-6
    rope_theta: float = 10000.0
    pos: str = "rope"
    version: int = 1
    gate: str = "vector"     # merge gate: "vector" or "scalar"
    ws_rank: int = 0         # 0: full W_s; k: W_s = U V (merge.ws_u [d, k], merge.ws_v [k, d])
    order: str = "sxf"       # sublayer order of a block (permutation of s, x, f)

    def to_c(self) -> A.rlt_config:
        return A.rlt_config(self.L, self.d, self.H, self.dh, self.W, self.G, self.F, self.V,
                            A.RLT_MERGE_GATED if self.merge == "gated" else A.RLT_MERGE_CONVEX,
                            A.RLT_POS_ROPE if self.pos == "rope" else A.RLT_POS_NONE,
                            A.RLT_BF16 if self.dtype == "bf16" else A.RLT_F32,
                            self.alpha, self.eps, self.rope_theta, self.version,
                            A.RLT_GATE_SCALAR if self.gate == "scalar" else A.RLT_GATE_VECTOR, self.ws_rank,
                            A.ORDERS.index(self.order))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


class DecoderState:
    """Device buffers of B_cap rows: s, SWA ring, pos, pending."""

    def __init__(self, cfg: ModelConfig, B_cap: int, device="cuda"):
        self.cfg = cfg
        self.B_cap = B_cap
        sizes = A.rlt_state_layout(cfg.to_c(), B_cap)
        es = 2 if cfg.dtype == "bf16" else 4
        ring_elems = sizes[1] // es
        self.s = torch.empty((B_cap, cfg.d), dtype=torch.float32, device=device)
        self.ring_k = torch.empty(max(ring_elems, 1), dtype=cfg.torch_dtype, device=device)
        self.ring_v = torch.empty(max(ring_elems, 1), dtype=cfg.torch_dtype, device=device)
        self.pos = torch.zeros(B_cap, dtype=torch.int32, device=device)
        self.pending = torch.full((B_cap,), -1, dtype=torch.int32, device=device)
        self.version = cfg.version

    def c(self) -> A.rlt_state:
        return A.rlt_state(self.s.data_ptr(), self.ring_k.data_ptr(), self.ring_v.data_ptr(),
                           self.pos.data_ptr(), self.pending.data_ptr(), self.B_cap, self.version)

    def ring(self, which: str) -> torch.Tensor:
        """View [L, B_cap, W-1, d] of the keys ("k") or values ("v")."""
        c = self.cfg
        t = self.ring_k if which == "k" else self.ring_v
        return t[: c.L * self.B_cap * (c.W - 1) * c.d].view(c.L, self.B_cap, c.W - 1, c.d)


class Decoder:
    """A context (``rlt_create``) over device copies of the parameters."""

    def __init__(self, cfg: ModelConfig, params: Dict[str, object], max_rows: int, max_ctx: int,
                 device="cuda", launch: Optional[Dict[str, int]] = None):
        """launch: optional ``rlt_dbg_launch`` fields (tests and tuning sweeps)."""
        self.cfg = cfg
        self.device = device
        self.params = {}
        for k, v in params.items():
            self.params[k] = to_device(v, cfg.dtype, device).contiguous()
        p = self.params
        L = cfg.L
        self._arrays = {}
        for name in _MATRICES + _LAYER_VECS:
            arr = (A.P * L)(*[p["layer.%d.%s" % (l, name)].data_ptr() for l in range(L)])
            self._arrays[name] = arr
        gated = cfg.merge == "gated"
        w = A.rlt_weights()
        w.s_star = p["s_star"].data_ptr()
        w.merge_norm = p["merge.norm"].data_ptr() if gated else None
        w.merge_wg = p["merge.wg"].data_ptr()
        w.merge_bg = p["merge.bg"].data_ptr()
        w.merge_ws = p["merge.ws"].data_ptr() if gated and not cfg.ws_rank else None
        w.merge_ws_u = p["merge.ws_u"].data_ptr() if gated and cfg.ws_rank else None
        w.merge_ws_v = p["merge.ws_v"].data_ptr() if gated and cfg.ws_rank else None
        for name, arr in self._arrays.items():
            setattr(w, name, C.cast(arr, C.POINTER(A.P)))
        w.out_norm = p["out.norm"].data_ptr()
        w.w_out = p["out.w"].data_ptr()
        self._w = w
        self._cfg_c = cfg.to_c()
        self.max_rows, self.max_ctx = max_rows, max_ctx
        if launch:
            self.ctx = A.rlt_dbg_create(self._cfg_c, w, max_rows, max_ctx, A.rlt_dbg_launch(**launch))
        else:
            self.ctx = A.rlt_create(self._cfg_c, w, max_rows, max_ctx)

    def close(self):
        if getattr(self, "ctx", None):
            A.rlt_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- entry points --------------------------------------------------------
    def init_state(self, st: DecoderState, rows: torch.Tensor, poison: bool = False, stream=None):
        stc = st.c()
        A.check(A.rlt_init_state(self.ctx, stc, rows.data_ptr(), rows.numel(),
                                 A.RLT_INIT_POISON if poison else 0,
                                 current_stream() if stream is None else stream), "rlt_init_state")

    @staticmethod
    def memory(k: torch.Tensor, v: torch.Tensor, mem_len: torch.Tensor) -> A.rlt_memory:
        """k, v shaped [G, B, T, d] (contiguous); mem_len int32 [B]. The
        returned struct holds raw device pointers: the caller keeps the three
        tensors alive while it is in use."""
        G, B, T, d = k.shape
        return A.rlt_memory(k.data_ptr(), v.data_ptr(), B * T * d, T * d, d, mem_len.data_ptr())

    def step(self, st: DecoderState, rows: torch.Tensor, e: torch.Tensor, mem: A.rlt_memory, *,
             consume_tok=None, s_out=None, logits=None, argmax=None, score_tok=None, logp=None,
             uniform=None, temperature=1.0, top_k=0, top_p=1.0, sample_tok=None, sample_logmu=None,
             z_trace=None, graph=False, defer=False, noalloc=False, stream=None) -> int:
        """One transition of the listed rows (rlt_decoder_step, or with
        noalloc=True rlt_decoder_step_noalloc, which allocates nothing)."""
        io = A.rlt_step_io()
        io.n = rows.numel()
        io.rows = rows.data_ptr()
        io.e = e.data_ptr()
        io.mem = mem
        io.consume_tok = _ptr(consume_tok)
        io.s_out = _ptr(s_out)
        io.logits = _ptr(logits)
        io.argmax = _ptr(argmax)
        io.score_tok = _ptr(score_tok)
        io.logp = _ptr(logp)
        io.uniform = _ptr(uniform)
        io.temperature = temperature
        io.top_k = top_k
        io.sample_tok = _ptr(sample_tok)
        io.sample_logmu = _ptr(sample_logmu)
        io.z_trace = _ptr(z_trace)
        io.flags = (A.RLT_STEP_GRAPH if graph else 0) | (A.RLT_STEP_DEFER if defer else 0)
        io.top_p = top_p
        self._keep = (io, st.c())
        fn = A.rlt_decoder_step_noalloc if noalloc else A.rlt_decoder_step
        return fn(self.ctx, self._keep[1], io, current_stream() if stream is None else stream)

    def replay(self, st: DecoderState, lens: np.ndarray, splits: np.ndarray, e: torch.Tensor,
               mem: A.rlt_memory, tokens: torch.Tensor, logp: torch.Tensor, rows: Optional[np.ndarray] = None,
               s_trace: Optional[torch.Tensor] = None, stream=None) -> int:
        """e [B, T, d]; tokens int32 [B, T]; logp float32 [B, T]; s_trace [B, T, d]."""
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        splits = np.ascontiguousarray(splits, dtype=np.int32)
        io = A.rlt_replay_io()
        io.B = len(lens)
        rows_keep = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
        io.rows_host = None if rows_keep is None else rows_keep.ctypes.data
        io.len_host = lens.ctypes.data
        io.split_host = splits.ctypes.data
        io.e = e.data_ptr()
        io.e_stride_b = e.stride(0)
        io.e_stride_t = e.stride(1)
        io.mem = mem
        io.tokens = tokens.data_ptr()
        io.tok_stride_b = tokens.stride(0)
        io.logp = logp.data_ptr()
        io.logp_stride_b = logp.stride(0)
        if s_trace is not None:
            io.s_trace = s_trace.data_ptr()
            io.s_stride_b = s_trace.stride(0)
        stc = st.c()
        return A.rlt_replay_sequence(self.ctx, stc, io, current_stream() if stream is None else stream)

    def grad_buffers(self) -> Dict[str, torch.Tensor]:
        """Zeroed float32 gradient buffers, one per parameter of the default
        variants (keys as the parameters)."""
        names = ["s_star", "merge.wg", "merge.bg", "out.norm", "out.w"]
        if self.cfg.merge == "gated":
            names += ["merge.norm", "merge.ws"]
        names += ["layer.%d.%s" % (l, n) for l in range(self.cfg.L) for n in _MATRICES + _LAYER_VECS]
        return {n: torch.zeros(self.params[n].shape, dtype=torch.float32, device=self.device) for n in names}

    def replay_backward(self, grads: Dict[str, torch.Tensor], lens: np.ndarray, splits: np.ndarray,
                        e: torch.Tensor, mem: A.rlt_memory, tokens: torch.Tensor, w: torch.Tensor,
                        logp: Optional[torch.Tensor] = None, de: Optional[torch.Tensor] = None,
                        dmem_k: Optional[torch.Tensor] = None, dmem_v: Optional[torch.Tensor] = None,
                        stream=None) -> int:
        """Full-BPTT gradients of sum_b sum_t w[b, t] log p(x_{t+1} | x_{1:t}),
        accumulated into ``grads`` (from ``grad_buffers``); e [B, T, d];
        tokens int32 [B, T]; w, logp float32 [B, T]; de float32 [B, T, d];
        dmem_k / dmem_v float32 [G, B, T, d]."""
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        splits = np.ascontiguousarray(splits, dtype=np.int32)
        io = A.rlt_backward_io()
        io.B = len(lens)
        io.len_host = lens.ctypes.data
        io.split_host = splits.ctypes.data
        io.e, io.e_stride_b, io.e_stride_t = e.data_ptr(), e.stride(0), e.stride(1)
        io.mem = mem
        io.tokens, io.tok_stride_b = tokens.data_ptr(), tokens.stride(0)
        io.w, io.w_stride_b = w.data_ptr(), w.stride(0)
        if logp is not None:
            io.logp, io.logp_stride_b = logp.data_ptr(), logp.stride(0)
        if de is not None:
            io.de, io.de_stride_b, io.de_stride_t = de.data_ptr(), de.stride(0), de.stride(1)
        if dmem_k is not None:
            io.dmem_k, io.dmem_v = dmem_k.data_ptr(), dmem_v.data_ptr()
            io.dmem_stride_g, io.dmem_stride_b, io.dmem_stride_t = dmem_k.stride(0), dmem_k.stride(1), dmem_k.stride(2)
        L = self.cfg.L
        gr = A.rlt_grads()
        keep = []
        for field, key in (("s_star", "s_star"), ("merge_norm", "merge.norm"), ("merge_wg", "merge.wg"),
                           ("merge_bg", "merge.bg"), ("merge_ws", "merge.ws"), ("out_norm", "out.norm"),
                           ("w_out", "out.w")):
            if key in grads:
                setattr(gr, field, grads[key].data_ptr())
        for name in _MATRICES + _LAYER_VECS:
            keys = ["layer.%d.%s" % (l, name) for l in range(L)]
            if all(k in grads for k in keys):
                arr = (A.P * L)(*[grads[k].data_ptr() for k in keys])
                keep.append(arr)
                setattr(gr, name, C.cast(arr, C.POINTER(A.P)))
        return A.rlt_replay_backward(self.ctx, io, gr, current_stream() if stream is None else stream)

    def score(self, s: torch.Tensor, tokens: torch.Tensor, logp: torch.Tensor, *, temperature=1.0, top_k=0,
              top_p=1.0, logmu=None, logmu_behaviour=None, ratio=None, stream=None) -> int:
        io = A.rlt_score_io(s.shape[0], s.data_ptr(), tokens.data_ptr(), logp.data_ptr(), temperature, top_k,
                            _ptr(logmu), _ptr(logmu_behaviour), _ptr(ratio), top_p)
        return A.rlt_score_logprobs(self.ctx, io, current_stream() if stream is None else stream)

    def trajectory_log_ratio(self, lens: np.ndarray, splits: np.ndarray, logp: torch.Tensor, logmu: torch.Tensor,
                             out: torch.Tensor, stream=None) -> int:
        """out[b] = sum over t = splits[b] .. lens[b]-1 of logp[b, t] - logmu[b, t]."""
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        splits = np.ascontiguousarray(splits, dtype=np.int32)
        return A.rlt_trajectory_log_ratio(self.ctx, len(lens), lens.ctypes.data, splits.ctypes.data, logp.data_ptr(),
                                          logp.stride(0), logmu.data_ptr(), logmu.stride(0), out.data_ptr(),
                                          current_stream() if stream is None else stream)

    def sync_error(self, stream=None) -> int:
        return A.rlt_sync_error(self.ctx, current_stream() if stream is None else stream)

    def refresh_weights(self, version: int, stream=None) -> int:
        """The weight tensors were changed in place: rebuild the context's
        operand-order weight copy and adopt ``version`` (rlt_refresh_weights);
        states must then carry the new version (re-initialise them)."""
        rc = A.rlt_refresh_weights(self.ctx, version, current_stream() if stream is None else stream)
        if rc == A.RLT_OK:
            self.cfg.version = version
            self._cfg_c = self.cfg.to_c()
        return rc

    # -- exact prefix snapshots ---------------------------------------------------
    def snapshot(self, st: DecoderState, rows, stream=None) -> np.ndarray:
        """Snapshots of the listed rows: a uint8 array [n, bytes per row]
        (header, s, SWA cache), complete when this returns."""
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        per = A.rlt_snapshot_bytes(self._cfg_c)
        buf = np.zeros((len(rows), per), dtype=np.uint8)
        A.check(A.rlt_state_snapshot(self.ctx, st.c(), rows.ctypes.data, len(rows), buf.ctypes.data,
                                     current_stream() if stream is None else stream), "rlt_state_snapshot")
        return buf

    def restore(self, st: DecoderState, rows, snap: np.ndarray, stream=None) -> int:
        """Restore snapshot i into row rows[i]; returns the status code."""
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        snap = np.ascontiguousarray(snap, dtype=np.uint8)
        return A.rlt_state_restore(self.ctx, st.c(), rows.ctypes.data, len(rows), snap.ctypes.data,
                                   current_stream() if stream is None else stream)

    # -- encoder memory ------------------------------------------------------
    def memory_weights(self, params: Dict[str, object]) -> "MemoryWeights":
        """Device copies of the memory-map weights keyed "memory.{g}.norm_e",
        ".wk", ".wv" (one set per group)."""
        return MemoryWeights(self.cfg, params, self.device)

    def memory_append(self, mw: "MemoryWeights", mem: A.rlt_memory, B_cap: int, T_cap: int, rows: torch.Tensor,
                      e: torch.Tensor, stream=None) -> int:
        """Append one entry per listed memory row from e [n, d] (next position)."""
        return A.rlt_memory_append(self.ctx, mw.c, mem, B_cap, T_cap, rows.data_ptr(), rows.numel(), e.data_ptr(),
                                   current_stream() if stream is None else stream)

    def memory_prefill(self, mw: "MemoryWeights", mem: A.rlt_memory, T_cap: int, lens: np.ndarray,
                       e: torch.Tensor, stream=None) -> int:
        """Entries 1..lens[b] of memory rows b < len(lens) from e [B, T, d]."""
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        return A.rlt_memory_prefill(self.ctx, mw.c, mem, T_cap, len(lens), lens.ctypes.data, e.data_ptr(),
                                    e.stride(0), e.stride(1), current_stream() if stream is None else stream)

    def dbg_gemm(self, Amat: torch.Tensor, W: torch.Tensor, out: torch.Tensor, stream=None,
                 packed: bool = False) -> int:
        M, K = Amat.shape
        N = W.shape[0]
        fn = A.rlt_dbg_gemm_packed if packed else A.rlt_dbg_gemm
        return fn(self.ctx, Amat.data_ptr(), W.data_ptr(), M, N, K, out.data_ptr(),
                  current_stream() if stream is None else stream)


class MemoryWeights:
    """Device copies of the encoder-memory maps' parameters and the pointer
    arrays of ``rlt_memory_weights``."""

    def __init__(self, cfg: ModelConfig, params: Dict[str, object], device="cuda"):
        self.params = {k: to_device(v, cfg.dtype, device).contiguous() for k, v in params.items()}
        G = cfg.G
        self._arrays = {n: (A.P * G)(*[self.params["memory.%d.%s" % (g, n)].data_ptr() for g in range(G)])
                        for n in ("norm_e", "wk", "wv")}
        self.c = A.rlt_memory_weights(*[C.cast(self._arrays[n], C.POINTER(A.P)) for n in ("norm_e", "wk", "wv")])
