"""ctypes mirror of include/rlt.h and include/rlt_debug.h.

Argument marshalling only: every function forwards to ``librlt.so``. The
library must be built (``stateful_sequence_model_amd.build``); importing
this module without it raises, there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librlt.so")

RLT_OK, RLT_EINVAL, RLT_ESHAPE, RLT_EPREFIX, RLT_ESTALE = 0, -1, -2, -3, -4
RLT_EPENDING, RLT_EHIP, RLT_ENOMEM, RLT_EUNSUPPORTED = -5, -6, -7, -8
RLT_F32, RLT_BF16 = 0, 1
RLT_MERGE_GATED, RLT_MERGE_CONVEX = 0, 1
RLT_POS_NONE, RLT_POS_ROPE = 0, 1
RLT_STEP_GRAPH, RLT_STEP_DEFER = 1, 2
RLT_INIT_POISON = 1
RLT_GATE_VECTOR, RLT_GATE_SCALAR = 0, 1
ORDERS = ("sxf", "sfx", "xsf", "xfs", "fsx", "fxs")   # RLT_ORDER_SXF .. RLT_ORDER_FXS

STATUS_NAMES = {0: "RLT_OK", -1: "RLT_EINVAL", -2: "RLT_ESHAPE", -3: "RLT_EPREFIX", -4: "RLT_ESTALE",
                -5: "RLT_EPENDING", -6: "RLT_EHIP", -7: "RLT_ENOMEM", -8: "RLT_EUNSUPPORTED"}

P = C.c_void_p
i32, i64, u64, f32 = C.c_int32, C.c_int64, C.c_uint64, C.c_float


class rlt_config(C.Structure):
    _fields_ = [("n_layers", i32), ("d_model", i32), ("n_heads", i32), ("d_head", i32), ("window", i32),
                ("n_groups", i32), ("d_ffn", i32), ("vocab", i32), ("merge_kind", i32), ("pos_kind", i32),
                ("dtype", i32), ("alpha", f32), ("rms_eps", f32), ("rope_theta", f32),
                ("weights_version", u64), ("merge_gate", i32), ("merge_rank", i32), ("block_order", i32)]


class rlt_weights(C.Structure):
    _fields_ = [("s_star", P), ("merge_norm", P), ("merge_wg", P), ("merge_bg", P), ("merge_ws", P),
                ("norm_s", C.POINTER(P)), ("wq", C.POINTER(P)), ("wk", C.POINTER(P)), ("wv", C.POINTER(P)),
                ("wo", C.POINTER(P)), ("norm_m", C.POINTER(P)), ("wqm", C.POINTER(P)), ("wom", C.POINTER(P)),
                ("norm_d", C.POINTER(P)), ("w_gate", C.POINTER(P)), ("w_up", C.POINTER(P)),
                ("w_down", C.POINTER(P)), ("out_norm", P), ("w_out", P), ("merge_ws_u", P), ("merge_ws_v", P)]


class rlt_state(C.Structure):
    _fields_ = [("s", P), ("ring_k", P), ("ring_v", P), ("pos", P), ("pending", P), ("B_cap", i32),
                ("version", u64)]


class rlt_memory(C.Structure):
    _fields_ = [("k", P), ("v", P), ("stride_g", i64), ("stride_b", i64), ("stride_t", i64), ("mem_len", P)]


class rlt_step_io(C.Structure):
    _fields_ = [("n", i32), ("rows", P), ("e", P), ("mem", rlt_memory), ("consume_tok", P), ("s_out", P),
                ("logits", P), ("argmax", P), ("score_tok", P), ("logp", P), ("uniform", P),
                ("temperature", f32), ("top_k", i32), ("sample_tok", P), ("sample_logmu", P),
                ("z_trace", P), ("flags", i32), ("top_p", f32)]


class rlt_replay_io(C.Structure):
    _fields_ = [("B", i32), ("rows_host", P), ("len_host", P), ("split_host", P), ("e", P),
                ("e_stride_b", i64), ("e_stride_t", i64), ("mem", rlt_memory), ("tokens", P),
                ("tok_stride_b", i64), ("logp", P), ("logp_stride_b", i64), ("s_trace", P),
                ("s_stride_b", i64)]


class rlt_score_io(C.Structure):
    _fields_ = [("n", i32), ("s", P), ("tokens", P), ("logp", P), ("temperature", f32), ("top_k", i32),
                ("logmu", P), ("logmu_behaviour", P), ("ratio", P), ("top_p", f32)]


class rlt_snapshot_header(C.Structure):
    _fields_ = [("magic", C.c_uint32), ("layout", C.c_uint32), ("weights_version", u64), ("n_layers", i32),
                ("d_model", i32), ("window", i32), ("dtype", i32), ("pos", i32), ("pending", i32),
                ("reserved", i32 * 6)]


RLT_SNAPSHOT_MAGIC = 0x53544C52
RLT_NOALLOC_MAX_ROWS = 65536


class rlt_memory_weights(C.Structure):
    _fields_ = [("norm_e", C.POINTER(P)), ("wk", C.POINTER(P)), ("wv", C.POINTER(P))]


class rlt_grads(C.Structure):
    _fields_ = [("s_star", P), ("merge_norm", P), ("merge_wg", P), ("merge_bg", P), ("merge_ws", P),
                ("norm_s", C.POINTER(P)), ("wq", C.POINTER(P)), ("wk", C.POINTER(P)), ("wv", C.POINTER(P)),
                ("wo", C.POINTER(P)), ("norm_m", C.POINTER(P)), ("wqm", C.POINTER(P)), ("wom", C.POINTER(P)),
                ("norm_d", C.POINTER(P)), ("w_gate", C.POINTER(P)), ("w_up", C.POINTER(P)),
                ("w_down", C.POINTER(P)), ("out_norm", P), ("w_out", P)]


class rlt_backward_io(C.Structure):
    _fields_ = [("B", i32), ("len_host", P), ("split_host", P), ("e", P), ("e_stride_b", i64),
                ("e_stride_t", i64), ("mem", rlt_memory), ("tokens", P), ("tok_stride_b", i64), ("w", P),
                ("w_stride_b", i64), ("logp", P), ("logp_stride_b", i64), ("de", P), ("de_stride_b", i64),
                ("de_stride_t", i64), ("dmem_k", P), ("dmem_v", P), ("dmem_stride_g", i64),
                ("dmem_stride_b", i64), ("dmem_stride_t", i64)]


class rlt_narrow_report(C.Structure):
    _fields_ = [("S", i32), ("mb", i32), ("kslice", i32), ("w_seg_max", i32), ("w_row_max", i32), ("pad_", i32),
                ("a_row_max", i64), ("a_col_end", i64), ("partial_end", i64), ("ssq_end", i64),
                ("steps_missing", i64), ("steps_repeated", i64)]


class rlt_dbg_launch(C.Structure):
    _fields_ = [("xattn_chunk", i32), ("swa_hpw", i32), ("xattn_hpw", i32), ("fused_rows", i32),
                ("no_packed", i32), ("one_term", i32), ("replay_graph_min", i32),
                ("no_big_tile", i32), ("xattn_combine_kernel", i32),
                ("one_row_pf", i32), ("no_lt_dma", i32),
                ("bwd_activations", i32)]


_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "rlt_create": (C.c_int, [C.POINTER(rlt_config), C.POINTER(rlt_weights), i32, i32, C.POINTER(P)]),
    "rlt_destroy": (None, [P]),
    "rlt_state_layout": (C.c_int, [C.POINTER(rlt_config), i32, C.POINTER(C.c_size_t)]),
    "rlt_last_error": (C.c_char_p, []),
    "rlt_init_state": (C.c_int, [P, C.POINTER(rlt_state), P, i32, i32, P]),
    "rlt_decoder_step": (C.c_int, [P, C.POINTER(rlt_state), C.POINTER(rlt_step_io), P]),
    "rlt_decoder_step_noalloc": (C.c_int, [P, C.POINTER(rlt_state), C.POINTER(rlt_step_io), P]),
    "rlt_replay_sequence": (C.c_int, [P, C.POINTER(rlt_state), C.POINTER(rlt_replay_io), P]),
    "rlt_score_logprobs": (C.c_int, [P, C.POINTER(rlt_score_io), P]),
    "rlt_sync_error": (C.c_int, [P, P]),
    "rlt_refresh_weights": (C.c_int, [P, u64, P]),
    "rlt_trajectory_log_ratio": (C.c_int, [P, i32, P, P, P, i64, P, i64, P, P]),
    "rlt_snapshot_bytes": (C.c_int, [C.POINTER(rlt_config), C.POINTER(C.c_size_t)]),
    "rlt_state_snapshot": (C.c_int, [P, C.POINTER(rlt_state), P, i32, P, P]),
    "rlt_state_restore": (C.c_int, [P, C.POINTER(rlt_state), P, i32, P, P]),
    "rlt_memory_append": (C.c_int, [P, C.POINTER(rlt_memory_weights), C.POINTER(rlt_memory), i32, i32, P, i32, P, P]),
    "rlt_memory_prefill": (C.c_int, [P, C.POINTER(rlt_memory_weights), C.POINTER(rlt_memory), i32, i32, P, P, i64,
                                     i64, P]),
    "rlt_replay_backward": (C.c_int, [P, C.POINTER(rlt_backward_io), C.POINTER(rlt_grads), P]),
    "rlt_dbg_create": (C.c_int, [C.POINTER(rlt_config), C.POINTER(rlt_weights), i32, i32,
                                 C.POINTER(rlt_dbg_launch), C.POINTER(P)]),
    "rlt_dbg_gemm": (C.c_int, [P, P, P, i32, i32, i32, P, P]),
    "rlt_dbg_gemm_packed": (C.c_int, [P, P, P, i32, i32, i32, P, P]),
    "rlt_dbg_product_shape": (C.c_int, [P, i32, i32, i32, i32, i32]),
    "rlt_dbg_stream_read": (C.c_int, [P, i64, i32, P, P]),
    "rlt_dbg_mfma_loop": (C.c_int, [i32, i32, P, P]),
    "rlt_dbg_narrow_bounds": (C.c_int, [i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, i64,
                                        C.POINTER(rlt_narrow_report)]),
    "rlt_dbg_profile": (C.c_int, [P, i32]),
    "rlt_dbg_profile_read": (C.c_int, [P, i32, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
}

RLT_PROF_XATTN, RLT_PROF_XCOMBINE, RLT_PROF_SWA, RLT_PROF_GEMM, RLT_PROF_NORM, RLT_PROF_READOUT, RLT_PROF_FUSED = range(7)
PROF_NAMES = ["xattn", "xcombine", "swa", "gemm", "norm", "readout", "fused"]


def lib():
    """The loaded ``librlt.so``. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("librlt.so not built: run `python -m stateful_sequence_model_amd.build` "
                               "(there is no fallback implementation)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class RltError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = lib().rlt_last_error().decode(errors="replace")
        super().__init__("%s returned %s (%d): %s" % (where, STATUS_NAMES.get(code, "?"), code, msg))


def check(code: int, where: str) -> int:
    if code != RLT_OK:
        raise RltError(code, where)
    return code


# thin wrappers with the C names ----------------------------------------------

def rlt_create(cfg: rlt_config, w: rlt_weights, max_rows: int, max_ctx: int) -> int:
    h = P()
    check(lib().rlt_create(C.byref(cfg), C.byref(w), max_rows, max_ctx, C.byref(h)), "rlt_create")
    return h.value


def rlt_dbg_create(cfg: rlt_config, w: rlt_weights, max_rows: int, max_ctx: int, opt: rlt_dbg_launch) -> int:
    h = P()
    check(lib().rlt_dbg_create(C.byref(cfg), C.byref(w), max_rows, max_ctx, C.byref(opt), C.byref(h)),
          "rlt_dbg_create")
    return h.value


def rlt_destroy(ctx: int) -> None:
    lib().rlt_destroy(ctx)


def rlt_state_layout(cfg: rlt_config, B_cap: int):
    out = (C.c_size_t * 5)()
    check(lib().rlt_state_layout(C.byref(cfg), B_cap, out), "rlt_state_layout")
    return list(out)


def rlt_last_error() -> str:
    return lib().rlt_last_error().decode(errors="replace")


def rlt_init_state(ctx: int, st: rlt_state, rows: int, n: int, flags: int, stream: int) -> int:
    return lib().rlt_init_state(ctx, C.byref(st), rows, n, flags, stream)


def rlt_decoder_step(ctx: int, st: rlt_state, io: rlt_step_io, stream: int) -> int:
    return lib().rlt_decoder_step(ctx, C.byref(st), C.byref(io), stream)


def rlt_decoder_step_noalloc(ctx: int, st: rlt_state, io: rlt_step_io, stream: int) -> int:
    return lib().rlt_decoder_step_noalloc(ctx, C.byref(st), C.byref(io), stream)


def rlt_replay_sequence(ctx: int, st: rlt_state, io: rlt_replay_io, stream: int) -> int:
    return lib().rlt_replay_sequence(ctx, C.byref(st), C.byref(io), stream)


def rlt_replay_backward(ctx: int, io: rlt_backward_io, grads: rlt_grads, stream: int) -> int:
    return lib().rlt_replay_backward(ctx, C.byref(io), C.byref(grads), stream)


def rlt_score_logprobs(ctx: int, io: rlt_score_io, stream: int) -> int:
    return lib().rlt_score_logprobs(ctx, C.byref(io), stream)


def rlt_sync_error(ctx: int, stream: int) -> int:
    return lib().rlt_sync_error(ctx, stream)


def rlt_refresh_weights(ctx: int, version: int, stream: int) -> int:
    return lib().rlt_refresh_weights(ctx, version, stream)


def rlt_trajectory_log_ratio(ctx: int, B: int, len_host, split_host, logp: int, logp_sb: int, logmu: int,
                             logmu_sb: int, out: int, stream: int) -> int:
    return lib().rlt_trajectory_log_ratio(ctx, B, len_host, split_host, logp, logp_sb, logmu, logmu_sb, out, stream)


def rlt_snapshot_bytes(cfg: rlt_config) -> int:
    out = C.c_size_t(0)
    check(lib().rlt_snapshot_bytes(C.byref(cfg), C.byref(out)), "rlt_snapshot_bytes")
    return out.value


def rlt_state_snapshot(ctx: int, st: rlt_state, rows_host, n: int, dst, stream: int) -> int:
    return lib().rlt_state_snapshot(ctx, C.byref(st), rows_host, n, dst, stream)


def rlt_state_restore(ctx: int, st: rlt_state, rows_host, n: int, src, stream: int) -> int:
    return lib().rlt_state_restore(ctx, C.byref(st), rows_host, n, src, stream)


def rlt_memory_append(ctx: int, mw: rlt_memory_weights, mem: rlt_memory, B_cap: int, T_cap: int, rows: int, n: int,
                      e: int, stream: int) -> int:
    return lib().rlt_memory_append(ctx, C.byref(mw), C.byref(mem), B_cap, T_cap, rows, n, e, stream)


def rlt_memory_prefill(ctx: int, mw: rlt_memory_weights, mem: rlt_memory, T_cap: int, B: int, len_host, e: int,
                       e_stride_b: int, e_stride_t: int, stream: int) -> int:
    return lib().rlt_memory_prefill(ctx, C.byref(mw), C.byref(mem), T_cap, B, len_host, e, e_stride_b, e_stride_t,
                                    stream)


def rlt_dbg_gemm(ctx: int, A: int, W: int, M: int, N: int, K: int, out: int, stream: int) -> int:
    return lib().rlt_dbg_gemm(ctx, A, W, M, N, K, out, stream)


def rlt_dbg_gemm_packed(ctx: int, A: int, W: int, M: int, N: int, K: int, out: int, stream: int) -> int:
    return lib().rlt_dbg_gemm_packed(ctx, A, W, M, N, K, out, stream)


def rlt_dbg_product_shape(ctx: int, rb: int, cb: int, lt: int, pf: int, pre: int) -> int:
    return lib().rlt_dbg_product_shape(ctx, rb, cb, lt, pf, pre)


def rlt_dbg_profile(ctx: int, enable: int) -> int:
    return lib().rlt_dbg_profile(ctx, enable)


def rlt_dbg_profile_read(ctx: int, kind: int):
    ms, n = C.c_double(), C.c_int64()
    check(lib().rlt_dbg_profile_read(ctx, kind, C.byref(ms), C.byref(n)), "rlt_dbg_profile_read")
    return ms.value, n.value


def exported_symbols():
    return list(_SIGS)
