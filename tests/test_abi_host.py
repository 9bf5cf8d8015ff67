"""Host-only checks of the C ABI (no GPU needed): the library loads, every
function declared in include/*.h is exported, the ctypes mirror has the
C layout, and host-checkable argument errors come back as status codes."""
import ctypes as C
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")


def _declared():
    names = set()
    for h in glob.glob(os.path.join(INC, "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(rlt_\w+)\s*\(", src, flags=re.M))
    return names


def test_library_exports_every_declared_function():
    from stateful_sequence_model_amd import _abi
    L = _abi.lib()
    decl = _declared()
    assert {"rlt_create", "rlt_destroy", "rlt_state_layout", "rlt_last_error", "rlt_init_state",
            "rlt_decoder_step", "rlt_replay_sequence", "rlt_score_logprobs", "rlt_sync_error",
            "rlt_memory_append", "rlt_memory_prefill", "rlt_snapshot_bytes", "rlt_state_snapshot",
            "rlt_state_restore", "rlt_trajectory_log_ratio", "rlt_replay_backward", "rlt_dbg_gemm"} <= decl
    for name in decl:
        assert hasattr(L, name), name
    assert decl == set(_abi.exported_symbols())


def test_ctypes_layout_matches_header(tmp_path):
    """Compile a C program against include/rlt.h that prints sizeof/offsetof
    of every struct field and compare with the ctypes mirror."""
    from stateful_sequence_model_amd import _abi
    structs = {"rlt_config": _abi.rlt_config, "rlt_weights": _abi.rlt_weights, "rlt_state": _abi.rlt_state,
               "rlt_memory": _abi.rlt_memory, "rlt_step_io": _abi.rlt_step_io,
               "rlt_replay_io": _abi.rlt_replay_io, "rlt_score_io": _abi.rlt_score_io,
               "rlt_memory_weights": _abi.rlt_memory_weights, "rlt_snapshot_header": _abi.rlt_snapshot_header,
               "rlt_grads": _abi.rlt_grads, "rlt_backward_io": _abi.rlt_backward_io,
               "rlt_dbg_launch": _abi.rlt_dbg_launch, "rlt_narrow_report": _abi.rlt_narrow_report}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "rlt.h"', '#include "rlt_debug.h"',
             "int main(void){"]
    for sname, cls in structs.items():
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (sname, sname))
        for fname, _ in cls._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (sname, fname, sname, fname))
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", INC, str(src), "-o", str(exe)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)], text=True).splitlines())
    for sname, cls in structs.items():
        assert int(got[sname]) == C.sizeof(cls), sname
        for fname, _ in cls._fields_:
            assert int(got["%s.%s" % (sname, fname)]) == getattr(cls, fname).offset, (sname, fname)


def _cfg(**kw):
    from stateful_sequence_model_amd import ModelConfig
    base = dict(L=2, d=64, H=4, dh=16, W=4, G=1, F=128, V=256, dtype="f32", merge="convex")
    base.update(kw)
    return ModelConfig(**base).to_c()


def test_state_layout_sizes():
    from stateful_sequence_model_amd import _abi
    s = _abi.rlt_state_layout(_cfg(), 3)
    assert s == [3 * 64 * 4, 2 * 3 * 3 * 64 * 4, 2 * 3 * 3 * 64 * 4, 12, 12]
    s = _abi.rlt_state_layout(_cfg(dtype="bf16", dh=32, H=2, W=1), 5)
    assert s[1] == 0 and s[2] == 0 and s[0] == 5 * 64 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(d=60), -2),                   # d != H * dh
    (dict(dh=16, dtype="bf16"), -8),    # head width 16 needs float32
    (dict(dh=48, H=2, d=96), -8),       # unsupported head width
    (dict(G=2, L=3), -8),               # groups must be 1 or L_D
    (dict(W=0), -1),
    (dict(V=250), -8),                  # vocab multiple of 32
    (dict(gate="scalar"), -8),          # scalar gate: gated merge only (_cfg is convex)
    (dict(merge="gated", ws_rank=48), -8),   # rank not a multiple of 32
    (dict(merge="gated", ws_rank=96), -8),   # rank above d
    (dict(ws_rank=32), -1),             # low rank needs the gated merge
])
def test_config_validation(kw, code):
    from stateful_sequence_model_amd import _abi
    out = (C.c_size_t * 5)()
    cfg = _cfg(**kw)
    assert _abi.lib().rlt_state_layout(C.byref(cfg), 4, out) == code
    assert _abi.rlt_last_error()


def test_config_rejects_bad_enums():
    from stateful_sequence_model_amd import _abi
    out = (C.c_size_t * 5)()
    for field, value in (("merge_gate", 2), ("block_order", 6), ("block_order", -1)):
        cfg = _cfg()
        setattr(cfg, field, value)
        assert _abi.lib().rlt_state_layout(C.byref(cfg), 4, out) == _abi.RLT_EINVAL, field


def test_create_rejects_missing_weights_before_touching_the_device():
    from stateful_sequence_model_amd import _abi
    cfg = _cfg()
    w = _abi.rlt_weights()
    h = C.c_void_p()
    assert _abi.lib().rlt_create(C.byref(cfg), C.byref(w), 4, 32, C.byref(h)) == _abi.RLT_EINVAL
    assert h.value is None
    opt = _abi.rlt_dbg_launch()
    assert _abi.lib().rlt_dbg_create(C.byref(cfg), C.byref(w), 4, 32, C.byref(opt), C.byref(h)) == _abi.RLT_EINVAL
    assert _abi.lib().rlt_dbg_create(C.byref(cfg), C.byref(w), 4, 32, None, C.byref(h)) == _abi.RLT_EINVAL
    assert h.value is None


def test_null_arguments_are_rejected():
    from stateful_sequence_model_amd import _abi
    L = _abi.lib()
    assert L.rlt_decoder_step(None, None, None, None) == _abi.RLT_EINVAL
    assert L.rlt_replay_sequence(None, None, None, None) == _abi.RLT_EINVAL
    assert L.rlt_score_logprobs(None, None, None) == _abi.RLT_EINVAL
    assert L.rlt_init_state(None, None, None, 0, 0, None) == _abi.RLT_EINVAL
    assert L.rlt_sync_error(None, None) == _abi.RLT_EINVAL
    assert L.rlt_memory_append(None, None, None, 0, 0, None, 0, None, None) == _abi.RLT_EINVAL
    assert L.rlt_state_snapshot(None, None, None, 0, None, None) == _abi.RLT_EINVAL
    assert L.rlt_state_restore(None, None, None, 0, None, None) == _abi.RLT_EINVAL
    assert L.rlt_refresh_weights(None, 2, None) == _abi.RLT_EINVAL
    assert L.rlt_dbg_gemm(None, None, None, 1, 32, 32, None, None) == _abi.RLT_EINVAL
    assert L.rlt_dbg_gemm_packed(None, None, None, 1, 32, 64, None, None) == _abi.RLT_EINVAL
    assert L.rlt_memory_prefill(None, None, None, 0, 0, None, None, 0, 0, None) == _abi.RLT_EINVAL
    assert L.rlt_replay_backward(None, None, None, None) == _abi.RLT_EINVAL
    assert L.rlt_dbg_stream_read(None, 16, 1, None, None) == _abi.RLT_EINVAL
    assert L.rlt_dbg_mfma_loop(1, 1, None, None) == _abi.RLT_EINVAL
    # sizes are checked before any launch (the sink pointer is never touched)
    assert L.rlt_dbg_mfma_loop(0, 1, 16, None) == _abi.RLT_ESHAPE
    assert L.rlt_dbg_mfma_loop(1, 0, 16, None) == _abi.RLT_ESHAPE


def test_snapshot_size_and_magic():
    """One row's snapshot: header, s (float32), both SWA caches; the magic
    constant spells "RLTS" in memory order."""
    from stateful_sequence_model_amd import _abi
    import ctypes as C
    cfg = _cfg()
    per = _abi.rlt_snapshot_bytes(cfg)
    assert C.sizeof(_abi.rlt_snapshot_header) == 64
    assert per == 64 + 64 * 4 + 2 * 2 * 3 * 64 * 4   # L=2, W-1=3, d=64, float32
    assert _abi.RLT_SNAPSHOT_MAGIC.to_bytes(4, "little") == b"RLTS"
