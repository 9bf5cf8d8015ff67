"""Host-side walk of the narrow product tile's address arithmetic (no GPU).

The narrow tile (``gemm_bf16_body``: calls of up to 32 rows of the products
that have no fragment-order weight copy, the memory construction's small
calls, and every product of the persistent step) takes its K split, row
blocks and per-wave K slice from the launcher's plan and its load and store
addresses from a handful of index functions. ``rlt_dbg_narrow_bounds`` runs
the launcher's plan and those same functions on the CPU over every
workgroup and lane; this test checks, for every product shape of the bf16
workloads at row counts up to the context's capacity (the tile edges and
the capacity itself), that each read
stays inside the activations (rows < M_pad, columns < K) and the weights
(segment, row, column), each partial and row-statistics store inside its
buffer, and that every 32-wide K step is multiplied exactly once.
"""
import ctypes as C

import pytest

import synth

PAIR_PLAIN, PAIR_ROPE, PAIR_DUAL = 0, 1, 2


def _sites(wl):
    """(name, nseg, seg_rows, K, pairing) of every product of a transition,
    the memory construction and the readout."""
    d, F, V = wl.d, wl.F, wl.V
    sites = [("qkv", 3, d, d, PAIR_ROPE), ("wo", 1, d, d, PAIR_PLAIN), ("wqm", 1, d, d, PAIR_ROPE),
             ("wom", 1, d, d, PAIR_PLAIN), ("gate/up", 2, F, d, PAIR_DUAL), ("down", 1, d, F, PAIR_PLAIN),
             ("vocab", 1, V, d, PAIR_PLAIN), ("merge gate", 1, d, 2 * d, PAIR_PLAIN),
             ("merge W_s", 1, d, d, PAIR_PLAIN), ("memory k/v", 2, d, d, PAIR_ROPE)]
    if wl.ws_rank:
        sites += [("W_s V", 1, wl.ws_rank, d, PAIR_PLAIN), ("W_s U", 1, d, wl.ws_rank, PAIR_PLAIN)]
    return [s for s in sites if (s[1] * s[2]) % 32 == 0 and s[3] % 32 == 0]


def _walk(n, nseg, seg_rows, K, pairing, dh, M_pad, nr, target, cap):
    from stateful_sequence_model_amd import _abi
    rep = _abi.rlt_narrow_report()
    npairs = nseg * seg_rows // 32
    rc = _abi.lib().rlt_dbg_narrow_bounds(n, npairs, K, pairing, dh, nseg, seg_rows, M_pad, nr, target, cap,
                                          C.byref(rep))
    assert rc == 0, _abi.lib().rlt_last_error()
    return rep, npairs


# the bf16 workloads (the float32 one runs its own product kernel; bf16
# contexts need heads of at least 32, which rlt_create enforces)
@pytest.mark.parametrize("wl", [synth.SMALL, synth.MID, synth.REF, synth.RAGGED, synth.SMALL.with_(ws_rank=64)],
                         ids=lambda w: w.name + ("_lowrank" if w.ws_rank else ""))
def test_narrow_tile_accesses_stay_in_bounds(wl):
    checked = 0
    for max_rows in (1, 5, 16, 32, 33, 100, 128, 256):
        M_pad = (max_rows + 127) // 128 * 128
        cap = 8 * M_pad * max(3 * wl.d, 2 * wl.F)
        nr = min(max_rows, 32)
        for name, nseg, seg_rows, K, pairing in _sites(wl):
            pads = [M_pad] if name != "memory k/v" else [max(M_pad, 8192)]
            for mp in pads:
                rows = sorted(set([1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, max_rows]) & set(range(1, max_rows + 1)))
                for n in rows:
                    for target in (0, 256):
                        rep, npairs = _walk(n, nseg, seg_rows, K, pairing, wl.dh, mp, nr, target, cap)
                        where = (name, max_rows, n, target, rep.S, rep.mb, rep.kslice)
                        assert 0 <= rep.a_row_max < mp, where
                        assert rep.a_col_end <= K, where
                        assert 0 <= rep.w_seg_max < nseg and 0 <= rep.w_row_max < seg_rows, where
                        assert rep.partial_end <= cap, where
                        assert rep.ssq_end <= npairs * mp, where
                        assert rep.steps_missing == 0 and rep.steps_repeated == 0, where
                        assert (rep.S == 1) == (rep.partial_end == 0), where
                        checked += 1
    assert checked > 100


def test_narrow_walk_catches_a_short_activation_buffer():
    """The walk reports what the kernel would read: a tile of 64 rows (a
    33-row call) reads rows up to 63, past a 40-row buffer."""
    rep, _ = _walk(33, 1, 256, 256, PAIR_PLAIN, 32, 40, 32, 0, 1 << 30)
    assert rep.mb == 4 and rep.a_row_max == 63
