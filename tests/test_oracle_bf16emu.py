"""Pins of the rounding-emulation oracle (``oracle.bf16emu``), CPU only.

The emulation is a diagnostic: the plain float64 oracle stays the definition
of the transition. It is pinned (1) in its rounding function, against
torch's float32 -> bfloat16 conversion (round to nearest, ties to even), and
(2) in its arithmetic, which with the identity in place of the rounding must
equal the plain oracle ("Recurrent Looped Transformer" §2.3 eqs.
(2.4)-(2.6), §2.5 eqs. (2.9)-(2.16)) to 1e-12 for every merge, gate, rank
and sublayer order; a planted mistake in the rearranged products (a dropped
rstd, a gain applied twice, a missing residual) breaks (2). Where the
rounding is applied is not pinned here (identity rounding hides it): the GPU
tests compare the library with this oracle to far tighter tolerances than
with the plain one, which a missing or extra rounding point would break.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import Oracle
from oracle.bf16emu import RoundingOracle, bf16_round, two_term
from tests.helpers import e_of, memory_of, oracle_config, oracle_weights, rel_l2


def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        rng.standard_normal(1000)]).astype(np.float32)
    # exact ties: a float32 whose low 16 bits are 0x8000, both parities of bit 16
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), ref)


def _emu_vs_plain(wl, n=6, rows=(0, 1)):
    raw = synth.make_weights(wl)
    w = oracle_weights(raw)
    plain = Oracle(oracle_config(wl), w)
    idf = lambda a: np.asarray(a, dtype=np.float64)
    ident = RoundingOracle(oracle_config(wl), w, act=idf, kv=idf)
    rounded = RoundingOracle(oracle_config(wl), w, act=bf16_round)
    worst_id, worst_rnd = 0.0, 0.0
    for b in rows:
        mem, E = memory_of(wl, b), e_of(wl, b)
        sp, si, sr = plain.initial_state(), ident.initial_state(), rounded.initial_state()
        for t in range(n):
            sp, si, sr = (o.transition(s, E[t], mem) for o, s in ((plain, sp), (ident, si), (rounded, sr)))
            zp, zi, zr = plain.logits(sp.s), ident.logits(si.s), rounded.logits(sr.s)
            worst_id = max(worst_id, rel_l2(si.s, sp.s), rel_l2(zi, zp))
            worst_rnd = max(worst_rnd, rel_l2(sr.s, sp.s), rel_l2(zr, zp))
    return worst_id, worst_rnd


@pytest.mark.parametrize("over", [dict(), dict(merge="convex"), dict(gate="scalar"), dict(ws_rank=64),
                                  dict(order="xsf"), dict(order="fxs"), dict(G=4)],
                         ids=["gated", "convex", "scalar-gate", "rank64", "xsf", "fxs", "G=L"])
def test_identity_rounding_equals_plain_oracle(over):
    wl = synth.SMALL.with_(dtype="bf16", B=2, T=8, L=2, **over)
    worst_id, worst_rnd = _emu_vs_plain(wl)
    assert worst_id < 1e-12, worst_id
    # the rounding contract moves the results by bf16 noise, no more
    assert 1e-6 < worst_rnd < 2e-2, worst_rnd


def test_two_term_carries_sixteen_bits():
    """hi + lo with hi = bf16(x), lo = bf16(x - hi): relative error below
    2^-16 (each term keeps 8 significant bits; the remainder is at most half
    an ulp of hi), exact for bf16-valued x (lo = 0)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000)
    err = np.abs(two_term(x) - x) / np.abs(x)
    assert err.max() < 2.0 ** -16
    b = bf16_round(x)
    assert np.array_equal(two_term(b), b)
