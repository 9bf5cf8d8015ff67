"""GPU parity of the decoder transition against the CPU oracle.

Tolerances (stated for the two precisions the library computes in):
  float32 mode: relative L2 of s_t and of the logits <= 1e-4 at every
                checked (sequence, step);
  bfloat16 mode: relative L2 <= 2e-2 at every checked (sequence, step) and
                 top-1 agreement of the logits >= 99 %, against the float64
                 oracle run on the identical bf16-valued weights and inputs.
Integer work (positions, ring slot placement, pending tokens) is exact.
"""
import numpy as np
import pytest

import synth
from oracle import Memory, Oracle
from tests.gpu_common import GpuRun, require_gpu, torch
from tests.helpers import make_oracle, oracle_config, oracle_weights, rel_l2, widen

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOP1_BF16 = 0.99


def _oracle_run(run: GpuRun, b: int, nsteps: int, orc: Oracle = None, over=None):
    """oracle s_t and logits for sequence b of the run, t = 1..nsteps."""
    wl = run.wl
    orc = orc or Oracle(oracle_config(wl, **(over or {})), oracle_weights(run.raw))
    mem = Memory([widen(run.mk[g, b]) for g in range(wl.G)], [widen(run.mv[g, b]) for g in range(wl.G)])
    E = widen(run.E[b])
    st = orc.initial_state()
    S, Z = [], []
    for t in range(1, nsteps + 1):
        st = orc.transition(st, E[t - 1], mem)
        S.append(st.s)
        Z.append(orc.logits(st.s))
    return np.array(S), np.array(Z), st, orc


def _compare(S, Z, So, Zo, tol):
    worst_s = max(rel_l2(S[i], So[i]) for i in range(len(So)))
    worst_z = max(rel_l2(Z[i], Zo[i]) for i in range(len(Zo)))
    top1 = np.mean([np.argmax(Z[i]) == np.argmax(Zo[i]) for i in range(len(Zo))])
    return worst_s, worst_z, top1


def test_gemm_kernel_parity():
    """The matrix-product kernel alone (bf16 MFMA, all M-tile sizes and a K
    split) against float64 products of the same bf16 values."""
    require_gpu()
    from stateful_sequence_model_amd import to_device
    wl = synth.SMALL
    run = GpuRun(wl, B=1, T=4, max_rows=200)
    rng = np.random.default_rng(0)
    # above 32 rows with N/32 even and 64 | K the LDS tile (128 rows x 64 or
    # 128 columns) runs: its K loop has a 2-stage body and a tail of 0-1
    # stages of 64 (K = 192, 448, 704: odd stage counts; the last with a K
    # split whose final split is empty); N = 96 (odd pair count) falls back
    # to the narrow tile; M = 200 spans two row tiles; N = 32768 takes the
    # 128-column tile
    for M, N, K in [(1, 256, 512), (5, 64, 256), (16, 768, 256), (33, 96, 512), (70, 256, 384), (128, 512, 512),
                    (200, 128, 256), (70, 256, 192), (128, 512, 448), (96, 1024, 704), (40, 32768, 256)]:
        Abits = synth.normal(7, "dbgA%d" % M, (M, K), dtype="bf16")
        Wbits = synth.normal(7, "dbgW%d" % M, (N, K), sigma=0.05, dtype="bf16")
        Ad, Wd = to_device(Abits, "bf16"), to_device(Wbits, "bf16")
        out = torch.empty((M, N), device="cuda")
        assert run.dec.dbg_gemm(Ad, Wd, out) == 0
        torch.cuda.synchronize()
        ref = widen(Abits) @ widen(Wbits).T
        err = np.abs(out.double().cpu().numpy() - ref).max() / np.abs(ref).max()
        assert err < 1e-5, (M, N, K, err)


def test_gemm_operand_order_parity():
    """The operand-order product of the decoder's bf16 calls (both operands
    in the 32x32x16 instruction's order, no K split) against float64
    products: the three tile shapes (32 rows x 1 pair: M=70 N=256; 64 x 1:
    M=64 N=6144; 64 x 2: M=200 N=8192), K of 1, 3, 7 and 11 chunks of 64
    (waves with 0-3 chunks, the 2-deep register ring's tail), a ragged last
    row tile, and calls of 1-32 rows (lanes of absent rows load nothing):
    eight waves per workgroup with a 4-deep ring up to 256 workgroups (waves
    with 0-2 chunks here; full turns of that ring run in the model-level
    tests, K = 2816 and 5504), four waves beyond (M=3 N=9216: 288
    workgroups); the 64 x 2 tile with eight waves (M=100 N=6144: 192
    workgroups, ragged second row tile) and 64 x 1 with four (M=64 N=9600:
    304)."""
    require_gpu()
    from stateful_sequence_model_amd import to_device
    wl = synth.SMALL
    run = GpuRun(wl, B=1, T=4, max_rows=200)
    for M, N, K in [(70, 256, 64), (33, 96, 192), (64, 6144, 448), (200, 8192, 704), (128, 512, 704),
                    (40, 32768, 256), (1, 256, 64), (5, 2048, 704), (16, 96, 192), (32, 4096, 256),
                    (3, 9216, 448), (100, 6144, 448), (64, 9600, 256)]:
        Abits = synth.normal(8, "pkA%d" % M, (M, K), dtype="bf16")
        Wbits = synth.normal(8, "pkW%d" % N, (N, K), sigma=0.05, dtype="bf16")
        Ad, Wd = to_device(Abits, "bf16"), to_device(Wbits, "bf16")
        out = torch.empty((M, N), device="cuda")
        assert run.dec.dbg_gemm(Ad, Wd, out, packed=True) == 0
        torch.cuda.synchronize()
        ref = widen(Abits) @ widen(Wbits).T
        err = np.abs(out.double().cpu().numpy() - ref).max() / np.abs(ref).max()
        assert err < 1e-5, (M, N, K, err)


def test_tiny_fp32_full_sequence():
    """Tiny float32 workload (L_D=2, d=64, 4x16 heads, W=4, convex merge):
    all 32 transitions against the oracle."""
    require_gpu()
    wl = synth.TINY
    run = GpuRun(wl)
    run.init()
    S, Z = run.run(wl.T)
    So, Zo, _, _ = _oracle_run(run, 0, wl.T)
    ws, wz, top1 = _compare(S[:, 0], Z[:, 0], So, Zo, TOL_F32)
    assert ws < TOL_F32 and wz < TOL_F32, (ws, wz)
    assert int(run.st.pos[0].item()) == wl.T


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_batched(dtype):
    """Small workload (L_D=4, d=256, 8x32 heads, W=16, per-layer memory
    G=L_D, gated merge), 16 sequences x 256 transitions in one batch."""
    require_gpu()
    wl = synth.SMALL.with_(dtype=dtype)
    run = GpuRun(wl)
    run.init()
    S, Z = run.run(wl.T)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    agree = []
    worst_s = worst_z = 0.0
    for b in range(wl.B):
        So, Zo, st, _ = _oracle_run(run, b, wl.T)
        ws, wz, top1 = _compare(S[:, b], Z[:, b], So, Zo, tol)
        worst_s, worst_z = max(worst_s, ws), max(worst_z, wz)
        agree.append(top1)
    print("small %s: max rel L2 s %.2e logits %.2e, top-1 %.4f" % (dtype, worst_s, worst_z, np.mean(agree)))
    assert worst_s < tol and worst_z < tol
    if dtype == "bf16":
        assert np.mean(agree) >= TOP1_BF16
    assert torch.equal(run.st.pos.cpu(), torch.full((wl.B,), wl.T, dtype=torch.int32))


@pytest.mark.parametrize("dtype,dh", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_head_widths(dtype, dh):
    """Head widths whose per-head lane groups (4, 8 or 16 lanes per head)
    the other small cases do not reach: L_D=2, d=256, W=8, 3 sequences x 24
    transitions against the oracle."""
    require_gpu()
    wl = synth.SMALL.with_(L=2, H=256 // dh, dh=dh, W=8, G=1, B=3, T=24, dtype=dtype)
    run = GpuRun(wl)
    run.init()
    S, Z = run.run(wl.T)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    agree = []
    for b in range(wl.B):
        So, Zo, _, _ = _oracle_run(run, b, wl.T)
        ws, wz, top1 = _compare(S[:, b], Z[:, b], So, Zo, tol)
        assert ws < tol and wz < tol, (b, ws, wz)
        agree.append(top1)
    if dtype == "bf16":
        assert np.mean(agree) >= TOP1_BF16, agree


def test_ring_slots_hold_retained_positions():
    """After t transitions every layer's ring holds the retained positions
    max(1, t-W+2)..t at slot (j-1) mod (W-1); compared with the oracle cache."""
    require_gpu()
    wl = synth.SMALL.with_(B=3)
    run = GpuRun(wl, T=40)
    run.init()
    nsteps = 37
    run.run(nsteps)
    for b in range(3):
        _, _, st, _ = _oracle_run(run, b, nsteps)
        for l in range(wl.L):
            rk = run.st.ring("k")[l, b].float().double().cpu().numpy()
            rv = run.st.ring("v")[l, b].float().double().cpu().numpy()
            assert sorted(st.hist[l]) == list(range(nsteps - wl.W + 2, nsteps + 1))
            for j, (k, v) in st.hist[l].items():
                sl = (j - 1) % (wl.W - 1)
                assert rel_l2(rk[sl], k) < TOL_BF16 and rel_l2(rv[sl], v) < TOL_BF16, (l, b, j)
