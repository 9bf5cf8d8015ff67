#!/usr/bin/env python3
"""Benchmark of the batched recurrent decoder state transition on one MI355X.

Workload (default ``reference_depth``): L_D=48, d=2048, 16 heads x 128,
W=256, G=1, SwiGLU 5504, vocab 32000, B=128 sequences, T=4096, bf16 weights
N(0, 0.02/sqrt(96)), bf16 encoder memory [B, T, d]. One step = one
``rlt_decoder_step`` over all B rows (merge, 48 decoder blocks, final norm,
vocabulary projection, argmax), captured once in a hipGraph and replayed.

The per-step cost is affine in the position t (the prefix cross-attention
reads t memory entries per row and layer), so the mean cost over a full run
t = 1..T equals the cost at t = T/2: the timed steps are centred on T/2,
starting from a synthetically pre-filled state (full SWA ring, pos set).

The K timed steps are run --repeats times (3) at the same positions and the
median is reported. Printed: one JSON line with the metric, the dominant
kernel's roofline (algorithmic bytes / live HIP-event duration), the CPU
oracle baseline and, for the default reference-depth run, the step at
batches 1, 8 and 16 (t ~ 40 and t ~ T/2) against the step's algorithmic
bytes at 8 TB/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def matrix_params(wl) -> int:
    d, F, V, L = wl.d, wl.F, wl.V, wl.L
    merge = 3 * d * d if wl.merge == "gated" else 2 * d * d
    return merge + L * (6 * d * d + 3 * d * F) + V * d


def step_bytes(wl, B: int, t: int, es: int) -> dict:
    """Algorithmic HBM bytes of one step over B rows at position t."""
    weights = matrix_params(wl) * es
    hist = min(t - 1, wl.W - 1)
    ring = wl.L * B * (hist * 2 * wl.d * es + (2 * wl.d * es if wl.W > 1 else 0))
    memory = wl.L * B * t * 2 * wl.d * es
    small = B * (wl.d * es + 2 * wl.d * 4)
    return dict(weights=weights, ring=ring, memory=memory, small=small,
                total=weights + ring + memory + small)


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, t0: int, budget_s: float, raw) -> dict:
    """The float32 oracle timed on this host on a bounded sample: one
    sequence, consecutive transitions (with the readout) from a pre-filled
    state at t0, first with the BLAS thread pool at its default size (all
    cores), then with one thread; each leg gets half the budget. As a
    cross-check of the affine cost model, one transition (all threads) at
    t = 1, W, T/4, T/2, 3T/4 and T: cost fitted as a + b t and averaged over a
    full run t = 1..T."""
    import numpy as np
    import synth
    from oracle import Config, Memory, Oracle, state_from_ring
    from threadpoolctl import threadpool_info, threadpool_limits

    def widen(a):
        return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)

    cfg = Config(L=wl.L, d=wl.d, H=wl.H, dh=wl.dh, W=wl.W, G=wl.G, F=wl.F, V=wl.V, merge=wl.merge,
                 alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos)
    orc = Oracle(cfg, {k: widen(v) for k, v in raw.items()}, dtype=np.float32)
    nT = max(t0 + 64, wl.T + 1)
    mem = Memory([widen(synth.make_memory(wl, "k", g, 0, 1, nT)[0]) for g in range(wl.G)],
                 [widen(synth.make_memory(wl, "v", g, 0, 1, nT)[0]) for g in range(wl.G)])
    rk = np.stack([widen(synth.make_ring_prefill(wl, "k", l, 0, 1)[0]) for l in range(wl.L)])
    rv = np.stack([widen(synth.make_ring_prefill(wl, "v", l, 0, 1)[0]) for l in range(wl.L)])
    s0 = widen(synth.normal(wl.seed, "s_prefill", (wl.d,)))
    E = widen(synth.make_e(wl, 0, 1, nT)[0])
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])

    def leg(budget):
        st = state_from_ring(cfg, s0, t0 - 1, rk, rv, dtype=np.float32)
        n = 0
        t_start = time.perf_counter()
        while True:
            st = orc.transition(st, E[st.pos], mem)
            orc.logits(st.s)
            n += 1
            el = time.perf_counter() - t_start
            if el >= budget or n >= 60:
                return n, el

    n_all, el_all = leg(budget_s / 2)
    with threadpool_limits(limits=1):
        n_one, el_one = leg(budget_s / 2)
    prof = {}
    for t in sorted({1, wl.W, wl.T // 4, wl.T // 2, 3 * wl.T // 4, wl.T}):
        st = state_from_ring(cfg, s0, t - 1, rk, rv, dtype=np.float32)
        t_start = time.perf_counter()
        st = orc.transition(st, E[st.pos], mem)
        orc.logits(st.s)
        prof[t] = time.perf_counter() - t_start
    ts = np.array(sorted(prof), dtype=np.float64)
    b, a = np.polyfit(ts, np.array([prof[t] for t in sorted(prof)]), 1)
    mean_cost = a + b * (wl.T + 1) / 2.0
    return {"value": n_all / el_all, "unit": "transitions/s", "cores": int(threads), "kind": "oracle",
            "value_1_thread": n_one / el_one, "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "t_profile_s": {int(t): round(v, 4) for t, v in prof.items()},
            "affine_fit_full_run_value": round(float(1.0 / mean_cost), 3),
            "sample": "float32 oracle, 1 sequence, transitions (incl. readout) from a pre-filled state at "
                      "t=%d: %d in %.1f s on %d BLAS threads, %d in %.1f s on 1 thread; plus one transition "
                      "at each of t=%s (all threads), fitted as a + b t over t = 1..%d"
                      % (t0, n_all, el_all, threads, n_one, el_one, ",".join(str(int(t)) for t in ts), wl.T)}


def measured_traffic(x_bytes: float):
    """HBM bytes per cross-attention launch from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary (calibrated on a plain copy), scaled to
    this launch's algorithmic bytes -- or None when the kernel source has
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "k_xattn_reference_depth_traffic.json")
    try:
        rec = json.load(open(path))
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest()[:16] != rec.get("sources_sha256_16"):
        return None
    return int(rec["traffic_over_algorithmic"] * x_bytes)


def small_batches(wl, raw, cfg, mk, mv, es: int, graph: bool, batches=(1, 8, 16), K: int = 20, Wu: int = 3) -> list:
    """The step at small batches (a context of exactly that many rows each),
    timed at t ~ 40 and t ~ T/2 from a pre-filled state, against the step's
    algorithmic bytes at 8 TB/s (the small-batch HBM target); rows use the
    first rows of the main run's memory."""
    import torch
    from stateful_sequence_model_amd import Decoder, DecoderState, _abi
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed + 1)
    res = []
    for B in batches:
        dec = Decoder(cfg, raw, max_rows=B, max_ctx=wl.T)
        st = DecoderState(cfg, B)
        for l in range(wl.L):
            st.ring("k")[l].normal_(generator=gen)
            st.ring("v")[l].normal_(generator=gen)
        mem_len = torch.full((B,), wl.T, dtype=torch.int32, device="cuda")
        mem = Decoder.memory(mk[:, :B], mv[:, :B], mem_len)
        e = torch.empty((B, wl.d), device="cuda", dtype=cfg.torch_dtype).normal_(generator=gen)
        rows = torch.arange(B, dtype=torch.int32, device="cuda")
        argmax = torch.empty(B, dtype=torch.int32, device="cuda")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for t_c in (40, wl.T // 2):
                st.s.normal_(generator=gen)
                st.pos.fill_(t_c - K // 2 - Wu)
                st.pending.fill_(-1)
                for _ in range(Wu):
                    _abi.check(dec.step(st, rows, e, mem, argmax=argmax, graph=graph), "rlt_decoder_step")
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record(stream)
                for _ in range(K):
                    _abi.check(dec.step(st, rows, e, mem, argmax=argmax, graph=graph), "rlt_decoder_step")
                ev1.record(stream)
                torch.cuda.synchronize()
                _abi.check(dec.sync_error(), "device error")
                ms = ev0.elapsed_time(ev1) / K
                t_mid = t_c - K // 2 + (K - 1) / 2.0
                sb = step_bytes(wl, B, int(round(t_mid)), es)["total"]
                gbs = sb / (ms / 1e3) / 1e9
                res.append({"batch": B, "t_mid": t_mid, "ms_per_step": round(ms, 4),
                            "transitions_per_s": round(B / (ms / 1e3), 1), "step_algorithmic_GBs": round(gbs, 1),
                            "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4)})
                log("small batch B=%d t~%d: %.3f ms/step, %.1f GB/s (%.1f%% of 8 TB/s)"
                    % (B, t_mid, ms, gbs, 100 * gbs / HBM_PEAK_GBS))
        dec.close()
        del dec, st
        torch.cuda.empty_cache()
    return res


def calibrate(torch, nbytes: int = 4 << 30, reps: int = 10) -> dict:
    """Achievable HBM rates on this device, and known-size launches for the
    counter calibration: a plain copy (read + write), a read-only reduction
    over nbytes of bf16, and the library's streaming read of the same nbytes
    with non-temporal 16-byte loads (the load of the attention kernels) and
    with plain ones."""
    from stateful_sequence_model_amd import _abi
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def stream_read(nt):
        _abi.check(_abi.lib().rlt_dbg_stream_read(src.data_ptr(), nbytes, nt, sink.data_ptr(), stream),
                   "rlt_dbg_stream_read")
    res = {}
    for name, fn, moved in (("copy", lambda: dst.copy_(src), 2 * nbytes),
                            ("read_sum", lambda: src.sum(dtype=torch.float32), nbytes),
                            ("stream_read_nt", lambda: stream_read(1), nbytes),
                            ("stream_read", lambda: stream_read(0), nbytes)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name + "_GBs"] = round(moved * reps / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    # matrix cores: independent chains of the bf16 32x32x16 instruction
    blocks, iters = 1024, 20000
    flops = 4 * 4 * 32768 * iters * blocks

    def mfma():
        _abi.check(_abi.lib().rlt_dbg_mfma_loop(blocks, iters, sink.data_ptr(), stream), "rlt_dbg_mfma_loop")
    mfma()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        mfma()
    e1.record()
    torch.cuda.synchronize()
    res["mfma_bf16_TFLOPs"] = round(flops * 5 / (e0.elapsed_time(e1) / 1e3) / 1e12, 1)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="preset (default: reference_depth; small_batched for --mode backward)")
    ap.add_argument("--batch", type=int, default=0, help="override B")
    ap.add_argument("--t-center", type=int, default=0, help="centre of the timed positions (default T/2)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--repeats", type=int, default=3,
                    help="timed runs of --steps steps each (same positions); the median is reported")
    ap.add_argument("--no-small-batch", action="store_true",
                    help="skip the small-batch lines (batches 1, 8, 16 at t ~ 40 and t ~ T/2) that the "
                         "default reference-depth run adds")
    ap.add_argument("--calibrate", action="store_true",
                    help="also time a plain 4 GiB device copy and read-only sum (achievable HBM rates)")
    ap.add_argument("--launch", action="append", default=[], metavar="FIELD=VALUE",
                    help="launch option of the context (rlt_dbg_launch field, for tuning sweeps)")
    ap.add_argument("--mode", choices=("step", "memory_prefill", "backward", "replay", "shapes"), default="step",
                    help="step: the decoder transition (default); memory_prefill: token-parallel "
                         "construction of the encoder memory of the whole batch; backward: full-BPTT "
                         "replay backward of the whole batch; replay: current-policy replay from H_0 of "
                         "ragged sequences (default preset ragged_rl_replay, lengths capped by "
                         "--replay-max-len); shapes: the step with each product tile shape forced "
                         "in turn (rlt_dbg_product_shape), against the library's own choice")
    ap.add_argument("--replay-max-len", type=int, default=1024,
                    help="replay mode: upper end of the uniform length draw (the preset's lower end kept)")
    ap.add_argument("--replay-waves", type=int, default=1,
                    help="replay mode: the sequences (longest first) replayed as this many calls of "
                         "B / waves sequences each, whose dense memory [G][B/waves][T][d] is reused "
                         "(the preset's full draw, U[64, 8192] over 256 sequences, needs 309 GB as one "
                         "buffer: two waves fit one GPU); timed once, with graphs")
    args = ap.parse_args()

    if args.gpus != 1:
        log("bench.py measures one GPU only: the library has no multi-GPU path "
            "(sequences would shard across GPUs with no per-step exchange). Use --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    from stateful_sequence_model_amd import Decoder, DecoderState, ModelConfig, _abi, to_device

    default = {"backward": "small_batched", "replay": "ragged_rl_replay"}.get(args.mode, "reference_depth")
    wl = synth.PRESETS[args.workload or default]
    if args.batch:
        wl = wl.with_(B=args.batch)
    if args.mode == "memory_prefill":
        return bench_memory_prefill(args, wl)
    if args.mode == "backward":
        return bench_backward(args, wl)
    if args.mode == "replay":
        return bench_replay(args, wl)
    if args.mode == "shapes":
        return bench_shapes(args, wl)
    B, T = wl.B, wl.T
    es = 2 if wl.dtype == "bf16" else 4
    K, Wu = args.steps, args.warmup
    t_center = args.t_center or T // 2
    pos0 = max(0, t_center - K // 2 - Wu)
    assert pos0 + Wu + K <= T, "timed positions exceed T"
    torch.cuda.set_device(0)
    dev = "cuda"

    tg = time.perf_counter()
    raw = synth.make_weights(wl)
    log("weights generated in %.1fs" % (time.perf_counter() - tg))
    cfg = ModelConfig(L=wl.L, d=wl.d, H=wl.H, dh=wl.dh, W=wl.W, G=wl.G, F=wl.F, V=wl.V, dtype=wl.dtype,
                      merge=wl.merge, alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos)
    launch = {k: int(v) for k, v in (a.split("=", 1) for a in args.launch)}
    dec = Decoder(cfg, raw, max_rows=B, max_ctx=T, launch=launch or None)
    st = DecoderState(cfg, B)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    tdt = cfg.torch_dtype
    # encoder memory [G, B, T, d] and a pre-filled state (values N(0,1)),
    # generated in place: no float32 temporaries. (The cross-attention
    # kernel streams the memory at ~6.6 TB/s from freshly allocated buffers
    # but at ~6.0 TB/s when the buffers land in memory fragmented by large
    # freed temporaries.)
    mk = torch.empty((wl.G, B, T, wl.d), device=dev, dtype=tdt).normal_(generator=gen)
    mv = torch.empty((wl.G, B, T, wl.d), device=dev, dtype=tdt).normal_(generator=gen)
    for l in range(wl.L):
        st.ring("k")[l].normal_(generator=gen)
        st.ring("v")[l].normal_(generator=gen)
    e = torch.empty((B, wl.d), device=dev, dtype=tdt).normal_(generator=gen)
    mem_len = torch.full((B,), T, dtype=torch.int32, device=dev)
    mem = Decoder.memory(mk, mv, mem_len)
    rows = torch.arange(B, dtype=torch.int32, device=dev)
    argmax = torch.empty(B, dtype=torch.int32, device=dev)

    def reset(pos):
        st.s.copy_(torch.randn(st.s.shape, generator=gen, device=dev))
        st.pos.fill_(pos)
        st.pending.fill_(-1)

    stream = torch.cuda.Stream()
    graph = not args.no_graph
    with torch.cuda.stream(stream):
        reset(pos0)
        torch.cuda.synchronize()
        for _ in range(Wu):
            _abi.check(dec.step(st, rows, e, mem, argmax=argmax, graph=graph), "rlt_decoder_step")
        torch.cuda.synchronize()
        t_first = int(st.pos[0].item()) + 1
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        runs = []
        for r in range(max(1, args.repeats)):
            if r:  # the same positions again
                reset(t_first - 1)
                torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(K):
                _abi.check(dec.step(st, rows, e, mem, argmax=argmax, graph=graph), "rlt_decoder_step")
            ev1.record(stream)
            torch.cuda.synchronize()
            runs.append(ev0.elapsed_time(ev1))
            _abi.check(dec.sync_error(), "device error")
            assert int(st.pos[0].item()) == t_first + K - 1
        ms = sorted(runs)[len(runs) // 2]
        # live per-kernel timing (direct launches, same positions as the timed steps)
        P = max(1, min(args.profile_steps, K))
        reset(t_first - 1)
        torch.cuda.synchronize()
        _abi.check(_abi.rlt_dbg_profile(dec.ctx, 1), "profile")
        for _ in range(P):
            _abi.check(dec.step(st, rows, e, mem, argmax=argmax, graph=False), "rlt_decoder_step")
        torch.cuda.synchronize()
        prof = {name: _abi.rlt_dbg_profile_read(dec.ctx, i) for i, name in enumerate(_abi.PROF_NAMES)}
        _abi.check(_abi.rlt_dbg_profile(dec.ctx, 0), "profile")

    ms_step = ms / K
    t_mid = t_first + (K - 1) / 2.0
    value = B * K / (ms / 1e3)
    sb = step_bytes(wl, B, int(round(t_mid)), es)
    # dominant kernel: prefix cross-attention partials; unit = one memory
    # position of one row (K and V, 2*d elements)
    x_ms, x_n = prof["xattn"]
    x_avg_ms = x_ms / max(x_n, 1)
    t_prof_mid = t_first + (P - 1) / 2.0
    rows_per_launch = B * wl.L * P / max(x_n, 1)   # B, or B/2 when a call runs as two streams
    x_bytes = rows_per_launch * t_prof_mid * 2 * wl.d * es
    breakdown = {k: round(v[0] / P, 4) for k, v in prof.items()}
    log("ms/step %.3f  transitions/s %.1f  step algorithmic GB/s %.1f (%.1f%% of 8 TB/s)" %
        (ms_step, value, sb["total"] / (ms_step / 1e3) / 1e9, 100 * sb["total"] / (ms_step / 1e3) / 8e12))
    log("per-step kernel ms (direct launches):", breakdown)
    f_ms, f_n = prof["fused"]
    if x_n == 0 and f_n > 0:
        # small call: the whole transition (all but the readout) is one
        # persistent kernel; unit = the step's algorithmic bytes
        f_avg_ms = f_ms / f_n
        f_bytes = step_bytes(wl, B, int(round(t_prof_mid)), es)["total"]
        achieved = f_bytes / (f_avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": "k_fused (persistent step: merge, %d blocks, final norm, logits)" % wl.L,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "avg_launch_ms": round(f_avg_ms, 5), "algorithmic_bytes_per_launch": int(f_bytes)}
        log("fused: %d launches, avg %.4f ms, %.1f GB/s" % (f_n, f_avg_ms, achieved))
    else:
        achieved = x_bytes / (x_avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": "k_xattn (prefix cross-attention)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(x_bytes),
                "avg_launch_ms": round(x_avg_ms, 5), "algorithmic_bytes_per_launch": int(x_bytes)}
        log("xattn: %d launches, avg %.4f ms, %.1f GB/s" % (x_n, x_avg_ms, achieved))

    out = {
        "metric": "decoder state-transitions/sec (seq*token) at L_D=%d" % wl.L,
        "value": round(value, 2),
        "unit": "transitions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "L_D": wl.L, "d": wl.d, "heads": "%dx%d" % (wl.H, wl.dh), "W": wl.W,
                   "G": wl.G, "ffn": wl.F, "vocab": wl.V, "batch": B, "T": T,
                   "timed_positions": [t_first, t_first + K - 1], "hipgraph": graph,
                   **({"launch": launch} if launch else {})},
        "roofline": roof,
        "step_roofline": {"algorithmic_bytes": int(sb["total"]),
                          "achieved_GBs": round(sb["total"] / (ms_step / 1e3) / 1e9, 1),
                          "frac": round(sb["total"] / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                          "bytes_split": {k: int(v) for k, v in sb.items() if k != "total"}},
        "kernel_ms_per_step": breakdown,
        "timing": {"repeats": len(runs), "statistic": "median",
                   "ms_per_step_runs": [round(x / K, 4) for x in runs]},
    }
    if wl.name == "reference_depth" and not args.batch and not args.t_center and not args.no_small_batch:
        out["small_batch"] = small_batches(wl, raw, cfg, mk, mv, es, graph)
    if args.calibrate:
        out["calibration"] = calibrate(torch)
    if not args.no_cpu_baseline:
        del mk, mv
        torch.cuda.empty_cache()
        log("timing the CPU oracle (%.0f s budget)..." % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(wl, t_center, args.cpu_seconds, raw)
    print(json.dumps(out), flush=True)


def bench_memory_prefill(args, wl):
    """Token-parallel memory construction [eq. (2.2)] of all B x T entries of
    every group: one rlt_memory_prefill call per timed step. Dominated by the
    [B*T, d] x [d, 2d] products per group (MFMA-bound), reported against
    the dense bf16 peak."""
    import numpy as np
    import torch
    import synth
    from stateful_sequence_model_amd import Decoder, ModelConfig, _abi

    B, T, d, G = wl.B, wl.T, wl.d, wl.G
    es = 2 if wl.dtype == "bf16" else 4
    torch.cuda.set_device(0)
    cfg = ModelConfig(L=wl.L, d=wl.d, H=wl.H, dh=wl.dh, W=wl.W, G=wl.G, F=wl.F, V=wl.V, dtype=wl.dtype,
                      merge=wl.merge, alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos)
    # the decoder weights are not used by the memory maps: with one memory
    # group a one-layer context of the same widths suffices
    ctx_wl = wl.with_(L=1) if G == 1 else wl
    ctx_cfg = ModelConfig(**{**cfg.__dict__, "L": ctx_wl.L})
    launch = {k: int(v) for k, v in (a.split("=", 1) for a in args.launch)}
    dec = Decoder(ctx_cfg, synth.make_weights(ctx_wl), max_rows=128, max_ctx=T, launch=launch or None)
    mw = dec.memory_weights(synth.make_memory_weights(wl))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    tdt = cfg.torch_dtype
    e = torch.randn((B, T, d), generator=gen, device="cuda").to(tdt)
    K = torch.empty((G, B, T, d), dtype=tdt, device="cuda")
    V = torch.empty_like(K)
    mem_len = torch.zeros(B, dtype=torch.int32, device="cuda")
    mem = Decoder.memory(K, V, mem_len)
    lens = np.full(B, T, dtype=np.int32)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            _abi.check(dec.memory_prefill(mw, mem, T, lens, e), "rlt_memory_prefill")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            _abi.check(dec.memory_prefill(mw, mem, T, lens, e), "rlt_memory_prefill")
        e1.record(stream)
        torch.cuda.synchronize()
    _abi.check(dec.sync_error(), "device error")
    ms = e0.elapsed_time(e1) / args.steps
    entries = B * T
    flops = 2.0 * entries * d * (2 * d) * G
    tflops = flops / (ms / 1e3) / 1e12
    peak = 2500.0 if wl.dtype == "bf16" else 157.3
    moved = entries * d * es * (1 + 2 * G) + G * 2 * d * d * es  # e read, K and V written, weights read
    log("memory prefill: %.3f ms per call, %.1f M entries/s, %.1f TFLOP/s (%.1f%% of the dense peak)" %
        (ms, entries / (ms / 1e3) / 1e6, tflops, 100 * tflops / peak))
    print(json.dumps({
        "metric": "encoder-memory entries/sec (token-parallel prefill, all %d groups)" % G,
        "value": round(entries / (ms / 1e3), 1), "unit": "entries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name + " memory prefill", "batch": B, "T": T, "d": d, "G": G},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None,
                     "algorithmic_flops_per_call": flops, "hbm_bytes_min_per_call": int(moved)},
    }), flush=True)


# product tile shapes of the sweep: (rb, cb, lt, pf, pre) as rlt_dbg_product_shape
# takes them; rb = 0 is the library's own choice
SWEEP_SHAPES = [(0, 1, 0, 2, -1), (1, 1, 0, 2, -1), (1, 1, 0, 3, -1), (1, 2, 0, 2, -1), (2, 1, 0, 2, -1),
                (1, 2, 1, 1, 0), (1, 2, 2, 1, 0), (1, 2, 4, 1, 0), (1, 2, 8, 1, 0),
                (1, 4, 1, 1, 0), (1, 4, 2, 1, 0), (1, 4, 4, 1, 0), (1, 4, 8, 1, 0)]


def bench_shapes(args, wl):
    """The decoder step (direct launches, --steps steps after --warmup) with
    each operand-order product shape forced in turn: ms per step and the
    products' share (HIP events per launch, rlt_dbg_profile). Run under
    rocprofv3 --kernel-trace for the per-product durations; the shapes run in
    the order of SWEEP_SHAPES."""
    import torch
    import synth
    from stateful_sequence_model_amd import Decoder, DecoderState, ModelConfig, _abi
    B, T = wl.B, wl.T
    t0 = args.t_center or T // 2
    K, Wu = args.steps, args.warmup
    raw = synth.make_weights(wl)
    cfg = ModelConfig(L=wl.L, d=wl.d, H=wl.H, dh=wl.dh, W=wl.W, G=wl.G, F=wl.F, V=wl.V, dtype=wl.dtype,
                      merge=wl.merge, alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos)
    dec = Decoder(cfg, raw, max_rows=B, max_ctx=T)
    st = DecoderState(cfg, B)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    tdt = cfg.torch_dtype
    mk = torch.empty((wl.G, B, T, wl.d), device="cuda", dtype=tdt).normal_(generator=gen)
    mv = torch.empty_like(mk).normal_(generator=gen)
    for l in range(wl.L):
        st.ring("k")[l].normal_(generator=gen)
        st.ring("v")[l].normal_(generator=gen)
    e = torch.empty((B, wl.d), device="cuda", dtype=tdt).normal_(generator=gen)
    mem_len = torch.full((B,), T, dtype=torch.int32, device="cuda")
    mem = Decoder.memory(mk, mv, mem_len)
    rows = torch.arange(B, dtype=torch.int32, device="cuda")
    argmax = torch.empty(B, dtype=torch.int32, device="cuda")
    res = []
    for sh in SWEEP_SHAPES:
        _abi.check(_abi.lib().rlt_dbg_product_shape(dec.ctx, *sh), "rlt_dbg_product_shape")
        st.s.normal_(generator=gen)
        st.pos.fill_(max(0, t0 - K // 2 - Wu))
        st.pending.fill_(-1)
        for _ in range(Wu):
            _abi.check(dec.step(st, rows, e, mem, argmax=argmax), "rlt_decoder_step")
        torch.cuda.synchronize()
        _abi.check(_abi.rlt_dbg_profile(dec.ctx, 1), "profile")
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(K):
            _abi.check(dec.step(st, rows, e, mem, argmax=argmax), "rlt_decoder_step")
        ev1.record()
        torch.cuda.synchronize()
        g_ms, g_n = _abi.rlt_dbg_profile_read(dec.ctx, _abi.PROF_NAMES.index("gemm"))
        _abi.check(_abi.rlt_dbg_profile(dec.ctx, 0), "profile")
        ms = ev0.elapsed_time(ev1) / K
        res.append({"rb": sh[0], "cb": sh[1], "lt": sh[2], "pf": sh[3], "pre": sh[4],
                    "ms_per_step": round(ms, 4), "products_ms_per_step": round(g_ms / K, 4)})
        log("shape rb=%d cb=%d lt=%d pf=%d pre=%d: %.3f ms/step, products %.3f ms (direct launches)"
            % (sh + (ms, g_ms / K)))
    _abi.check(dec.sync_error(), "device error")
    print(json.dumps({"mode": "shapes", "workload": wl.name, "batch": B, "t": t0, "steps": K,
                      "warmup": Wu, "shapes": res}), flush=True)


def bench_replay(args, wl):
    """Current-policy replay from H_0 ("Recurrent Looped Transformer" App. A.4,
    §4.1: ready transitions of uneven length batched tick by tick) of B ragged
    sequences: one rlt_replay_sequence call per timed step, every position from
    the split scored. The preset's length draw U[len_lo, len_hi] is capped at
    --replay-max-len (the prefix cross-attention makes a sequence's cost grow
    with the square of its length: the uncapped draw is hours of GPU time per
    call); value = transitions (sum of len - 1) per second. Timed twice: with
    the runs of ticks of one active set captured as graphs (the default on a
    stream) and with every tick launched directly."""
    import numpy as np
    import torch
    import synth
    from stateful_sequence_model_amd import Decoder, DecoderState, ModelConfig, _abi

    wl = wl.with_(len_hi=min(wl.len_hi, args.replay_max_len)) if wl.ragged else wl
    lens, splits = synth.make_lengths(wl)
    if args.replay_waves > 1:
        return bench_replay_waves(args, wl, lens, splits)
    B, T, d, G = wl.B, int(lens.max()), wl.d, wl.G
    steps = max(1, min(args.steps, 3))
    torch.cuda.set_device(0)
    raw = synth.make_weights(wl)
    cfg = ModelConfig(L=wl.L, d=d, H=wl.H, dh=wl.dh, W=wl.W, G=G, F=wl.F, V=wl.V, dtype=wl.dtype,
                      merge=wl.merge, alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    tdt = cfg.torch_dtype
    e = torch.empty((B, T, d), device="cuda", dtype=tdt).normal_(generator=gen)
    mk = torch.empty((G, B, T, d), device="cuda", dtype=tdt).normal_(generator=gen)
    mv = torch.empty((G, B, T, d), device="cuda", dtype=tdt).normal_(generator=gen)
    mem_len = torch.from_numpy(lens).cuda()  # kept alive: the memory struct holds its pointer
    mem = Decoder.memory(mk, mv, mem_len)
    tokens = torch.randint(0, wl.V, (B, T), generator=gen, device="cuda", dtype=torch.int32)
    logp = torch.empty((B, T), device="cuda")
    trans = int((lens - 1).sum())
    stream = torch.cuda.Stream()
    res = {}
    for label, gmin in (("graphs", 0), ("direct", -1)):
        dec = Decoder(cfg, raw, max_rows=B, max_ctx=T, launch={"replay_graph_min": gmin})
        st = DecoderState(cfg, B)
        with torch.cuda.stream(stream):
            for _ in range(max(1, args.warmup if args.warmup < 2 else 1)):
                _abi.check(dec.replay(st, lens, splits, e, mem, tokens, logp, stream=stream.cuda_stream), "replay")
            stream.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                _abi.check(dec.replay(st, lens, splits, e, mem, tokens, logp, stream=stream.cuda_stream), "replay")
            stream.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / steps
        _abi.check(dec.sync_error(), "device error")
        res[label] = ms
        log("replay (%s): %.1f ms per call, %d transitions, %.1f transitions/s" % (label, ms, trans, trans / (ms / 1e3)))
        dec.close()
        del st
    ms = res["graphs"]
    out = {
        "metric": "replay transitions/sec (ragged, from H_0, seq*token)",
        "value": round(trans / (ms / 1e3), 1), "unit": "transitions/s", "n_gpus": 1, "steps": steps,
        "warmup": 1, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name + " replay", "L_D": wl.L, "d": d, "heads": "%dx%d" % (wl.H, wl.dh),
                   "W": wl.W, "G": G, "batch": B, "lengths": "U[%d, %d]" % (wl.len_lo, wl.len_hi),
                   "max_len": T, "transitions": trans},
        "direct_launch_ms_per_call": round(res["direct"], 3),
        "graph_speedup": round(res["direct"] / ms, 3),
    }
    print(json.dumps(out), flush=True)


def bench_replay_waves(args, wl, lens, splits):
    """The replay of bench_replay at the preset's own length draw: sequences
    sorted longest first and replayed in --replay-waves calls of B / waves
    sequences (each call batches its own ragged set tick by tick, as the whole
    batch would), through one context and one memory buffer sized for the
    longest wave; value = all calls' transitions / their summed time."""
    import numpy as np
    import torch
    import synth
    from stateful_sequence_model_amd import Decoder, DecoderState, ModelConfig, _abi

    nw = args.replay_waves
    order = np.argsort(-lens, kind="stable")
    B, d, G = wl.B, wl.d, wl.G
    Bw = (B + nw - 1) // nw
    T = int(lens.max())
    torch.cuda.set_device(0)
    raw = synth.make_weights(wl)
    cfg = ModelConfig(L=wl.L, d=d, H=wl.H, dh=wl.dh, W=wl.W, G=G, F=wl.F, V=wl.V, dtype=wl.dtype,
                      merge=wl.merge, alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    tdt = cfg.torch_dtype
    log("replay waves: %d x %d sequences, T = %d, memory %.1f GB" % (nw, Bw, T, 2 * G * Bw * T * d * 2 / 1e9))
    e = torch.empty((Bw, T, d), device="cuda", dtype=tdt).normal_(generator=gen)
    mk = torch.empty((G, Bw, T, d), device="cuda", dtype=tdt)
    mv = torch.empty((G, Bw, T, d), device="cuda", dtype=tdt)
    for g in range(G):  # per group, so that no temporary of the whole buffer is needed
        mk[g].normal_(generator=gen)
        mv[g].normal_(generator=gen)
    log("memory filled")
    tokens = torch.randint(0, wl.V, (Bw, T), generator=gen, device="cuda", dtype=torch.int32)
    logp = torch.empty((Bw, T), device="cuda")
    dec = Decoder(cfg, raw, max_rows=Bw, max_ctx=T)
    st = DecoderState(cfg, Bw)
    stream = torch.cuda.Stream()
    total_ms, trans, per_wave, alg = 0.0, 0, [], 0.0
    with torch.cuda.stream(stream):
        for w in range(nw):
            idx = order[w * Bw:(w + 1) * Bw]
            lw, sw = np.ascontiguousarray(lens[idx]), np.ascontiguousarray(splits[idx])
            mem_len = torch.from_numpy(lw).cuda()  # kept alive: the memory struct holds its pointer
            # the whole buffer's strides (a group spans Bw rows); the wave uses its first rows
            mem = _abi.rlt_memory(mk.data_ptr(), mv.data_ptr(), Bw * T * d, T * d, d, mem_len.data_ptr())
            stream.synchronize()
            t0 = time.perf_counter()
            _abi.check(dec.replay(st, lw, sw, e[:len(idx)], mem, tokens[:len(idx)], logp[:len(idx)],
                                  stream=stream.cuda_stream), "replay")
            stream.synchronize()
            ms = (time.perf_counter() - t0) * 1e3
            tw = int((lw - 1).sum())
            # algorithmic bytes: the weights once per tick, each active row's
            # retained window and memory prefix once per layer
            wb = 0.0
            for t in range(1, int(lw.max())):
                n = int((lw - 1 >= t).sum())
                wb += matrix_params(wl) * 2 + n * wl.L * (min(t - 1, wl.W - 1) + 1 + t) * 2 * d * 2
            per_wave.append({"sequences": int(len(idx)), "lengths": [int(lw.min()), int(lw.max())],
                             "transitions": tw, "ms": round(ms, 1), "algorithmic_bytes": int(wb),
                             "achieved_GBs": round(wb / (ms / 1e3) / 1e9, 1)})
            alg += wb
            log("wave %d: %d sequences, lengths %d..%d, %d transitions in %.1f ms (%.1f transitions/s)"
                % (w, len(idx), lw.min(), lw.max(), tw, ms, tw / (ms / 1e3)))
            total_ms += ms
            trans += tw
    _abi.check(dec.sync_error(), "device error")
    dec.close()
    out = {
        "metric": "replay transitions/sec (ragged, from H_0, seq*token)",
        "value": round(trans / (total_ms / 1e3), 1), "unit": "transitions/s", "n_gpus": 1, "steps": 1,
        "warmup": 0, "ms_per_step": round(total_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name + " replay", "L_D": wl.L, "d": d, "heads": "%dx%d" % (wl.H, wl.dh),
                   "W": wl.W, "G": G, "batch": B, "waves": nw, "lengths": "U[%d, %d]" % (wl.len_lo, wl.len_hi),
                   "max_len": T, "transitions": trans},
        "waves": per_wave,
        "step_roofline": {"algorithmic_bytes": int(alg), "achieved_GBs": round(alg / (total_ms / 1e3) / 1e9, 1),
                          "frac": round(alg / (total_ms / 1e3) / (HBM_PEAK_GBS * 1e9), 4)},
    }
    print(json.dumps(out), flush=True)


def bench_backward(args, wl):
    """Full-BPTT replay backward [RLT §5.4, App. B] of B sequences of T
    tokens (every position scored, loss weights N(0,1)): one
    rlt_replay_backward call per timed step, gradients of every parameter,
    e_t and the memory. The kernels compute in float32 on the vector ALUs
    (no matrix cores), so the call's algorithmic rate is reported against the
    fp32 vector peak."""
    import numpy as np
    import torch
    import synth
    from stateful_sequence_model_amd import Decoder, ModelConfig, _abi

    B, T, d, G, L = wl.B, wl.T, wl.d, wl.G, wl.L
    steps = min(args.steps, 5)
    torch.cuda.set_device(0)
    raw = synth.make_weights(wl)
    cfg = ModelConfig(L=L, d=d, H=wl.H, dh=wl.dh, W=wl.W, G=G, F=wl.F, V=wl.V, dtype=wl.dtype,
                      merge=wl.merge, alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos)
    launch = {k: int(v) for k, v in (a.split("=", 1) for a in args.launch)}
    dec = Decoder(cfg, raw, max_rows=B, max_ctx=T, launch=launch or None)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    tdt = cfg.torch_dtype
    e = torch.randn((B, T, d), generator=gen, device="cuda").to(tdt)
    mk = torch.randn((G, B, T, d), generator=gen, device="cuda").to(tdt)
    mv = torch.randn((G, B, T, d), generator=gen, device="cuda").to(tdt)
    mem = Decoder.memory(mk, mv, torch.full((B,), T, dtype=torch.int32, device="cuda"))
    tokens = torch.randint(0, wl.V, (B, T), generator=gen, device="cuda", dtype=torch.int32)
    w = torch.randn((B, T), generator=gen, device="cuda")
    de = torch.zeros((B, T, d), device="cuda")
    dmk = torch.zeros((G, B, T, d), device="cuda")
    dmv = torch.zeros((G, B, T, d), device="cuda")
    grads = dec.grad_buffers()
    lens = np.full(B, T, dtype=np.int32)
    splits = np.ones(B, dtype=np.int32)

    def call():
        _abi.check(dec.replay_backward(grads, lens, splits, e, mem, tokens, w, de=de, dmem_k=dmk, dmem_v=dmv),
                   "rlt_replay_backward")

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    trans = B * (T - 1)
    # algorithmic flops: forward products 2P, backward 4P (inputs and weights)
    # per transition, P = decoder matrices + readout; attention forward
    # 4 d (window + prefix) per layer, backward twice that
    P = matrix_params(wl) + wl.V * d
    att = sum(min(t, wl.W) + t for t in range(1, T))
    flops = 6.0 * P * trans + 12.0 * d * L * att * B
    tflops = flops / (ms / 1e3) / 1e12
    peak = 157.3
    log("replay backward: %.1f ms per call (%d transitions), %.1f transitions/s, %.2f TFLOP/s" %
        (ms, trans, trans / (ms / 1e3), tflops))
    out = {
        "metric": "replay-backward transitions/sec (full BPTT, seq*token)",
        "value": round(trans / (ms / 1e3), 1), "unit": "transitions/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name + " replay backward", "L_D": L, "d": d, "batch": B, "T": T, "W": wl.W,
                   "G": G, "params": wl.dtype, **({"launch": launch} if launch else {})},
        "roofline": {"bound": "alu", "achieved": round(tflops, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 5), "traffic": None, "scope": "whole call (fp32 vector ALU)",
                     "algorithmic_flops_per_call": flops},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(wl, raw, budget_s=args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_backward(wl, raw, budget_s: float) -> dict:
    """The gradient oracle (float64 autograd twin) on one sequence, growing
    its length until the budget is spent."""
    import numpy as np
    import torch
    from oracle.rlt_oracle import Config
    from oracle.rlt_grad import replay_grads

    def widen(a):
        if a.dtype == np.uint16:
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.astype(np.float64)

    cfg = Config(L=wl.L, d=wl.d, H=wl.H, dh=wl.dh, W=wl.W, G=wl.G, F=wl.F, V=wl.V, merge=wl.merge,
                 alpha=wl.alpha, eps=wl.eps, rope_theta=wl.rope_theta, pos=wl.pos)
    w = {k: widen(v) for k, v in raw.items()}
    rng = np.random.default_rng(1)
    n, spent, done = 4, 0.0, 0
    while spent < budget_s and n <= wl.T:
        sq = dict(E=rng.standard_normal((n, wl.d)), mem_k=[rng.standard_normal((n, wl.d)) for _ in range(wl.G)],
                  mem_v=[rng.standard_normal((n, wl.d)) for _ in range(wl.G)], tokens=rng.integers(0, wl.V, n),
                  length=n, split=1, w=rng.standard_normal(n))
        t0 = time.perf_counter()
        replay_grads(cfg, w, [sq])
        spent += time.perf_counter() - t0
        done += n - 1
        n *= 2
    return {"value": round(done / spent, 2), "unit": "transitions/s", "cores": torch.get_num_threads(),
            "kind": "oracle", "sample": "float64 autograd twin, single sequences of 4, 8, ... tokens "
            "(%d transitions, %.1f s)" % (done, spent)}


if __name__ == "__main__":
    main()
