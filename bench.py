#!/usr/bin/env python3
"""Benchmark of the hybrid attention chunk step (Hybrid Forcing) on one MI355X.

Workload: one attention layer at the 832x480 shape -- 12 heads x 128, 1560 tokens per
latent frame (30x52 patches), a chunk of 3 frames (4680 queries) attending to a 6-frame
window (9360 keys) in 64x64 blocks with 25% of the key blocks kept (37 of 147), and a
linear state that starts from 18 absorbed frames.  A timed step is one hf_hybrid_step
with commit: append the chunk to the KV ring, block select, block-sparse attention with
the fused linear readout, and absorption of the 3 evicted frames into the state.

Inputs are seeded synthetic bf16 activations (rank-8 smooth spatial field + noise per
head, see hybrid_sparse_linear_hf_amd/synth.py); 12 distinct chunks (~518 MB of Q/K/V)
rotate through the steps so that the 256 MB last-level cache cannot hold them.

Prints ONE JSON line.  value = effective TFLOP/s on kept blocks over the whole step
(4*D*sum_i |Q_i| * sum_{j kept} |K_j|, exact from each step's block indices).
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix-core peak (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak
ROOT = Path(__file__).resolve().parent
ATTN_SOURCES = [ROOT / "hybrid_sparse_linear_hf_amd" / "csrc" / n for n in ("sparse_attn.hip", "hf_internal.h")]
ATTN_PMC_SUMMARY = ROOT / "profiles" / "hybrid_step_832x480_layer_hbm_traffic.md"
METRIC = "hybrid-attn chunk step ms + TFLOP/s on kept blocks (832x480 shape, 1 GPU)"
PHASE_STEPS = 20               # untimed steps after the timed region that record the phase events


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime (recorded inside hf_hybrid_step)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.rt.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        self.rt.hipEventSynchronize(ctypes.c_void_p(b))
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def kept_flops(idx: np.ndarray, Nq: int, Nk: int, bq: int, bk: int, D: int) -> float:
    """4*D*sum over (b,h,i) of |Q_i| * sum_{j in idx} |K_j|."""
    nqb = idx.shape[2]
    qsz = np.minimum(bq, Nq - np.arange(nqb) * bq).astype(np.float64)
    ksz = np.minimum(bk, Nk - idx.astype(np.int64) * bk).astype(np.float64)
    return float(4.0 * D * np.sum(qsz[None, None, :] * ksz.sum(axis=-1)))


def cpu_baseline(cfg, sample_heads: int, min_seconds: float):
    """The fp64 oracle (test infrastructure) timed on the host on a bounded sample: the full
    step (select, sparse attention, readout, absorb of the evicted frames) on `sample_heads`
    heads of the same workload, repeated until `min_seconds` of wall time have passed."""
    import oracle
    from hybrid_sparse_linear_hf_amd import synth

    heads = list(range(sample_heads))
    inp = synth.field_step_inputs(cfg, heads=heads)
    f64 = synth.f64_from_bf16_bits
    Q, K, V = f64(inp["q"]), f64(inp["k_win"]), f64(inp["v_win"])
    S0, z0 = oracle.absorb(f64(inp["k_ev"]), f64(inp["v_ev"]))
    Kev, Vev = K[:, :, :cfg.C * cfg.T], V[:, :, :cfg.C * cfg.T]   # the frames this step evicts
    k = cfg.top_k()
    reps, fl = 0, 0.0
    t0 = time.perf_counter()
    while True:
        S, z = S0.copy(), z0.copy()
        out, idx, _ = oracle.hybrid_step(Q, K, V, S, z, cfg.bq, cfg.bk, k)
        oracle.absorb(Kev, Vev, S, z)
        fl += kept_flops(idx, cfg.Nq, cfg.Nk, cfg.bq, cfg.bk, cfg.D)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    # one step of one head on a single thread
    threads = oracle.num_threads()
    one = {key: val[:, :1] for key, val in (("Q", Q), ("K", K), ("V", V), ("S", S0), ("z", z0))}
    oracle.set_num_threads(1)
    try:
        t1 = time.perf_counter()
        S1, z1 = one["S"].copy(), one["z"].copy()
        oracle.hybrid_step(one["Q"], one["K"], one["V"], S1, z1, cfg.bq, cfg.bk, k)
        oracle.absorb(one["K"][:, :, :cfg.C * cfg.T], one["V"][:, :, :cfg.C * cfg.T], S1, z1)
        t_one = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(threads)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full steps (select + sparse attention + readout + absorb of {cfg.C} "
                      f"frames) on {sample_heads} of {cfg.H} heads of the {cfg.name} workload, fp64, "
                      f"{dt:.1f} s wall, {dt / reps * 1e3:.0f} ms per step",
            "cpu_model": cpu_model(), "one_thread_ms_per_head_step": round(t_one * 1e3, 1),
            "ms_per_step": dt / reps * 1e3}


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_peaks(torch, dev):
    """Reference rates measured on this GPU: a large bf16 GEMM through torch (hipBLASLt) for
    the matrix cores, and a 1 GiB device copy (bytes read + written) for HBM."""
    n = 8192
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm = 2 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    src = torch.empty(1 << 28, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(3):
        dst.copy_(src)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy = 2 * src.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {"bf16_gemm_tflops": round(gemm, 1), "gemm": "torch.matmul bf16 8192x8192x8192 (hipBLASLt), 10 reps",
            "copy_gbs": round(copy, 1), "copy": "1 GiB fp32 device copy, bytes read + written, 10 reps"}


def pmc_traffic(profile: Path, sources: list[Path]):
    """HBM bytes per launch of the attention kernel from a committed rocprofv3 --pmc summary,
    or None when the kernel's sources have changed since the counters were taken."""
    if not profile.exists():
        return None, "no counter summary"
    fields = {}
    for line in profile.read_text().splitlines():
        if line.startswith("- ") and ": " in line:
            key, val = line[2:].split(": ", 1)
            fields[key.strip()] = val.strip().strip("`")
    h = hashlib.sha256()
    for src in sources:
        h.update(src.read_bytes())
    if fields.get("source_sha256") != h.hexdigest():
        return None, "kernel changed since the counters were taken"
    try:
        return int(fields["traffic_bytes_per_launch"]), profile.name
    except (KeyError, ValueError):
        return None, "summary has no traffic_bytes_per_launch"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--chunks", type=int, default=12, help="distinct input chunks rotated through the steps")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads in the oracle CPU sample (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum wall time of the oracle CPU sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run a plain 256 MiB elementwise copy (for counter calibration)")
    ap.add_argument("--keep", type=float, default=None, help="override the kept fraction of key blocks")
    ap.add_argument("--window", type=int, default=None, help="override the window length in frames")
    ap.add_argument("--mode", choices=("step", "hier", "cag", "bwd", "stack", "sweep", "horizon"), default="step",
                    help="step: the hybrid step (default); hier: hierarchical selection + attention on a 21-frame "
                         "window; cag: a stream from an empty window under the chunk-aware keep schedule; "
                         "bwd: training forward (with lse) and backward of the attention + readout; stack: a "
                         "30-layer x 4-stream chunk captured in a HIP graph; sweep: keep ratios on a 21-frame window "
                         "against dense; horizon: 200 consecutive committed steps timed one by one")
    ap.add_argument("--top-frames", type=int, default=6, help="hier: frames kept per query block")
    ap.add_argument("--top-k", type=int, default=128, help="hier: key blocks kept per query block")
    ap.add_argument("--stream", type=int, default=16, help="cag: chunks in the stream")
    ap.add_argument("--horizon", type=int, default=200, help="horizon: committed steps in the stream")
    ap.add_argument("--layers", type=int, default=30, help="stack: layers in the stack")
    ap.add_argument("--rope", type=str, default=None, metavar="DT,CAP",
                    help="step: time the step with the relative temporal rotary embedding (rotated features DT, "
                         "offset cap CAP frames, base 10000)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures the single-GPU hybrid attention step; --gpus {args.gpus} is not supported "
              "(the path shards by head/stream with no exchange; multi-GPU runs are out of scope)", file=sys.stderr)
        sys.exit(2)

    import torch

    import hybrid_sparse_linear_hf_amd as hf
    from hybrid_sparse_linear_hf_amd import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.mode == "hier":
        return bench_hier(args)
    if args.mode == "cag":
        return bench_cag(args)
    if args.mode == "bwd":
        return bench_bwd(args)
    if args.mode == "stack":
        return bench_stack(args)
    if args.mode == "sweep":
        return bench_sweep(args)
    if args.mode == "horizon":
        return bench_horizon(args)
    cfg = synth.LAYER_832x480
    rope = None
    if args.rope:
        dt, cap = (int(x) for x in args.rope.split(","))
        rope = hf.Rope(dt, cap, 10000.0)
        import dataclasses
        cfg = dataclasses.replace(cfg, name=f"{cfg.name}_rope{dt}_cap{cap}")
    if args.keep is not None or args.window is not None:
        import dataclasses
        cfg = dataclasses.replace(cfg, keep=args.keep if args.keep is not None else cfg.keep,
                                  W=args.window if args.window is not None else cfg.W,
                                  name=f"{cfg.name}_keep{args.keep}_w{args.window}")
    g = hf.Geometry(cfg.B, cfg.H, cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    top_k = cfg.top_k()
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- stream set-up: state from 18 frames, W-C frames committed, rotating current chunks
    kw = dict(B=cfg.B, H=cfg.H, D=cfg.D, gh=cfg.gh, gw=cfg.gw)
    ev = cfg.n_evicted
    ring = hf.Ring(g)
    ws = hf.new_workspace(g)
    S = torch.zeros((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dev)
    z = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=torch.float32, device=dev)
    hf.hf_linear_absorb(g, to_dev(synth.field_frames(synth.K_ID, 0, ev, **kw)),
                        to_dev(synth.field_frames(synth.V_ID, 0, ev, **kw)), ev * cfg.T, S, z, ws)
    hist = cfg.W - cfg.C
    for f in range(0, hist, cfg.C):
        # commit the window's history frames chunk by chunk through the ring
        kc = synth.field_frames(synth.K_ID, ev + f, cfg.C, **kw)
        vc = synth.field_frames(synth.V_ID, ev + f, cfg.C, **kw)
        ring.set_state(0, f)
        hf.hf_ring_append(g, ring, to_dev(kc), to_dev(vc))
    ring.set_state(0, hist)
    chunks = []
    for s in range(args.chunks):
        f0 = ev + hist + cfg.C * s
        chunks.append(tuple(to_dev(synth.field_frames(t, f0, cfg.C, **kw)) for t in (synth.Q_ID, synth.K_ID, synth.V_ID)))
    torch.cuda.synchronize()

    n_total = args.warmup + args.steps
    idx_bufs = [torch.empty((cfg.B, cfg.H, g.n_qb, top_k), dtype=torch.int32, device=dev) for _ in range(args.steps)]
    idx_warm = torch.empty_like(idx_bufs[0])
    out = torch.empty((cfg.B, cfg.H, cfg.Nq, cfg.D), dtype=torch.float32, device=dev)
    hip = HipEvents()
    # The timed steps record no events: each recorded event costs several microseconds of
    # GPU timeline.  The phase events come from PHASE_STEPS further steps of the same stream
    # after the timed region.
    evs = [[hip.create() for _ in range(6)] for _ in range(PHASE_STEPS)]
    idx_ph = [torch.empty_like(idx_warm) for _ in range(PHASE_STEPS)]

    def step(i, timed_slot=None, flags=hf.HF_STEP_COMMIT, events=None, idx=None):
        q, k, v = chunks[i % len(chunks)]
        if idx is None:
            idx = idx_bufs[timed_slot] if timed_slot is not None else idx_warm
        if rope is None:
            hf.hf_hybrid_step(g, q, k, v, ring, top_k, flags, S, z, idx, out, ws, events=events)
        else:
            hf.hf_hybrid_step_rope(g, q, k, v, ring, top_k, flags, S, z, idx, out, ws, rope, events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s, timed_slot=s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert n_total == args.warmup + args.steps
    # What the absorb adds to a step, on one window: the last step's chunk attended on the
    # ring as it is now, R times with the commit (state and descriptor restored between the
    # repetitions; the commit itself writes nothing the next repetition reads) and R times
    # without it.  Same window, same kept blocks, same cache state for both: the difference
    # of the attention launches (whose extra workgroups form the absorb partials in a
    # committed step) plus the state pass that adds them (ev4 -> ev5) is the absorb's cost.
    R = 12
    q_ab, k_ab, v_ab = chunks[(n_total - 1) % len(chunks)]
    S_snap, z_snap, desc = S.clone(), z.clone(), (ring.head, ring.n_committed)
    ev_ab = [[hip.create() for _ in range(6)] for _ in range(2 * R)]
    for r in range(2 * R):
        ring.set_state(*desc)
        S.copy_(S_snap)
        z.copy_(z_snap)
        hf.hf_hybrid_step(g, q_ab, k_ab, v_ab, ring, top_k, hf.HF_STEP_COMMIT if r < R else 0, S, z, idx_warm, out,
                          ws, events=ev_ab[r])
    torch.cuda.synchronize()
    ring.set_state(*desc)
    S.copy_(S_snap)
    z.copy_(z_snap)
    ab_attn = [hip.elapsed_ms(e[3], e[4]) for e in ev_ab[2:R]]
    ab_state = [hip.elapsed_ms(e[4], e[5]) for e in ev_ab[2:R]]
    nc_attn = [hip.elapsed_ms(e[3], e[4]) for e in ev_ab[R + 2:]]
    t_attn_c = float(np.median(ab_attn)) * 1e-3
    t_attn_nc = float(np.median(nc_attn)) * 1e-3
    t_state_ab = float(np.median(ab_state)) * 1e-3
    # the same A/B by the wall clock, with no events: blocks of RW repetitions with and
    # without the commit, alternating; the restores are the same in both arms
    RW, NB = 20, 4
    blk = {True: [], False: []}
    for b in range(2 * NB):
        commit = b % 2 == 0
        torch.cuda.synchronize()
        t0b = time.perf_counter()
        for r in range(RW):
            ring.set_state(*desc)
            S.copy_(S_snap)
            z.copy_(z_snap)
            hf.hf_hybrid_step(g, q_ab, k_ab, v_ab, ring, top_k, hf.HF_STEP_COMMIT if commit else 0, S, z, idx_warm,
                              out, ws)
        torch.cuda.synchronize()
        blk[commit].append((time.perf_counter() - t0b) / RW)
    ring.set_state(*desc)
    S.copy_(S_snap)
    z.copy_(z_snap)
    t_abs_wall = max(float(np.median(blk[True]) - np.median(blk[False])), 1e-9)
    # phase events: further steps of the stream
    for p in range(PHASE_STEPS):
        step(n_total + p, events=evs[p], idx=idx_ph[p])
    torch.cuda.synchronize()
    n_total += PHASE_STEPS

    # [steps, 5] ms: (empty) | select (its pool launch also appends the chunk to the ring and prepares
    # the readout operands) | (empty) | attention + readout (+ the absorb partials) | state pass
    phases = np.array([[hip.elapsed_ms(e[p], e[p + 1]) for p in range(5)] for e in evs])
    step_ms = np.array([hip.elapsed_ms(e[0], e[5]) for e in evs])
    if args.calib_copy:
        # plain copy kernel of known size: reads and writes 256 MiB each
        src = torch.randn(64 << 20, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    # hot-cache attention: the last step's queries and kept lists again on the ring as it is
    # now (same shapes and access pattern; operands resident in L2 / MALL), with the readout
    q_last = chunks[(n_total - 1) % len(chunks)][0]
    idx_last = idx_ph[-1]
    attn_hot = []
    for rep in range(23):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if rope is None:
            hf.hf_sparse_window_attn(g, q_last, ring, idx_last, top_k, S, z, out, ws)
        else:
            hf.hf_sparse_window_attn_rope(g, q_last, ring, idx_last, top_k, S, z, out, ws, rope)
        e1.record()
        attn_hot.append((e0, e1))
    torch.cuda.synchronize()
    t_attn_hot = float(np.median([a.elapsed_time(b) for a, b in attn_hot[3:]])) * 1e-3
    peaks = measured_peaks(torch, dev)
    flops = np.array([kept_flops(b.cpu().numpy(), cfg.Nq, cfg.Nk, cfg.bq, cfg.bk, cfg.D) for b in idx_bufs])
    flops_ph = np.array([kept_flops(b.cpu().numpy(), cfg.Nq, cfg.Nk, cfg.bq, cfg.bk, cfg.D) for b in idx_ph])
    ms_step = wall * 1e3 / args.steps
    value = flops.sum() / wall / 1e12
    t_sel = phases[:, 1].mean() * 1e-3
    t_evpair = phases[:, 2].mean() * 1e-3   # ev2 -> ev3: nothing runs between them
    t_attn = phases[:, 3].mean() * 1e-3
    t_state = phases[:, 4].mean() * 1e-3   # the state pass adding the absorb partials
    t_abs = t_abs_wall   # what the absorb adds to a step
    attn_tflops = flops_ph.mean() / t_attn / 1e12
    if rope is None:
        traffic, traffic_src = pmc_traffic(ATTN_PMC_SUMMARY, ATTN_SOURCES)
    else:
        traffic, traffic_src = None, "the counter summary covers the unrotated kernel instance only"
    BH, T, D = cfg.B * cfg.H, cfg.T, cfg.D
    absorb_bytes = BH * (cfg.C * T * D * 2 * 2 + 2 * (D * D + D) * 4)
    append_bytes = BH * cfg.C * T * D * 2 * 2 * 2
    prep_bytes = BH * (D * D * (4 + 2) + D * 4 * 2)
    select_bytes = BH * (cfg.Nq * D * 2 + cfg.Nk * D * 2 + g.n_qb * top_k * 4) + append_bytes + prep_bytes
    select_alg = BH * (cfg.Nq * D * 2 + cfg.Nk * D * 2 + g.n_qb * top_k * 4)
    floor_us = (flops.mean() / (PEAK_BF16_TFLOPS * 1e12) + select_alg / (PEAK_HBM_GBS * 1e9)) * 1e6

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded rank-8 spatial field + noise per head, bf16)",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "D": cfg.D, "tokens_per_frame": cfg.T,
                   "chunk_frames": cfg.C, "window_frames": cfg.W, "block": [cfg.bq, cfg.bk], "top_k": top_k,
                   "n_kb": g.n_kb(cfg.W - cfg.C), "state_frames_at_start": cfg.n_evicted,
                   "parallelism": "single GPU", "rotating_chunks": args.chunks},
        "step_ms_median": round(float(np.median(step_ms)), 4),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_source": traffic_src,
                     "kernel": f"sparse_attn_kernel<128, 2, {rope.temporal_dims // 16 if rope else 0}>",
                     "flops_per_launch": round(flops_ph.mean()), "launch_us": round(t_attn * 1e6, 2),
                     "frac_of_measured_gemm": round(attn_tflops / peaks["bf16_gemm_tflops"], 4),
                     "hot_cache_launch_us": round(t_attn_hot * 1e6, 2),
                     "hot_cache_note": "the last step's attention repeated on resident operands; includes the "
                                       "readout-operand launch",
                     "launch_note": "in a committed step the attention launch also forms the absorb partials"},
        "phases_us": {"select_append_prep": round(t_sel * 1e6, 2),
                      "event_pair_only": round(t_evpair * 1e6, 2),
                      "sparse_attn_readout_and_absorb_partials": round(t_attn * 1e6, 2),
                      "state_pass": round(t_state * 1e6, 2)},
        "phases_note": "HIP events recorded inside hf_hybrid_step on the step's stream: select = pool launch "
                       "(with the readout operands) + score/top-k launch (with the ring append); "
                       "event_pair_only = two events recorded back to back with no launch between them, "
                       "the cost of one recorded event, which every other phase figure also carries",
        "absorb_roofline": {"bound": "hbm", "achieved": round(absorb_bytes / t_abs / 1e9, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(absorb_bytes / t_abs / 1e9 / PEAK_HBM_GBS, 4),
                            "bytes_per_launch": absorb_bytes, "added_us_per_step": round(t_abs * 1e6, 2),
                            "events_estimate_us": round((max(t_attn_c - t_attn_nc, 0.0) + t_state_ab) * 1e6, 2),
                            "attention_launch_us_with_commit": round(t_attn_c * 1e6, 2),
                            "attention_launch_us_without_commit": round(t_attn_nc * 1e6, 2),
                            "state_pass_us": round(t_state_ab * 1e6, 2),
                            "frac_of_measured_copy": round(absorb_bytes / t_abs / 1e9 / peaks["copy_gbs"], 4),
                            "note": "what absorbing the 3 evicted frames adds to a step: the wall time per step "
                                    "with the commit minus without it, on one window with state and ring restored "
                                    "before every step (medians of 4 blocks of 20 steps per arm, no events); "
                                    "events_estimate_us is the same from HIP events: the attention launch with the "
                                    "commit (its extra workgroups form the absorb partials) minus without, plus the "
                                    "state pass (ev4 -> ev5, including an event's own cost)"},
        "select_roofline": {"bound": "hbm", "achieved": round(select_bytes / t_sel / 1e9, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "bytes_per_launch": select_bytes,
                            "note": "pool (+ ring append + readout operands) and score/top-k launches (ev1 -> ev2)"},
        "step_tflops_frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "step_tflops_frac_of_measured_gemm": round(value / peaks["bf16_gemm_tflops"], 4),
        "step_floor_us": round(floor_us, 2),
        "step_floor_note": "kept-block flops at bf16 peak + selection bytes (Q, window K, idx) at HBM peak",
        "measured_peaks": peaks,
        "cpu_baseline": None,
    }
    if args.cpu_heads > 0:
        cb = cpu_baseline(cfg, min(args.cpu_heads, cfg.H), args.cpu_seconds)
        res["cpu_baseline_ms_per_step"] = round(cb.pop("ms_per_step"), 1)
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


def _field_ring(cfg, hf, synth, torch, dev):
    """Ring holding W - C committed frames and the current chunk, a state from the absorbed
    frames, and the current chunk's queries (the layout of the step benchmark)."""
    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    g = hf.Geometry(cfg.B, cfg.H, cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    kw = dict(B=cfg.B, H=cfg.H, D=cfg.D, gh=cfg.gh, gw=cfg.gw)
    ev = cfg.n_evicted
    ring, ws = hf.Ring(g), hf.new_workspace(g)
    S = torch.zeros((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dev)
    z = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=torch.float32, device=dev)
    hf.hf_linear_absorb(g, to_dev(synth.field_frames(synth.K_ID, 0, ev, **kw)),
                        to_dev(synth.field_frames(synth.V_ID, 0, ev, **kw)), ev * cfg.T, S, z, ws)
    for f in range(0, cfg.W, cfg.C):
        ring.set_state(0, f)
        hf.hf_ring_append(g, ring, to_dev(synth.field_frames(synth.K_ID, ev + f, cfg.C, **kw)),
                          to_dev(synth.field_frames(synth.V_ID, ev + f, cfg.C, **kw)))
    ring.set_state(0, cfg.W - cfg.C)
    q = to_dev(synth.field_frames(synth.Q_ID, ev + cfg.W - cfg.C, cfg.C, **kw))
    torch.cuda.synchronize()
    return g, ring, ws, S, z, q


def bench_sweep(args):
    """The 832x480 shapes with a 21-frame window (32760 keys, 512 key blocks), keep ratio
    swept over 100 / 50 / 25 / 12.5 %: per ratio, block selection followed by the sparse
    attention with the readout, against the dense window attention (every block kept, no
    selection).  The crossover is the keep ratio where selection + sparse stops beating
    dense."""
    import torch
    import hybrid_sparse_linear_hf_amd as hf
    from hybrid_sparse_linear_hf_amd import synth

    cfg = synth.LAYER_832x480_W21
    dev = torch.device("cuda:0")
    g, ring, ws, S, z, q = _field_ring(cfg, hf, synth, torch, dev)
    nkb = g.n_kb(cfg.W - cfg.C)
    out = torch.empty((cfg.B, cfg.H, cfg.Nq, cfg.D), dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def timed(fn_sel, fn_attn):
        sel, att = [], []
        for it in range(args.warmup + args.steps):
            ev[0].record()
            fn_sel()
            ev[1].record()
            fn_attn()
            ev[2].record()
            torch.cuda.synchronize()
            if it >= args.warmup:
                sel.append(ev[0].elapsed_time(ev[1]))
                att.append(ev[1].elapsed_time(ev[2]))
        return float(np.median(sel)) * 1e3, float(np.median(att)) * 1e3

    dense_idx = torch.arange(nkb, dtype=torch.int32, device=dev).expand(cfg.B, cfg.H, g.n_qb, nkb).contiguous()
    _, t_dense = timed(lambda: None, lambda: hf.hf_sparse_window_attn(g, q, ring, dense_idx, nkb, S, z, out, ws))
    f_dense = kept_flops(dense_idx.cpu().numpy(), cfg.Nq, cfg.Nk, cfg.bq, cfg.bk, cfg.D)
    rows = []
    for keep in (1.0, 0.5, 0.25, 0.125):
        k = max(1, -(-int(round(keep * 1000)) * nkb // 1000))
        idx = torch.empty((cfg.B, cfg.H, g.n_qb, k), dtype=torch.int32, device=dev)
        t_sel, t_att = timed(lambda: hf.hf_block_select(g, q, ring, k, idx, None, ws),
                             lambda: hf.hf_sparse_window_attn(g, q, ring, idx, k, S, z, out, ws))
        fl = kept_flops(idx.cpu().numpy(), cfg.Nq, cfg.Nk, cfg.bq, cfg.bk, cfg.D)
        rows.append({"keep": keep, "top_k": k, "select_us": round(t_sel, 2), "attention_us": round(t_att, 2),
                     "total_us": round(t_sel + t_att, 2), "attention_tflops": round(fl / (t_att * 1e-6) / 1e12, 1),
                     "speedup_vs_dense": round(t_dense / (t_sel + t_att), 3)})
    beats = [r["keep"] for r in rows if r["speedup_vs_dense"] > 1.0]
    cpu = cpu_baseline_sweep(cfg, [r["top_k"] for r in rows], args.cpu_seconds) if args.cpu_heads > 0 else None
    res = {"metric": "keep-ratio sweep on a 21-frame window: select + sparse attention vs dense (832x480 shape, 1 GPU)",
           "value": rows[2]["total_us"], "unit": "us at keep 25 %", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(rows[2]["total_us"] * 1e-3, 4), "higher_is_better": False,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded rank-8 spatial field + noise per head, bf16)",
           "config": {"workload": cfg.name, "H": cfg.H, "D": cfg.D, "tokens_per_frame": cfg.T, "chunk_frames": cfg.C,
                      "window_frames": cfg.W, "block": [cfg.bq, cfg.bk], "n_kb": nkb},
           "dense_us": round(t_dense, 2), "dense_tflops": round(f_dense / (t_dense * 1e-6) / 1e12, 1),
           "sweep": rows,
           "crossover": ("selection + sparse beats dense at every keep ratio below 100 %" if set(beats) >= {0.5, 0.25, 0.125}
                         else f"selection + sparse beats dense at keep ratios {beats}"),
           "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


def cpu_baseline_sweep(cfg, top_ks, seconds):
    """The fp64 oracle (test infrastructure) at each keep ratio of the sweep, on a bounded
    sample: head 0, selection over every query block and the sparse attention + readout on
    its first 8 query blocks, repeated until `seconds` / len(top_ks) of wall time."""
    import oracle
    from hybrid_sparse_linear_hf_amd import synth

    inp = synth.field_step_inputs(cfg, heads=[0])
    f64 = synth.f64_from_bf16_bits
    Q, K, V = f64(inp["q"]), f64(inp["k_win"]), f64(inp["v_win"])
    S0, z0 = oracle.absorb(f64(inp["k_ev"]), f64(inp["v_ev"]))
    blocks = [(0, i) for i in range(8)]
    out = []
    for k in top_ks:
        reps, fl = 0, 0.0
        t0 = time.perf_counter()
        while True:
            _, idx, _ = oracle.hybrid_step(Q, K, V, S0, z0, cfg.bq, cfg.bk, k, blocks=blocks)
            fl += kept_flops(idx[:, :, :8], cfg.Nq, cfg.Nk, cfg.bq, cfg.bk, cfg.D)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds / len(top_ks):
                break
        out.append({"top_k": k, "value": round(fl / dt / 1e12, 5), "ms_per_sample": round(dt / reps * 1e3, 1)})
    return {"unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "head 0 of 12: selection over all 74 query blocks, sparse attention + readout on query blocks "
                      "0-7 (fp64), per keep ratio", "per_keep": out}


def bench_hier(args):
    """Hierarchical coarse-to-fine selection ([LF-de] §2.2) feeding the sparse attention, on
    the 832x480 shapes with a 21-frame window (32760 keys, 512 key blocks): per timed step,
    hf_block_select_hier (top_frames frames, then top_k blocks inside them) and
    hf_sparse_window_attn with the readout; the flat selection of the same top_k is timed
    beside it."""
    import torch
    import hybrid_sparse_linear_hf_amd as hf
    from hybrid_sparse_linear_hf_amd import synth

    cfg = synth.LAYER_832x480_W21
    dev = torch.device("cuda:0")
    g, ring, ws, S, z, q = _field_ring(cfg, hf, synth, torch, dev)
    nfr, nkb = cfg.W, g.n_kb(cfg.W - cfg.C)
    idx = torch.empty((cfg.B, cfg.H, g.n_qb, args.top_k), dtype=torch.int32, device=dev)
    idx_flat = torch.empty_like(idx)
    out = torch.empty((cfg.B, cfg.H, cfg.Nq, cfg.D), dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    sel, att, flat = [], [], []
    for it in range(args.warmup + args.steps):
        ev[0].record()
        hf.hf_block_select_hier(g, q, ring, args.top_frames, args.top_k, idx, ws)
        ev[1].record()
        hf.hf_sparse_window_attn(g, q, ring, idx, args.top_k, S, z, out, ws)
        ev[2].record()
        hf.hf_block_select(g, q, ring, args.top_k, idx_flat, None, ws)
        ev[3].record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            sel.append(ev[0].elapsed_time(ev[1]))
            att.append(ev[1].elapsed_time(ev[2]))
            flat.append(ev[2].elapsed_time(ev[3]))
    fl = kept_flops(idx.cpu().numpy(), cfg.Nq, nfr * cfg.T, cfg.bq, cfg.bk, cfg.D)
    t = (np.median(sel) + np.median(att)) * 1e-3
    res = {"metric": "hierarchical select + sparse attention, 21-frame window (832x480 shape, 1 GPU)",
           "value": round(fl / t / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(t * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded rank-8 spatial field + noise per head, bf16)",
           "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "D": cfg.D, "tokens_per_frame": cfg.T,
                      "chunk_frames": cfg.C, "window_frames": cfg.W, "block": [cfg.bq, cfg.bk], "n_kb": nkb,
                      "top_frames": args.top_frames, "top_k": args.top_k},
           "hier_select_us": round(float(np.median(sel)) * 1e3, 2),
           "flat_select_us": round(float(np.median(flat)) * 1e3, 2),
           "sparse_attn_readout_us": round(float(np.median(att)) * 1e3, 2),
           "kept_flops": round(fl),
           "attn_frac_of_bf16_peak": round(fl / (np.median(att) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    print(json.dumps(res), flush=True)


def bench_bwd(args):
    """Backward of the attention + readout at the 832x480 layer (selection held fixed):
    hf_sparse_window_attn_lse then hf_hybrid_attn_backward per timed step.  Algorithmic
    backward flops = 10 D per kept (query, key) pair (the products S = Q K^T, dP = dO V^T,
    dV = P^T dO, dQ = G K, dK = G^T Q), i.e. 2.5x the forward's kept flops."""
    import torch
    import hybrid_sparse_linear_hf_amd as hf
    from hybrid_sparse_linear_hf_amd import synth

    cfg = synth.LAYER_832x480
    dev = torch.device("cuda:0")
    g, ring, ws, S, z, q = _field_ring(cfg, hf, synth, torch, dev)
    top_k = cfg.top_k()
    Nk = cfg.W * cfg.T
    bws = hf.new_backward_workspace(g, top_k)
    idx = torch.empty((cfg.B, cfg.H, g.n_qb, top_k), dtype=torch.int32, device=dev)
    out = torch.empty((cfg.B, cfg.H, cfg.Nq, cfg.D), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H, cfg.Nq), dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev).manual_seed(0)
    dout = torch.randn((cfg.B, cfg.H, cfg.Nq, cfg.D), dtype=torch.float32, device=dev, generator=gen)
    dq = torch.empty_like(dout)
    dk = torch.empty((cfg.B, cfg.H, Nk, cfg.D), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    dS, dz = torch.empty_like(S), torch.empty_like(z)
    hf.hf_block_select(g, q, ring, top_k, idx, None, ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd, bwd = [], []
    for it in range(args.warmup + args.steps):
        ev[0].record()
        hf.hf_sparse_window_attn_lse(g, q, ring, idx, top_k, S, z, out, lse, ws)
        ev[1].record()
        hf.hf_hybrid_attn_backward(g, q, ring, idx, top_k, S, z, out, lse, dout, dq, dk, dv, dS, dz, bws)
        ev[2].record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            fwd.append(ev[0].elapsed_time(ev[1]))
            bwd.append(ev[1].elapsed_time(ev[2]))
    fl = kept_flops(idx.cpu().numpy(), cfg.Nq, Nk, cfg.bq, cfg.bk, cfg.D)
    tb = float(np.median(bwd)) * 1e-3
    res = {"metric": "hybrid attention backward (selection fixed), 832x480 layer, 1 GPU",
           "value": round(2.5 * fl / tb / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(tb * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded rank-8 spatial field + noise per head, bf16)",
           "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "D": cfg.D, "tokens_per_frame": cfg.T,
                      "chunk_frames": cfg.C, "window_frames": cfg.W, "block": [cfg.bq, cfg.bk], "top_k": top_k},
           "forward_lse_us": round(float(np.median(fwd)) * 1e3, 2),
           "backward_us": round(tb * 1e6, 2),
           "backward_algorithmic_flops": round(2.5 * fl),
           "backward_frac_of_bf16_peak": round(2.5 * fl / tb / 1e12 / PEAK_BF16_TFLOPS, 4)}
    print(json.dumps(res), flush=True)


def bench_stack(args):
    """The attention of a 30-layer stack for 4 batched streams at the 832x480 layer shapes
    (each layer its own ring, state and seeded bf16 Q/K/V, N(0,1)*0.5): one chunk = 30
    hf_hybrid_step calls with commit, captured once in a HIP graph and replayed.  Reports
    the chunk latency and the implied latent frames per second (4 streams x 3 frames per
    chunk), beside the same 30 calls launched eagerly."""
    import torch
    import hybrid_sparse_linear_hf_amd as hf
    from hybrid_sparse_linear_hf_amd import synth

    base = synth.LAYER_832x480
    n_layers, B = args.layers, 4
    g = hf.Geometry(B, base.H, base.D, base.T, base.C, base.W, base.bq, base.bk)
    hist = g.W - g.C
    top_k = base.top_k()
    dev = torch.device("cuda:0")
    ws = hf.new_workspace(g)
    out = torch.empty((B, g.H, g.Nq, g.D), dtype=torch.float32, device=dev)
    layers = []
    for layer in range(n_layers):
        gen = torch.Generator(device=dev).manual_seed(1000 + layer)

        def rnd(n):
            return (torch.randn((B, g.H, n, g.D), generator=gen, device=dev) * 0.5).to(torch.bfloat16)

        ring = hf.Ring(g)
        hf.hf_ring_append(g, ring, rnd(g.Nq), rnd(g.Nq))      # the window's committed history (W - C = C frames)
        ring.set_state(0, hist)
        S = torch.zeros((B, g.H, g.D, g.D), dtype=torch.float32, device=dev)
        z = torch.zeros((B, g.H, g.D), dtype=torch.float32, device=dev)
        hf.hf_linear_absorb(g, rnd(g.Nq), rnd(g.Nq), g.Nq, S, z, ws)
        idx = torch.empty((B, g.H, g.n_qb, top_k), dtype=torch.int32, device=dev)
        layers.append((ring, S, z, idx, rnd(g.Nq), rnd(g.Nq), rnd(g.Nq)))
    torch.cuda.synchronize()
    descs = [(L[0].head, L[0].n_committed) for L in layers]

    def chunk():
        for ring, S, z, idx, q, k, v in layers:
            hf.hf_hybrid_step(g, q, k, v, ring, top_k, hf.HF_STEP_COMMIT, S, z, idx, out, ws)

    def reset():     # every step starts from the same window position (replays repeat it)
        for (ring, *_), d in zip(layers, descs):
            ring.set_state(*d)

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # eager
    for _ in range(2):
        reset()
        chunk()
    torch.cuda.synchronize()
    eager = []
    for _ in range(args.steps):
        reset()
        e0.record()
        chunk()
        e1.record()
        torch.cuda.synchronize()
        eager.append(e0.elapsed_time(e1))
    # graph
    reset()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chunk()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    fl = sum(kept_flops(L[3].cpu().numpy(), g.Nq, (hist + g.C) * g.T, g.bq, g.bk, g.D) for L in layers)
    res = {"metric": "30-layer x 4-stream attention stack: chunk latency (832x480 layer shapes, HIP graph, 1 GPU)",
           "value": round(ms, 3), "unit": "ms per chunk", "n_gpus": 1, "steps": args.steps, "warmup": 2,
           "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic (seeded N(0,1)*0.5 bf16 per layer and stream)",
           "config": {"workload": f"stack_{n_layers}x4_832x480", "layers": n_layers, "streams": B, "H": g.H, "D": g.D,
                      "tokens_per_frame": g.T, "chunk_frames": g.C, "window_frames": g.W, "block": [g.bq, g.bk],
                      "top_k": top_k},
           "latent_frames_per_s": round(B * g.C / (ms * 1e-3), 1),
           "kept_tflops": round(fl / (ms * 1e-3) / 1e12, 1),
           "eager_ms_per_chunk": round(float(np.median(eager)), 3),
           "wall_ms_per_chunk": round(wall * 1e3 / args.steps, 3),
           "note": "attention only (no projections, MLP or VAE); not comparable with end-to-end generation rates"}
    print(json.dumps(res), flush=True)

def _frames_par(synth, tensor_id, f0, n, cfg, heads):
    """synth.field_frames of several heads drawn on a thread pool (one head per task)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(min(16, len(heads))) as ex:
        parts = ex.map(lambda h: synth.field_frames(tensor_id, f0, n, B=cfg.B, D=cfg.D, gh=cfg.gh, gw=cfg.gw,
                                                    heads=[h]), heads)
        return np.concatenate(list(parts), axis=1)


def bench_horizon(args):
    """The long-horizon stream at the 832x480 layer shapes: from a state of 18 absorbed frames
    and 3 committed window frames, `--horizon` consecutive hf_hybrid_step calls with commit,
    each appending a 3-frame chunk and absorbing the 3 frames it evicts into the fp32 state
    (S 12x128x128, z 12x128).  The stream runs twice from the same start: once timed by the
    wall clock alone, once with an event between consecutive steps for the per-step times.
    The chunks (distinct seeded field frames) rotate through the stream, all resident in
    device memory before the first step."""
    import torch
    import hybrid_sparse_linear_hf_amd as hf
    from hybrid_sparse_linear_hf_amd import synth

    cfg = synth.LAYER_832x480
    dev = torch.device("cuda:0")
    g = hf.Geometry(cfg.B, cfg.H, cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    heads = list(range(cfg.H))

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def frames(tid, f0, n):
        return to_dev(_frames_par(synth, tid, f0, n, cfg, heads))

    ev, hist, n = cfg.n_evicted, cfg.W - cfg.C, args.horizon
    k_ev, v_ev, k_hist, v_hist = frames(synth.K_ID, 0, ev), frames(synth.V_ID, 0, ev), \
        frames(synth.K_ID, ev, hist), frames(synth.V_ID, ev, hist)
    first = ev + hist
    chunks = [tuple(frames(t, first + cfg.C * c, cfg.C) for t in (synth.Q_ID, synth.K_ID, synth.V_ID))
              for c in range(args.chunks)]
    ring, ws = hf.Ring(g), hf.new_workspace(g)
    S = torch.zeros((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dev)
    z = torch.zeros_like(S[..., 0])
    top_k = cfg.top_k()
    idx = [torch.empty((cfg.B, cfg.H, g.n_qb, top_k), dtype=torch.int32, device=dev) for _ in range(n)]
    out = torch.empty((cfg.B, cfg.H, cfg.Nq, cfg.D), dtype=torch.float32, device=dev)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]

    def start():
        S.zero_()
        z.zero_()
        hf.hf_linear_absorb(g, k_ev, v_ev, ev * cfg.T, S, z, ws)
        ring.set_state(0, 0)
        hf.hf_ring_append(g, ring, k_hist, v_hist)
        ring.set_state(0, hist)
        torch.cuda.synchronize()

    def stream(events):
        for s in range(n):
            q, k, v = chunks[s % len(chunks)]
            if events:
                marks[s].record()
            hf.hf_hybrid_step(g, q, k, v, ring, top_k, hf.HF_STEP_COMMIT, S, z, idx[s], out, ws)
        if events:
            marks[n].record()

    start()               # warm-up pass (code objects, caches)
    stream(False)
    start()
    t0 = time.perf_counter()
    stream(False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    state_norm = float(torch.linalg.vector_norm(S).item())
    start()
    stream(True)
    torch.cuda.synchronize()
    per = np.array([marks[s].elapsed_time(marks[s + 1]) for s in range(n)])
    fl = np.array([kept_flops(i.cpu().numpy(), cfg.Nq, cfg.Nk, cfg.bq, cfg.bk, cfg.D) for i in idx])
    ms = wall * 1e3 / n
    q10 = max(1, n // 10)
    slope = float(np.polyfit(np.arange(n), per, 1)[0]) * 1e3 if n > 1 else 0.0
    res = {"metric": f"long-horizon stream: ms per committed chunk step over {n} steps (832x480 shape, 1 GPU)",
           "value": round(ms, 4), "unit": "ms per step", "n_gpus": 1, "steps": n, "warmup": n,
           "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic (seeded rank-8 spatial field + noise per head, bf16)",
           "config": {"workload": cfg.name + f"_horizon{n}", "B": cfg.B, "H": cfg.H, "D": cfg.D,
                      "tokens_per_frame": cfg.T, "chunk_frames": cfg.C, "window_frames": cfg.W,
                      "block": [cfg.bq, cfg.bk], "top_k": top_k, "state_frames_at_start": ev,
                      "state_frames_at_end": ev + cfg.C * n, "rotating_chunks": args.chunks},
           "kept_tflops": round(fl.sum() / wall / 1e12, 2),
           "per_step_ms": {"median": round(float(np.median(per)), 4), "p90": round(float(np.percentile(per, 90)), 4),
                           "max": round(float(per.max()), 4), "min": round(float(per.min()), 4),
                           f"first_{q10}_mean": round(float(per[:q10].mean()), 4),
                           f"last_{q10}_mean": round(float(per[-q10:].mean()), 4),
                           "slope_us_per_step": round(slope, 4)},
           "per_step_note": "HIP events between consecutive steps of a second pass from the same start (each "
                            "event adds a few microseconds); value is the wall clock of the pass without events",
           "final_state_fro_norm": round(state_norm, 3),
           "cpu_baseline": None}
    if args.cpu_heads > 0:
        res["cpu_baseline"] = cpu_baseline_horizon(cfg, min(args.cpu_heads, cfg.H), args.cpu_seconds)
    print(json.dumps(res), flush=True)


def cpu_baseline_horizon(cfg, sample_heads, seconds):
    """The fp64 oracle (test infrastructure) running the same stream on a bounded sample: the
    first consecutive steps on `sample_heads` heads (the window of frames, select + sparse
    attention + readout, then the 3 evicted frames absorbed into the state), until `seconds`
    of wall time have passed.  Drawing the frames is not timed."""
    import oracle
    from hybrid_sparse_linear_hf_amd import synth

    heads = list(range(sample_heads))
    f64 = synth.f64_from_bf16_bits
    T, C, ev, hist = cfg.T, cfg.C, cfg.n_evicted, cfg.W - cfg.C
    S, z = oracle.absorb(f64(_frames_par(synth, synth.K_ID, 0, ev, cfg, heads)),
                         f64(_frames_par(synth, synth.V_ID, 0, ev, cfg, heads)))
    win_k = f64(_frames_par(synth, synth.K_ID, ev, hist, cfg, heads))
    win_v = f64(_frames_par(synth, synth.V_ID, ev, hist, cfg, heads))
    k = cfg.top_k()
    steps, busy = [], 0.0
    f = ev + hist
    while busy < seconds:
        q, kc, vc = (f64(_frames_par(synth, t, f, C, cfg, heads)) for t in (synth.Q_ID, synth.K_ID, synth.V_ID))
        t0 = time.perf_counter()
        K = np.concatenate([win_k, kc], axis=2)
        V = np.concatenate([win_v, vc], axis=2)
        oracle.hybrid_step(q, K, V, S, z, cfg.bq, cfg.bk, k)
        S, z = oracle.absorb(K[:, :, :C * T], V[:, :, :C * T], S, z)   # the oldest C frames leave the window
        win_k, win_v = K[:, :, C * T:], V[:, :, C * T:]
        dt = time.perf_counter() - t0
        steps.append(dt)
        busy += dt
        f += C
    per = float(np.median(steps)) * 1e3
    return {"value": round(per, 1), "unit": "ms per step", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the first {len(steps)} consecutive committed steps of the stream on {sample_heads} of "
                      f"{cfg.H} heads (fp64), {busy:.1f} s of oracle time",
            "cpu_model": cpu_model(), "per_step_ms": [round(x * 1e3, 1) for x in steps],
            "ms_per_step_all_heads_est": round(per * cfg.H / sample_heads, 1)}


def bench_cag(args):
    """A stream of `--stream` chunks from an empty window at the 832x480 layer shapes (W=6),
    every step an hf_hybrid_step with commit, once with the chunk-aware growth keep counts
    ([LF-de] §2.1: hf_cag_schedule, first chunk dense, stream-wide sparsity 75 %) and once
    with a uniform 25 % keep.  Reports the wall time of each stream and its kept work."""
    import torch
    import hybrid_sparse_linear_hf_amd as hf
    from hybrid_sparse_linear_hf_amd import synth

    cfg = synth.LAYER_832x480
    dev = torch.device("cuda:0")
    g = hf.Geometry(cfg.B, cfg.H, cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    kw = dict(B=cfg.B, H=cfg.H, D=cfg.D, gh=cfg.gh, gw=cfg.gw)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    chunks = [tuple(to_dev(synth.field_frames(t, cfg.C * s, cfg.C, **kw)) for t in (synth.Q_ID, synth.K_ID, synth.V_ID))
              for s in range(args.stream)]
    n_kb = [g.n_kb(min(cfg.C * s, cfg.W - cfg.C)) for s in range(args.stream)]
    k_cag, s_cag, beta = hf.hf_cag_schedule(n_kb, 0.9, 0.75, 0.95)
    k_uni = [max(1, -(-n // 4)) for n in n_kb]
    out = torch.empty((cfg.B, cfg.H, cfg.Nq, cfg.D), dtype=torch.float32, device=dev)

    def run(ks):
        ring, ws = hf.Ring(g), hf.new_workspace(g)
        S = torch.zeros((cfg.B, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device=dev)
        z = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=torch.float32, device=dev)
        idxs = [torch.empty((cfg.B, cfg.H, g.n_qb, k), dtype=torch.int32, device=dev) for k in ks]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s, (q, k, v) in enumerate(chunks):
            hf.hf_hybrid_step(g, q, k, v, ring, ks[s], hf.HF_STEP_COMMIT, S, z, idxs[s], out, ws)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        fl = sum(kept_flops(i.cpu().numpy(), cfg.Nq, min(cfg.C * (s + 1), cfg.W) * cfg.T, cfg.bq, cfg.bk, cfg.D)
                 for s, i in enumerate(idxs))
        return wall, fl

    for _ in range(max(1, args.warmup // 5)):
        run(k_uni)
    walls = {"cag": [], "uniform": []}
    fls = {}
    for _ in range(5):
        for name, ks in (("cag", k_cag), ("uniform", k_uni)):
            w, fl = run(ks)
            walls[name].append(w)
            fls[name] = fl
    wc, wu = float(np.median(walls["cag"])), float(np.median(walls["uniform"]))
    res = {"metric": "chunk-aware growth stream: kept TFLOP/s over a 16-chunk stream (832x480 shape, 1 GPU)",
           "value": round(fls["cag"] / wc / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": 5,
           "warmup": max(1, args.warmup // 5), "ms_per_step": round(wc * 1e3 / args.stream, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded rank-8 spatial field + noise per head, bf16)",
           "config": {"workload": cfg.name + "_stream", "chunks": args.stream, "s_base": 0.9, "s_target": 0.75,
                      "s_max": 0.95, "n_kb": n_kb},
           "cag": {"top_k": k_cag, "sparsity": [round(x, 4) for x in s_cag], "beta": round(beta, 6),
                   "stream_ms": round(wc * 1e3, 3), "kept_flops": round(fls["cag"])},
           "uniform_25pct": {"top_k": k_uni, "stream_ms": round(wu * 1e3, 3), "kept_flops": round(fls["uniform"])}}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
