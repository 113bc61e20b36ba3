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
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} full steps (select + sparse attention + readout + absorb of {cfg.C} "
                      f"frames) on {sample_heads} of {cfg.H} heads of the {cfg.name} workload, fp64, "
                      f"{dt:.1f} s wall, {dt / reps * 1e3:.0f} ms per step",
            "ms_per_step": dt / reps * 1e3}


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
    cfg = synth.LAYER_832x480
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
    evs = [[hip.create() for _ in range(6)] for _ in range(args.steps)]

    def step(i, timed_slot=None):
        q, k, v = chunks[i % len(chunks)]
        idx = idx_bufs[timed_slot] if timed_slot is not None else idx_warm
        events = evs[timed_slot] if timed_slot is not None else None
        hf.hf_hybrid_step(g, q, k, v, ring, top_k, hf.HF_STEP_COMMIT, S, z, idx, out, ws, events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s, timed_slot=s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert n_total == args.warmup + args.steps

    # [steps, 5] ms: append | select | readout operands | attention + readout | absorb + state update
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
    flops = np.array([kept_flops(b.cpu().numpy(), cfg.Nq, cfg.Nk, cfg.bq, cfg.bk, cfg.D) for b in idx_bufs])
    ms_step = wall * 1e3 / args.steps
    value = flops.sum() / wall / 1e12
    t_app = phases[:, 0].mean() * 1e-3
    t_sel = phases[:, 1].mean() * 1e-3
    t_prep = phases[:, 2].mean() * 1e-3
    t_attn = phases[:, 3].mean() * 1e-3
    t_abs = phases[:, 4].mean() * 1e-3     # absorb partial sums + state update
    attn_tflops = flops.mean() / t_attn / 1e12
    traffic, traffic_src = pmc_traffic(ATTN_PMC_SUMMARY, ATTN_SOURCES)
    BH, T, D = cfg.B * cfg.H, cfg.T, cfg.D
    absorb_bytes = BH * (cfg.C * T * D * 2 * 2 + 2 * (D * D + D) * 4)
    select_bytes = BH * (cfg.Nq * D * 2 + cfg.Nk * D * 2 + g.n_qb * top_k * 4)
    append_bytes = BH * cfg.C * T * D * 2 * 2 * 2

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
                     "kernel": "sparse_attn_kernel<128, 2>",
                     "flops_per_launch": round(flops.mean()), "launch_us": round(t_attn * 1e6, 2)},
        "phases_us": {"append": round(t_app * 1e6, 2), "select": round(t_sel * 1e6, 2),
                      "readout_prep": round(t_prep * 1e6, 2), "sparse_attn_readout": round(t_attn * 1e6, 2),
                      "absorb_and_state": round(t_abs * 1e6, 2)},
        "absorb_roofline": {"bound": "hbm", "achieved": round(absorb_bytes / t_abs / 1e9, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(absorb_bytes / t_abs / 1e9 / PEAK_HBM_GBS, 4),
                            "bytes_per_launch": absorb_bytes,
                            "note": "absorb kernel + the state update that adds its partial sums (ev4 -> ev5)"},
        "select_roofline": {"bound": "hbm", "achieved": round(select_bytes / t_sel / 1e9, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "bytes_per_launch": select_bytes},
        "append_roofline": {"bound": "hbm", "achieved": round(append_bytes / t_app / 1e9, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "bytes_per_launch": append_bytes},
        "step_tflops_frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "cpu_baseline": None,
    }
    if args.cpu_heads > 0:
        cb = cpu_baseline(cfg, min(args.cpu_heads, cfg.H), args.cpu_seconds)
        res["cpu_baseline_ms_per_step"] = round(cb.pop("ms_per_step"), 1)
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
