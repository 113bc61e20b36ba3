"""Shared helpers of the GPU parity tests: put seeded bf16 inputs on the device, lay
frames into the KV ring, compare against the fp64 oracle."""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import hybrid_sparse_linear_hf_amd as hf
import oracle
from hybrid_sparse_linear_hf_amd import synth

MAX_ABS_TOL = 1e-2
MEAN_REL_TOL = 2e-3


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> contiguous bfloat16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda").contiguous()


def f64(bits: np.ndarray) -> np.ndarray:
    return synth.f64_from_bf16_bits(bits)


def fill_ring(ring: hf.Ring, k_bits: np.ndarray, v_bits: np.ndarray, n_frames: int, head: int) -> None:
    """Write logical window frames 0..n_frames-1 (k_bits/v_bits [B,H,n_frames*T,D]) into their slots."""
    g = ring.g
    k = dev_bf16(k_bits).view(g.B, g.H, n_frames, g.T, g.D)
    v = dev_bf16(v_bits).view(g.B, g.H, n_frames, g.T, g.D)
    for f in range(n_frames):
        s = (head + f) % g.W
        ring.k[:, :, s] = k[:, :, f]
        ring.vg[:, :, s] = hf.Ring.grouped(v[:, :, f])
    torch.cuda.synchronize()


def compare(out: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    """(max |out - ref|, sum |out - ref| / sum |ref|)."""
    d = np.abs(out.astype(np.float64) - ref)
    return float(d.max()), float(d.sum() / max(np.abs(ref).sum(), 1e-300))


def assert_close(out: np.ndarray, ref: np.ndarray, what: str = "") -> tuple[float, float]:
    mx, mr = compare(out, ref)
    assert mx <= MAX_ABS_TOL and mr <= MEAN_REL_TOL, f"{what}: max-abs {mx:.3e}, mean-rel {mr:.3e}"
    return mx, mr


def rows_of_blocks(blocks, Nq, bq, shape):
    """Boolean mask [B*H, Nq] of the query rows in the listed (plane, block) pairs."""
    m = np.zeros(shape, dtype=bool)
    for p, i in blocks:
        m[p, i * bq:min((i + 1) * bq, Nq)] = True
    return m


class StepInputs:
    """Device + oracle copies of one step: Q, window K/V (logical order), evicted K/V."""

    def __init__(self, q, k_win, v_win, k_ev=None, v_ev=None):
        self.q_bits, self.k_bits, self.v_bits = q, k_win, v_win
        self.kev_bits, self.vev_bits = k_ev, v_ev
        self.Q, self.K, self.V = f64(q), f64(k_win), f64(v_win)
        self.Kev = None if k_ev is None else f64(k_ev)
        self.Vev = None if v_ev is None else f64(v_ev)


_POOL = ThreadPoolExecutor(max_workers=8)


def field_frames_par(tensor_id, f0, n, heads, *, B=1, D=128, gh=30, gw=52, layer=0):
    """synth.field_frames for several heads, drawn on a thread pool (the draws release the
    GIL; BLAS is held to one thread meanwhile, so the small products do not contend)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        futs = [_POOL.submit(synth.field_frames, tensor_id, f0, n, B=B, D=D, gh=gh, gw=gw, layer=layer, heads=[h])
                for h in heads]
        return np.concatenate([f.result() for f in futs], axis=1)


class OracleStream:
    """The method's streaming loop written plainly: a window of frames, the state, and
    eviction of the oldest frames into the state once more than W - C are committed."""

    def __init__(self, B, H, D, T, C, W, S=None, z=None):
        self.T, self.C, self.W = T, C, W
        self.frames_k, self.frames_v = [], []
        self.S = np.zeros((B, H, D, D)) if S is None else S
        self.z = np.zeros((B, H, D)) if z is None else z

    def step(self, Qc, Kc, Vc, bq, bk, top_k, blocks=None):
        """Qc, Kc, Vc: fp64 [B,H,C*T,D] of the current chunk.  Returns (out, idx)."""
        K = np.concatenate(self.frames_k + [Kc], axis=2)
        V = np.concatenate(self.frames_v + [Vc], axis=2)
        out, idx, _ = oracle.hybrid_step(Qc, K, V, self.S, self.z, bq, bk, top_k, blocks=blocks)
        T = self.T
        for c in range(self.C):
            self.frames_k.append(Kc[:, :, c * T:(c + 1) * T])
            self.frames_v.append(Vc[:, :, c * T:(c + 1) * T])
        excess = len(self.frames_k) - (self.W - self.C)
        if excess > 0:
            Kev = np.concatenate(self.frames_k[:excess], axis=2)
            Vev = np.concatenate(self.frames_v[:excess], axis=2)
            self.S, self.z = oracle.absorb(Kev, Vev, self.S, self.z)
            del self.frames_k[:excess], self.frames_v[:excess]
        return out, idx


def random_chunks(g, n_steps, seed):
    rng = np.random.default_rng(seed)
    b = synth.bf16_bits_from_f32
    shape = (g.B, g.H, g.C * g.T, g.D)
    return [tuple(b(rng.standard_normal(shape).astype(np.float32)) for _ in range(3)) for _ in range(n_steps)]


def run_gpu_stream(g, chunks, keep, head0=0):
    """hf_hybrid_step with commit over `chunks` from an empty window.  `keep`: a ratio
    (top_k = ceil(keep * n_kb) per step) or a list of keep counts, one per step."""
    ring = hf.Ring(g)
    ring.set_state(head0, 0)
    ws = hf.new_workspace(g)
    S = torch.zeros((g.B, g.H, g.D, g.D), dtype=torch.float32, device="cuda")
    z = torch.zeros((g.B, g.H, g.D), dtype=torch.float32, device="cuda")
    outs, idxs = [], []
    for s, (q, k, v) in enumerate(chunks):
        top_k = keep[s] if isinstance(keep, (list, tuple)) else max(1, int(np.ceil(keep * g.n_kb(ring.n_committed))))
        idx = torch.empty((g.B, g.H, g.n_qb, top_k), dtype=torch.int32, device="cuda")
        out = torch.empty((g.B, g.H, g.Nq, g.D), dtype=torch.float32, device="cuda")
        hf.hf_hybrid_step(g, dev_bf16(q), dev_bf16(k), dev_bf16(v), ring, top_k, hf.HF_STEP_COMMIT, S, z, idx, out, ws)
        outs.append(out.cpu().numpy())
        idxs.append(idx.cpu().numpy())
    torch.cuda.synchronize()
    return outs, idxs, S.cpu().numpy().astype(np.float64), z.cpu().numpy().astype(np.float64), ring


