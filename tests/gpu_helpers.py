"""Shared helpers of the GPU parity tests: put seeded bf16 inputs on the device, lay
frames into the KV ring, compare against the fp64 oracle."""

from __future__ import annotations

import numpy as np
import torch

import hybrid_sparse_linear_hf_amd as hf
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
        ring.vt[:, :, s] = v[:, :, f].transpose(-1, -2)
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
