"""Seeded synthetic attention inputs for the hybrid attention step.

This module only *draws* inputs. It holds none of the method's arithmetic
(no pooling, scoring, selection, softmax, feature map or state update), so
both the HIP path and the fp64 oracle can consume what it produces without
sharing any computation.

Two recipes exist:

* ``tiny``: i.i.d. standard-normal fp32 tensors drawn from
  ``numpy.random.default_rng(seed)`` in a fixed order (Q, then all keys,
  then all values).  The token streams hold ``n_evicted`` frames that were
  already folded into the linear state, then the window frames, oldest
  first, the last ``C`` of which are the current chunk.

* ``field``: per (layer, stream, head) a smooth rank-8 spatial field on the
  ``gh x gw`` latent patch grid plus white noise, scaled by 0.5, standing in
  for the attention activations of a 832x480 video model (30x52 latent
  patches, 12 heads of width 128).  Each frame is seeded on its own so a
  frame has identical values whether it sits in the window or is being
  evicted, and streams of any length are reproducible:

      X[f, y, x, :] = 0.5 * ( sqrt(0.75) * sum_r g_r(f, y, x) * U^X_r
                              + sqrt(0.25) * xi ),      xi ~ N(0, I_D)
      g_r(f, y, x) = sqrt(2) * cos(2*pi*(a_r*y/gh + c_r*x/gw) + theta_r + omega_r*f)

  with a_r, c_r uniform in {0,1,2}, theta_r ~ U[0, 2*pi), omega_r ~
  U[-0.1, 0.1] and U^X_r ~ N(0, I_D/8), drawn from
  ``SeedSequence([seed, layer, stream, head, 99])``; the noise of frame f of
  tensor X (0=Q, 1=K, 2=V) comes from
  ``SeedSequence([seed, layer, stream, head, X, f])``.  Q, K and V share the
  fields g and have independent coefficients U^X.

Every tensor is rounded to bfloat16 with round-to-nearest-even; values are
returned as uint16 bit patterns (the bf16 storage both sides read) and can
be widened exactly to fp32 / fp64.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

Q_ID, K_ID, V_ID = 0, 1, 2
_RANK = 8


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f64_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return f32_from_bf16_bits(b).astype(np.float64)


# --------------------------------------------------------------------------------------
# tiny i.i.d. recipe
# --------------------------------------------------------------------------------------

@dataclass
class TinyStream:
    """i.i.d. N(0,1) tokens for a small, fully oracle-checkable step.

    Shapes: q [B,H,C*T,D]; k_all / v_all [B,H,(n_evicted+W)*T,D], frames in
    stream order: n_evicted already-absorbed frames, then the window (oldest
    first) whose last C frames are the current chunk.
    """

    q: np.ndarray
    k_all: np.ndarray
    v_all: np.ndarray
    T: int
    C: int
    W: int
    n_evicted: int


def tiny_stream(B=1, H=1, D=64, T=64, C=1, W=4, n_evicted=3, seed=0) -> TinyStream:
    rng = np.random.default_rng(seed)
    nq = C * T
    nkv = (n_evicted + W) * T
    q = rng.standard_normal((B, H, nq, D), dtype=np.float32)
    k = rng.standard_normal((B, H, nkv, D), dtype=np.float32)
    v = rng.standard_normal((B, H, nkv, D), dtype=np.float32)
    return TinyStream(q, k, v, T, C, W, n_evicted)


# --------------------------------------------------------------------------------------
# rank-8 smooth field recipe
# --------------------------------------------------------------------------------------

class FieldSource:
    """Deterministic per-frame bf16 activations for one (layer, stream, head)."""

    def __init__(self, D=128, gh=30, gw=52, seed=0, layer=0, stream=0, head=0):
        self.D, self.gh, self.gw = D, gh, gw
        self.key = (seed, layer, stream, head)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, stream, head, 99])))
        self.a = rng.integers(0, 3, size=_RANK)
        self.c = rng.integers(0, 3, size=_RANK)
        self.theta = rng.uniform(0.0, 2.0 * math.pi, size=_RANK)
        self.omega = rng.uniform(-0.1, 0.1, size=_RANK)
        self.U = [rng.standard_normal((_RANK, D)) / math.sqrt(_RANK) for _ in range(3)]
        yy, xx = np.meshgrid(np.arange(gh), np.arange(gw), indexing="ij")
        self._phase = (2.0 * math.pi * (np.outer(yy.ravel(), self.a) / gh + np.outer(xx.ravel(), self.c) / gw)
                       + self.theta)  # [T, R]

    @property
    def T(self) -> int:
        return self.gh * self.gw

    def frame_f32(self, tensor_id: int, f: int) -> np.ndarray:
        """fp32 values (before bf16 rounding) of frame f of tensor Q/K/V: [T, D]."""
        g = math.sqrt(2.0) * np.cos(self._phase + self.omega * f)  # [T, R]
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([*self.key, tensor_id, f])))
        xi = rng.standard_normal((self.T, self.D))
        x = 0.5 * (math.sqrt(0.75) * (g @ self.U[tensor_id]) + math.sqrt(0.25) * xi)
        return x.astype(np.float32)

    def frames_bf16(self, tensor_id: int, f0: int, n: int) -> np.ndarray:
        """bf16 bits of frames f0..f0+n-1, concatenated along tokens: [n*T, D] uint16."""
        return np.concatenate([bf16_bits_from_f32(self.frame_f32(tensor_id, f)) for f in range(f0, f0 + n)], axis=0)


def field_frames(tensor_id: int, f0: int, n: int, *, B=1, H=12, D=128, gh=30, gw=52, seed=0, layer=0,
                 heads=None) -> np.ndarray:
    """bf16 bits [B, len(heads), n*gh*gw, D] of frames f0..f0+n-1 for every (stream, head)."""
    heads = list(range(H)) if heads is None else list(heads)
    out = np.empty((B, len(heads), n * gh * gw, D), dtype=np.uint16)
    for b in range(B):
        for hi, h in enumerate(heads):
            out[b, hi] = FieldSource(D, gh, gw, seed, layer, b, h).frames_bf16(tensor_id, f0, n)
    return out


@dataclass(frozen=True)
class StepConfig:
    """Shape of one hybrid attention step on a streaming window."""

    name: str
    B: int
    H: int
    D: int
    T: int
    C: int
    W: int
    bq: int
    bk: int
    keep: float          # fraction of key blocks kept per query block (k = ceil(keep * n_kb))
    n_evicted: int       # frames already absorbed into the linear state before the step
    gh: int = 30
    gw: int = 52

    @property
    def Nq(self) -> int:
        return self.C * self.T

    @property
    def Nk(self) -> int:
        return self.W * self.T

    @property
    def n_qb(self) -> int:
        return -(-self.Nq // self.bq)

    @property
    def n_kb(self) -> int:
        return -(-self.Nk // self.bk)

    def top_k(self, n_kb: int | None = None) -> int:
        from fractions import Fraction
        n = self.n_kb if n_kb is None else n_kb
        k = Fraction(self.keep).limit_denominator(1 << 20) * n
        k = -(-k.numerator // k.denominator)
        return max(1, min(n, k))


# The configurations the step is measured and checked on.
TINY = StepConfig("tiny_d64_t64_w4", B=1, H=1, D=64, T=64, C=1, W=4, bq=16, bk=16, keep=2 / 16, n_evicted=3,
                  gh=8, gw=8)
LAYER_832x480 = StepConfig("832x480_layer_h12_d128_w6", B=1, H=12, D=128, T=1560, C=3, W=6, bq=64, bk=64,
                           keep=0.25, n_evicted=18)
LAYER_832x480_W21 = StepConfig("832x480_layer_h12_d128_w21", B=1, H=12, D=128, T=1560, C=3, W=21, bq=64, bk=64,
                               keep=0.25, n_evicted=18)


def field_step_inputs(cfg: StepConfig, *, seed=0, layer=0, first_frame=None, heads=None):
    """Q, window K/V and evicted K/V (bf16 bits) for one steady-state step of a field stream.

    Frames 0..n_evicted-1 are the absorbed history; the window holds frames
    n_evicted..n_evicted+W-1 (oldest first) and the current chunk is the last
    C of them, whose Q is returned.
    Returns dict(q [B,h,Nq,D], k_win/v_win [B,h,Nk,D], k_ev/v_ev [B,h,n_evicted*T,D]).
    """
    ev = cfg.n_evicted if first_frame is None else first_frame
    kw = dict(B=cfg.B, H=cfg.H, D=cfg.D, gh=cfg.gh, gw=cfg.gw, seed=seed, layer=layer, heads=heads)
    cur0 = ev + cfg.W - cfg.C
    return dict(
        q=field_frames(Q_ID, cur0, cfg.C, **kw),
        k_win=field_frames(K_ID, ev, cfg.W, **kw),
        v_win=field_frames(V_ID, ev, cfg.W, **kw),
        k_ev=field_frames(K_ID, 0, ev, **kw) if ev > 0 else None,
        v_ev=field_frames(V_ID, 0, ev, **kw) if ev > 0 else None,
    )
