"""fp64 CPU oracle of the Hybrid Forcing hybrid attention step -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark use
this package.  It loads ``liboracle.so`` (plain C, built by :func:`build`) through
ctypes and wraps its functions for numpy arrays.  It imports nothing from the HIP
library and the HIP library imports nothing from it.

Every wrapper takes and returns fp64 arrays shaped [B, H, N, D] (planes = B*H).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "liboracle.so"
_SOURCES = [_HERE / "hf_oracle.c"]


def build(verbose: bool = False) -> Path:
    """Compile liboracle.so with gcc (fp64, -O2, OpenMP, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", str(LIB_PATH) + ".tmp", *map(str, _SOURCES), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(str(LIB_PATH) + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)
_I64 = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            build()
        L = ctypes.CDLL(str(LIB_PATH))
        L.hfo_phi.argtypes = [ctypes.c_double]
        L.hfo_phi.restype = ctypes.c_double
        L.hfo_pool.argtypes = [_i64, _i64, _i64, _i64, _D, _D]
        L.hfo_block_scores.argtypes = [_i64, _i64, _i64, _i64, _D, _D, _D]
        L.hfo_select.argtypes = [_i64, _i64, _i64, _i64, _D, _I32]
        L.hfo_sparse_attn.argtypes = [_i64] * 7 + [_D, _D, _D, _I32, _I64, _i64, _D]
        L.hfo_sparse_attn_rope.argtypes = [_i64] * 10 + [ctypes.c_double, _D, _D, _D, _I32, _I64, _i64, _D]
        L.hfo_linear_readout.argtypes = [_i64, _i64, _i64, _i64, _D, _D, _D, ctypes.c_double, _I64, _i64, _D]
        L.hfo_absorb.argtypes = [_i64, _i64, _i64, _D, _D, _D, _D]
        L.hfo_hybrid_step.argtypes = ([_i64] * 7 + [ctypes.c_double, _D, _D, _D, _D, _D, _I64, _i64, _I32, _D, _D])
        L.hfo_sparse_attn_bwd.argtypes = [_i64] * 7 + [_D, _D, _D, _I32, _D, _D, _D, _D]
        L.hfo_linear_readout_bwd.argtypes = [_i64, _i64, _i64, _D, _D, _D, ctypes.c_double, _D, _D, _D, _D]
        L.hfo_absorb_bwd.argtypes = [_i64, _i64, _i64, _D, _D, _D, _D, _D, _D]
        L.hfo_num_threads.restype = ctypes.c_int
        L.hfo_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a, t=_D):
    return None if a is None else a.ctypes.data_as(t)


def _blocks(blocks):
    """[(plane, query_block), ...] -> (int64 array [n,2] or None, n)."""
    if blocks is None:
        return None, 0
    b = np.ascontiguousarray(np.asarray(blocks, dtype=np.int64).reshape(-1, 2))
    return b, b.shape[0]


def n_blocks(n: int, blk: int) -> int:
    return -(-n // blk)


def phi(x: float) -> float:
    return lib().hfo_phi(float(x))


def num_threads() -> int:
    return lib().hfo_num_threads()


def set_num_threads(n: int) -> None:
    lib().hfo_set_num_threads(int(n))


def pool(X, blk):
    X = _f64(X)
    B, H, N, D = X.shape
    out = np.empty((B, H, n_blocks(N, blk), D))
    lib().hfo_pool(B * H, N, D, blk, _p(X), _p(out))
    return out


def block_scores(qbar, kbar):
    qbar, kbar = _f64(qbar), _f64(kbar)
    B, H, nqb, D = qbar.shape
    nkb = kbar.shape[2]
    s = np.empty((B, H, nqb, nkb))
    lib().hfo_block_scores(B * H, nqb, nkb, D, _p(qbar), _p(kbar), _p(s))
    return s


def select(s, k):
    s = _f64(s)
    B, H, nqb, nkb = s.shape
    if not 1 <= k <= nkb:
        raise ValueError("need 1 <= k <= n_kb")
    idx = np.empty((B, H, nqb, k), dtype=np.int32)
    lib().hfo_select(B * H, nqb, nkb, k, _p(s), _p(idx, _I32))
    return idx


def sparse_attn(Q, K, V, idx, bq, bk, blocks=None, out=None):
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, H, Nq, D = Q.shape
    Nk = K.shape[2]
    k = idx.shape[-1]
    out = np.zeros_like(Q) if out is None else out
    bl, nb = _blocks(blocks)
    lib().hfo_sparse_attn(B * H, Nq, Nk, D, bq, bk, k, _p(Q), _p(K), _p(V), _p(idx, _I32), _p(bl, _I64), nb,
                          _p(out))
    return out


def sparse_attn_rope(Q, K, V, idx, bq, bk, T, temporal_dims, cap, base=10000.0, blocks=None, out=None):
    """Sparse attention with the relative temporal rotary embedding (query rotated by the
    clamped frame offset to each key's frame; see hfo_sparse_attn_rope)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, H, Nq, D = Q.shape
    Nk = K.shape[2]
    if Nq % T or Nk % T or temporal_dims % 2 or not 0 <= temporal_dims <= D or cap < 0:
        raise ValueError("need whole frames, an even temporal_dims <= D and cap >= 0")
    k = idx.shape[-1]
    out = np.zeros_like(Q) if out is None else out
    bl, nb = _blocks(blocks)
    lib().hfo_sparse_attn_rope(B * H, Nq, Nk, D, bq, bk, k, T, temporal_dims, cap, base, _p(Q), _p(K), _p(V),
                               _p(idx, _I32), _p(bl, _I64), nb, _p(out))
    return out


def linear_readout(Q, S, z, bq=64, eps=1e-6, blocks=None, out=None):
    Q, S, z = _f64(Q), _f64(S), _f64(z)
    B, H, Nq, D = Q.shape
    out = np.zeros_like(Q) if out is None else out
    bl, nb = _blocks(blocks)
    lib().hfo_linear_readout(B * H, Nq, D, bq, _p(Q), _p(S), _p(z), eps, _p(bl, _I64), nb, _p(out))
    return out


def absorb(K, V, S=None, z=None):
    """Return (S + sum phi(K)^T V, z + sum phi(K)) -- inputs are not modified."""
    K, V = _f64(K), _f64(V)
    B, H, n, D = K.shape
    S = np.zeros((B, H, D, D)) if S is None else _f64(S).copy()
    z = np.zeros((B, H, D)) if z is None else _f64(z).copy()
    lib().hfo_absorb(B * H, n, D, _p(K), _p(V), _p(S), _p(z))
    return S, z


def hybrid_step(Q, K, V, S, z, bq, bk, k, eps=1e-6, blocks=None, want_scores=False):
    """Whole step -> (out [B,H,Nq,D], idx [B,H,nqb,k], scores or None)."""
    Q, K, V, S, z = _f64(Q), _f64(K), _f64(V), _f64(S), _f64(z)
    B, H, Nq, D = Q.shape
    Nk = K.shape[2]
    nqb, nkb = n_blocks(Nq, bq), n_blocks(Nk, bk)
    if not 1 <= k <= nkb:
        raise ValueError("need 1 <= k <= n_kb")
    out = np.zeros_like(Q)
    idx = np.empty((B, H, nqb, k), dtype=np.int32)
    sc = np.empty((B, H, nqb, nkb)) if want_scores else None
    bl, nb = _blocks(blocks)
    lib().hfo_hybrid_step(B * H, Nq, Nk, D, bq, bk, k, eps, _p(Q), _p(K), _p(V), _p(S), _p(z), _p(bl, _I64), nb,
                          _p(idx, _I32), _p(sc), _p(out))
    return out, idx, sc


def hybrid_step_rope(Q, K, V, S, z, bq, bk, k, T, temporal_dims, cap, base=10000.0, eps=1e-6, blocks=None):
    """The step with the rotary embedding on the softmax branch: selection and readout
    from the raw features (as hybrid_step), sparse part by sparse_attn_rope.
    -> (out, idx)."""
    Q = _f64(Q)
    _, idx, _ = hybrid_step(Q, K, V, S, z, bq, bk, k, eps=eps, blocks=[(0, 0)])
    out = sparse_attn_rope(Q, K, V, idx, bq, bk, T, temporal_dims, cap, base, blocks=blocks)
    lin = linear_readout(Q, S, z, bq, eps, blocks=blocks)
    return out + lin, idx


def cag_schedule(n_kb, s_base, s_target, s_max):
    """Chunk-aware growth schedule ([LF-de] §2.1 "Chunk-bewusstes Wachstum"): chunk 0 is
    dense; chunk i >= 1 has sparsity s_i = clip(s_base - alpha_i * beta, 0, s_max) with
    alpha_i = 1 / sqrt(i + 1) (the page's alpha proportional to one over a square root,
    read against the chunk's position) and keeps k_i = ceil((1 - s_i) * n_kb[i]) key
    blocks; beta is the least value at which the kept blocks of all chunks reach
    (1 - s_target) of the dense total.

    Worked out exactly rather than searched: for 1 <= m < n = n_kb[i], chunk i keeps more
    than m blocks exactly when (1 - s_i) n > m, i.e. s_i < c = 1 - m / n.  Since s_i never
    exceeds s_max and c > 0, that holds for every beta when s_max < c, and otherwise
    exactly when s_base - beta / sqrt(i + 1) < c, i.e. beta > t = (s_base - 1 + m / n) *
    sqrt(i + 1).  So the total kept is a constant plus the number of breakpoints t below
    beta; the least beta reaching the goal is 0 if the total at 0 already does, else the
    r-th smallest breakpoint, r the number of blocks still missing (the total jumps just
    after it, so this is the infimum of the betas that reach the goal).  The keep counts
    returned are those just above that beta.  Returns (keep counts, sparsities, beta)."""
    import math
    n = len(n_kb)
    base = n_kb[0] + (n - 1)                 # chunk 0 dense, every later chunk keeps >= 1
    always = 0
    points = []                              # (t, chunk)
    for i in range(1, n):
        for m in range(1, n_kb[i]):
            if s_max < 1.0 - m / n_kb[i]:
                always += 1
            else:
                points.append(((s_base - 1.0 + m / n_kb[i]) * math.sqrt(i + 1), i))
    points.sort()
    goal = math.ceil((1.0 - s_target) * float(sum(n_kb)))     # kept totals are integers
    below0 = sum(1 for t, _ in points if t < 0.0)
    if base + always + below0 >= goal:
        beta = 0.0
        passed = [(t, i) for t, i in points if t < 0.0]
    else:
        beta = points[goal - base - always - 1][0]
        passed = [(t, i) for t, i in points if t <= beta]
    keep = [n_kb[0]] + [1] * (n - 1)
    for i in range(1, n):
        keep[i] += sum(1 for m in range(1, n_kb[i]) if s_max < 1.0 - m / n_kb[i])
    for _, i in passed:
        keep[i] += 1
    ss = [0.0] + [min(max(s_base - beta / math.sqrt(i + 1), 0.0), s_max) for i in range(1, n)]
    return keep, ss, beta


def frames_of_block(j, bk, Nk, T):
    """Window frames (first, last) that key block j = keys [j bk, min((j+1) bk, Nk)) touches."""
    return (j * bk) // T, (min((j + 1) * bk, Nk) - 1) // T


def hier_select(Q, K, bq, bk, T, k_frames, k):
    """Hierarchical coarse-to-fine block selection ([LF-de] §2.2 "Hierarchische Spärliche
    Attention"), in the pages' order:
      token compression -- queries pooled per query block, keys per key block and per
          window frame (T keys), all by the mean;
      frame selection -- per query block, score every window frame by the pooled query
          block . the frame-pooled keys / sqrt(D) and keep the k_frames best (ties to the
          lower frame);
      block selection -- among the key blocks that touch a kept frame, keep the k best by
          the usual block score (ties to the lower block), listed ascending.
    Q [B,H,Nq,D], K [B,H,Nk,D] with Nk a whole number of frames.  Returns
    (idx [B,H,nqb,k] int32, frames [B,H,nqb,k_frames] int32, block scores, frame scores)."""
    Q, K = _f64(Q), _f64(K)
    B, H, Nk, D = K.shape
    if Nk % T:
        raise ValueError("the window must hold whole frames")
    qbar, kbar, fbar = pool(Q, bq), pool(K, bk), pool(K, T)
    s = block_scores(qbar, kbar)
    sf = block_scores(qbar, fbar)
    frames = select(sf, k_frames)
    nqb, nkb = s.shape[2], s.shape[3]
    idx = np.empty((B, H, nqb, k), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                kept = set(int(f) for f in frames[b, h, i])
                cand = []
                for j in range(nkb):
                    f0, f1 = frames_of_block(j, bk, Nk, T)
                    if any(f in kept for f in range(f0, f1 + 1)):
                        cand.append((-s[b, h, i, j], j))
                if len(cand) < k:
                    raise ValueError("fewer key blocks in the kept frames than k")
                cand.sort()
                idx[b, h, i] = sorted(j for _, j in cand[:k])
    return idx, frames, s, sf


# ---------------------------------------------------------------- backward (idx held fixed)

def sparse_attn_bwd(Q, K, V, idx, bq, bk, dO):
    """Gradients of sum(sparse_attn(Q, K, V, idx) * dO) -> (dQ, dK, dV); the chain rule of
    the softmax over each query's kept keys (hf_oracle.h states the terms)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, H, Nq, D = Q.shape
    Nk = K.shape[2]
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    lib().hfo_sparse_attn_bwd(B * H, Nq, Nk, D, bq, bk, idx.shape[-1], _p(Q), _p(K), _p(V), _p(idx, _I32), _p(dO),
                              _p(dQ), _p(dK), _p(dV))
    return dQ, dK, dV


def linear_readout_bwd(Q, S, z, dO, eps=1e-6):
    """Gradients of sum(linear_readout(Q, S, z) * dO) -> (dQ, dS, dz)."""
    Q, S, z, dO = _f64(Q), _f64(S), _f64(z), _f64(dO)
    B, H, Nq, D = Q.shape
    dQ, dS, dz = np.zeros_like(Q), np.zeros_like(S), np.zeros_like(z)
    lib().hfo_linear_readout_bwd(B * H, Nq, D, _p(Q), _p(S), _p(z), eps, _p(dO), _p(dQ), _p(dS), _p(dz))
    return dQ, dS, dz


def absorb_bwd(K, V, dS, dz):
    """Gradients w.r.t. the absorbed tokens of sum(S_after * dS) + sum(z_after * dz) -> (dK, dV)."""
    K, V, dS, dz = _f64(K), _f64(V), _f64(dS), _f64(dz)
    B, H, n, D = K.shape
    dK, dV = np.zeros_like(K), np.zeros_like(V)
    lib().hfo_absorb_bwd(B * H, n, D, _p(K), _p(V), _p(dS), _p(dz), _p(dK), _p(dV))
    return dK, dV


def hybrid_step_bwd(Q, K, V, S, z, idx, bq, bk, dO, eps=1e-6):
    """Backward of the step output sparse_attn + linear_readout with the selection idx held
    fixed -> (dQ, dK, dV, dS, dz): dQ is the sum of both branches' terms."""
    dQ1, dK, dV = sparse_attn_bwd(Q, K, V, idx, bq, bk, dO)
    dQ2, dS, dz = linear_readout_bwd(Q, S, z, dO, eps)
    return dQ1 + dQ2, dK, dV, dS, dz
