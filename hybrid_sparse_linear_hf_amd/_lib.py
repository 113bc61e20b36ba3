"""ctypes binding of libhf (include/hf.h): argument marshalling only.

Every step of the hybrid attention path runs in the HIP kernels of libhf.so; this
module converts torch tensors to device pointers and the current HIP stream, calls
the C entry point of the same name, and raises HFError on a non-zero status.  There
is no fallback: if libhf.so is missing or fails to load, every call raises.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libhf.so"

HF_OK = 0
HF_STEP_COMMIT = 1
STATUS = {0: "HF_OK", 1: "HF_ERR_NULL", 2: "HF_ERR_SHAPE", 3: "HF_ERR_UNSUPPORTED", 4: "HF_ERR_RING_STATE",
          5: "HF_ERR_WORKSPACE", 6: "HF_ERR_HIP"}


class HFError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{fn} -> {self.status_name}: {detail}")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "D", "T", "C", "W", "bq", "bk")]


class KVRing(ctypes.Structure):
    _fields_ = [("k_dev", ctypes.c_void_p), ("vt_dev", ctypes.c_void_p), ("head", ctypes.c_int32),
                ("n_committed", ctypes.c_int32)]


class StepEvents(ctypes.Structure):
    _fields_ = [("ev", ctypes.c_void_p * 6)]


class Rope(ctypes.Structure):
    """Relative temporal rotary embedding (hf_rope): the first `temporal_dims` features of
    each head turned by the frame offset clamped to +-cap, frequencies base^(-2i/temporal_dims)."""
    _fields_ = [("temporal_dims", ctypes.c_int32), ("cap", ctypes.c_int32), ("base", ctypes.c_float)]


_lib = None
_P = ctypes.c_void_p


def lib():
    """Load libhf.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m hybrid_sparse_linear_hf_amd.build`")
        L = ctypes.CDLL(str(LIB_PATH))
        i32, u32, i64, f32, sz = ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        pd, pr = ctypes.POINTER(Dims), ctypes.POINTER(KVRing)
        L.hf_abi_version.restype = ctypes.c_int
        L.hf_status_str.restype = ctypes.c_char_p
        L.hf_status_str.argtypes = [ctypes.c_int]
        L.hf_last_error.restype = ctypes.c_char_p
        L.hf_workspace_size.argtypes = [pd, i32, ctypes.POINTER(sz)]
        L.hf_ring_init.argtypes = [pd, _P, _P, pr]
        L.hf_ring_append.argtypes = [pd, pr, _P, _P, _P]
        L.hf_block_select.argtypes = [pd, _P, pr, i32, _P, _P, _P, sz, _P]
        L.hf_sparse_window_attn.argtypes = [pd, _P, pr, _P, i32, _P, _P, f32, _P, _P, sz, _P]
        L.hf_linear_absorb.argtypes = [pd, _P, _P, i64, _P, _P, _P, sz, _P]
        L.hf_hybrid_step.argtypes = [pd, _P, _P, _P, pr, i32, u32, _P, _P, f32, _P, _P, _P, sz,
                                     ctypes.POINTER(StepEvents), _P]
        L.hf_block_select_hier.argtypes = [pd, _P, pr, i32, i32, _P, _P, _P, _P, _P, sz, _P]
        f64 = ctypes.c_double
        L.hf_cag_schedule.argtypes = [i32, ctypes.POINTER(i32), f64, f64, f64, ctypes.POINTER(i32),
                                      ctypes.POINTER(f64), ctypes.POINTER(f64)]
        L.hf_sparse_window_attn_lse.argtypes = [pd, _P, pr, _P, i32, _P, _P, f32, _P, _P, _P, sz, _P]
        L.hf_backward_workspace_size.argtypes = [pd, i32, ctypes.POINTER(sz)]
        L.hf_hybrid_attn_backward.argtypes = [pd, _P, pr, _P, i32, _P, _P, f32, _P, _P, _P, _P, _P, _P, _P, _P,
                                              _P, sz, _P]
        L.hf_linear_absorb_backward.argtypes = [pd, _P, _P, i64, _P, _P, _P, _P, _P, sz, _P]
        prope = ctypes.POINTER(Rope)
        L.hf_sparse_window_attn_rope.argtypes = [pd, _P, pr, _P, i32, _P, _P, f32, prope, _P, _P, sz, _P]
        L.hf_hybrid_step_rope.argtypes = [pd, _P, _P, _P, pr, i32, u32, _P, _P, f32, prope, _P, _P, _P, sz,
                                          ctypes.POINTER(StepEvents), _P]
        for fn in ("hf_workspace_size", "hf_ring_init", "hf_ring_append", "hf_block_select", "hf_sparse_window_attn",
                   "hf_linear_absorb", "hf_hybrid_step", "hf_cag_schedule", "hf_block_select_hier",
                   "hf_sparse_window_attn_lse", "hf_backward_workspace_size", "hf_hybrid_attn_backward",
                   "hf_linear_absorb_backward", "hf_sparse_window_attn_rope", "hf_hybrid_step_rope"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != HF_OK:
        raise HFError(fn, status, lib().hf_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def abi_version() -> int:
    return lib().hf_abi_version()


# ------------------------------------------------------------------ state containers

@dataclass
class Geometry:
    B: int
    H: int
    D: int
    T: int
    C: int
    W: int
    bq: int
    bk: int

    def dims(self) -> Dims:
        return Dims(self.B, self.H, self.D, self.T, self.C, self.W, self.bq, self.bk)

    @property
    def Nq(self) -> int:
        return self.C * self.T

    @property
    def n_qb(self) -> int:
        return -(-self.Nq // self.bq)

    def n_kb(self, n_committed: int) -> int:
        return -(-((n_committed + self.C) * self.T) // self.bk)


class Ring:
    """Device storage of the KV ring (keys [B,H,W,T,D], values transposed [B,H,W,D,T]) plus
    the host descriptor (head, n_committed)."""

    def __init__(self, g: Geometry, device="cuda"):
        self.g = g
        self.k = torch.zeros((g.B, g.H, g.W, g.T, g.D), dtype=torch.bfloat16, device=device)
        self.vt = torch.zeros((g.B, g.H, g.W, g.D, g.T), dtype=torch.bfloat16, device=device)
        self.desc = KVRing()
        _check("hf_ring_init", lib().hf_ring_init(ctypes.byref(g.dims()), self.k.data_ptr(), self.vt.data_ptr(),
                                                  ctypes.byref(self.desc)))

    @property
    def head(self) -> int:
        return self.desc.head

    @property
    def n_committed(self) -> int:
        return self.desc.n_committed

    def set_state(self, head: int, n_committed: int) -> None:
        self.desc.head, self.desc.n_committed = int(head), int(n_committed)


def workspace_size(g: Geometry, top_k: int = 1) -> int:
    n = ctypes.c_size_t(0)
    _check("hf_workspace_size", lib().hf_workspace_size(ctypes.byref(g.dims()), int(top_k), ctypes.byref(n)))
    return n.value


def new_workspace(g: Geometry, device="cuda") -> torch.Tensor:
    """Device workspace for every entry point (contents need no initialisation)."""
    return torch.zeros(workspace_size(g), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points

def hf_ring_append(g: Geometry, ring: Ring, k_cur, v_cur, stream=None) -> None:
    _check("hf_ring_append", lib().hf_ring_append(ctypes.byref(g.dims()), ctypes.byref(ring.desc), _ptr(k_cur),
                                                  _ptr(v_cur), _stream(stream)))


def hf_block_select(g: Geometry, q, ring: Ring, top_k: int, idx, scores, ws, stream=None) -> None:
    _check("hf_block_select",
           lib().hf_block_select(ctypes.byref(g.dims()), _ptr(q), ctypes.byref(ring.desc), int(top_k), _ptr(idx),
                                 _ptr(scores), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def hf_block_select_hier(g: Geometry, q, ring: Ring, top_frames: int, top_k: int, idx, ws, frames=None,
                         scores=None, frame_scores=None, stream=None) -> None:
    _check("hf_block_select_hier",
           lib().hf_block_select_hier(ctypes.byref(g.dims()), _ptr(q), ctypes.byref(ring.desc), int(top_frames),
                                      int(top_k), _ptr(idx), _ptr(frames), _ptr(scores), _ptr(frame_scores),
                                      _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def hf_sparse_window_attn(g: Geometry, q, ring: Ring, idx, top_k: int, S, z, out, ws, eps=1e-6, stream=None) -> None:
    _check("hf_sparse_window_attn",
           lib().hf_sparse_window_attn(ctypes.byref(g.dims()), _ptr(q), ctypes.byref(ring.desc), _ptr(idx),
                                       int(top_k), _ptr(S), _ptr(z), float(eps), _ptr(out), _ptr(ws),
                                       ws.numel() if ws is not None else 0, _stream(stream)))


def hf_linear_absorb(g: Geometry, k_ev, v_ev, n_tok: int, S, z, ws, stream=None) -> None:
    _check("hf_linear_absorb",
           lib().hf_linear_absorb(ctypes.byref(g.dims()), _ptr(k_ev), _ptr(v_ev), int(n_tok), _ptr(S), _ptr(z),
                                  _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def hf_hybrid_step(g: Geometry, q, k_cur, v_cur, ring: Ring, top_k: int, flags: int, S, z, idx, out, ws,
                   eps=1e-6, events=None, stream=None) -> None:
    """`events`: None or a sequence of 6 raw hipEvent_t handles (ints or None)."""
    ev = None
    if events is not None:
        ev = StepEvents()
        for i, e in enumerate(events):
            ev.ev[i] = e
    _check("hf_hybrid_step",
           lib().hf_hybrid_step(ctypes.byref(g.dims()), _ptr(q), _ptr(k_cur), _ptr(v_cur), ctypes.byref(ring.desc),
                                int(top_k), int(flags), _ptr(S), _ptr(z), float(eps), _ptr(idx), _ptr(out), _ptr(ws),
                                ws.numel() if ws is not None else 0, ctypes.byref(ev) if ev is not None else None,
                                _stream(stream)))


def _events(events):
    if events is None:
        return None
    ev = StepEvents()
    for i, e in enumerate(events):
        ev.ev[i] = e
    return ctypes.byref(ev)


def hf_sparse_window_attn_rope(g: Geometry, q, ring: Ring, idx, top_k: int, S, z, out, ws, rope: Rope, eps=1e-6,
                               stream=None) -> None:
    _check("hf_sparse_window_attn_rope",
           lib().hf_sparse_window_attn_rope(ctypes.byref(g.dims()), _ptr(q), ctypes.byref(ring.desc), _ptr(idx),
                                            int(top_k), _ptr(S), _ptr(z), float(eps),
                                            ctypes.byref(rope) if rope is not None else None, _ptr(out), _ptr(ws),
                                            ws.numel() if ws is not None else 0, _stream(stream)))


def hf_hybrid_step_rope(g: Geometry, q, k_cur, v_cur, ring: Ring, top_k: int, flags: int, S, z, idx, out, ws,
                        rope: Rope, eps=1e-6, events=None, stream=None) -> None:
    _check("hf_hybrid_step_rope",
           lib().hf_hybrid_step_rope(ctypes.byref(g.dims()), _ptr(q), _ptr(k_cur), _ptr(v_cur),
                                     ctypes.byref(ring.desc), int(top_k), int(flags), _ptr(S), _ptr(z), float(eps),
                                     ctypes.byref(rope) if rope is not None else None, _ptr(idx), _ptr(out),
                                     _ptr(ws), ws.numel() if ws is not None else 0, _events(events),
                                     _stream(stream)))


def hf_cag_schedule(n_kb, s_base: float, s_target: float, s_max: float):
    """Chunk-aware growth schedule (host call).  Returns (top_k list, sparsity list, beta)."""
    n = len(n_kb)
    nkb = (ctypes.c_int32 * n)(*[int(x) for x in n_kb])
    k = (ctypes.c_int32 * n)()
    s = (ctypes.c_double * n)()
    beta = ctypes.c_double(0.0)
    _check("hf_cag_schedule", lib().hf_cag_schedule(n, nkb, float(s_base), float(s_target), float(s_max), k, s,
                                                    ctypes.byref(beta)))
    return list(k), list(s), beta.value


# ------------------------------------------------------------------ backward (training)

def backward_workspace_size(g: Geometry, top_k: int) -> int:
    n = ctypes.c_size_t(0)
    _check("hf_backward_workspace_size", lib().hf_backward_workspace_size(ctypes.byref(g.dims()), int(top_k),
                                                                          ctypes.byref(n)))
    return n.value


def new_backward_workspace(g: Geometry, top_k: int, device="cuda") -> torch.Tensor:
    return torch.empty(backward_workspace_size(g, top_k), dtype=torch.uint8, device=device)


def hf_sparse_window_attn_lse(g: Geometry, q, ring: Ring, idx, top_k: int, S, z, out, lse, ws, eps=1e-6,
                              stream=None) -> None:
    _check("hf_sparse_window_attn_lse",
           lib().hf_sparse_window_attn_lse(ctypes.byref(g.dims()), _ptr(q), ctypes.byref(ring.desc), _ptr(idx),
                                           int(top_k), _ptr(S), _ptr(z), float(eps), _ptr(out), _ptr(lse), _ptr(ws),
                                           ws.numel() if ws is not None else 0, _stream(stream)))


def hf_hybrid_attn_backward(g: Geometry, q, ring: Ring, idx, top_k: int, S, z, out, lse, dout, dq, dk, dv, dS, dz,
                            bws, eps=1e-6, stream=None) -> None:
    _check("hf_hybrid_attn_backward",
           lib().hf_hybrid_attn_backward(ctypes.byref(g.dims()), _ptr(q), ctypes.byref(ring.desc), _ptr(idx),
                                         int(top_k), _ptr(S), _ptr(z), float(eps), _ptr(out), _ptr(lse), _ptr(dout),
                                         _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dS), _ptr(dz), _ptr(bws),
                                         bws.numel() if bws is not None else 0, _stream(stream)))


def hf_linear_absorb_backward(g: Geometry, k_ev, v_ev, n_tok: int, dS, dz, dk, dv, ws, stream=None) -> None:
    _check("hf_linear_absorb_backward",
           lib().hf_linear_absorb_backward(ctypes.byref(g.dims()), _ptr(k_ev), _ptr(v_ev), int(n_tok), _ptr(dS),
                                           _ptr(dz), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel() if ws is not None else 0,
                                           _stream(stream)))
