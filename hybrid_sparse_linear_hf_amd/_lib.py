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
    _fields_ = [("k_dev", ctypes.c_void_p), ("vg_dev", ctypes.c_void_p), ("head", ctypes.c_int32),
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
        L.hf_hybrid_step_noalloc.argtypes = [pd, _P, _P, _P, pr, i32, u32, _P, _P, f32, _P, _P,
                                             ctypes.POINTER(StepEvents), _P]
        for fn in ("hf_workspace_size", "hf_ring_init", "hf_ring_append", "hf_block_select", "hf_sparse_window_attn",
                   "hf_linear_absorb", "hf_hybrid_step", "hf_cag_schedule", "hf_block_select_hier",
                   "hf_sparse_window_attn_lse", "hf_backward_workspace_size", "hf_hybrid_attn_backward",
                   "hf_linear_absorb_backward", "hf_sparse_window_attn_rope", "hf_hybrid_step_rope",
                   "hf_hybrid_step_noalloc"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != HF_OK:
        raise HFError(fn, status, lib().hf_last_error().decode())


_DTYPE_NAME = {torch.bfloat16: "bfloat16", torch.float32: "float32", torch.float64: "float64",
               torch.int32: "int32", torch.uint8: "uint8"}


class _T:
    """A checked tensor argument (or None), turned into a raw pointer by _call."""
    __slots__ = ("name", "t")

    def __init__(self, name: str, t):
        self.name, self.t = name, t


def _arg(fn: str, name: str, t, dtype, numel: int | None, optional: bool = False) -> _T:
    """Check one tensor argument before its pointer crosses the C ABI, which cannot see
    dtypes, strides, sizes or devices: `dtype`, a contiguous layout and exactly `numel`
    elements (None: any size).  The device is checked by _call, after every argument's
    format, so a call fails on the first malformed argument whatever its device."""
    if t is None:
        if optional:
            return _T(name, None)
        raise ValueError(f"{fn}: {name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{fn}: {name} must be a torch.Tensor, not {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{fn}: {name} must be {_DTYPE_NAME[dtype]}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous (shape {tuple(t.shape)}, strides {t.stride()})")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{fn}: {name} must hold {numel} elements, got {t.numel()} (shape {tuple(t.shape)})")
    return _T(name, t)


def _ws(fn: str, ws, name: str = "ws"):
    """(checked tensor, bytes) of a workspace: a contiguous uint8 tensor (size checked by the library)."""
    if ws is None:
        return _T(name, None), 0
    return _arg(fn, name, ws, torch.uint8, None), ws.numel()


def _call(fn: str, cfunc, *args) -> None:
    """Every checked tensor must live on a GPU; then call the C entry point with raw
    pointers in their place and raise HFError on a non-zero status."""
    for a in args:
        if isinstance(a, _T) and a.t is not None and a.t.device.type != "cuda":
            raise ValueError(f"{fn}: {a.name} must be on a GPU, got device {a.t.device}")
    raw = [((None if a.t is None else ctypes.c_void_p(a.t.data_ptr())) if isinstance(a, _T)
            else a.handle() if isinstance(a, _Stream) else a) for a in args]
    _check(fn, cfunc(*raw))


class _Stream:
    """The HIP stream argument (torch's current stream by default), resolved by _call."""
    __slots__ = ("s",)

    def __init__(self, s):
        self.s = s

    def handle(self):
        s = torch.cuda.current_stream() if self.s is None else self.s
        return ctypes.c_void_p(s.cuda_stream)


def _stream(stream=None) -> _Stream:
    return _Stream(stream)


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
    """Device storage of the KV ring (keys [B,H,W,T,D], values in 8-token groups
    [B,H,W,T/8,D,8]) plus the host descriptor (head, n_committed)."""

    def __init__(self, g: Geometry, device="cuda"):
        self.g = g
        self.k = torch.zeros((g.B, g.H, g.W, g.T, g.D), dtype=torch.bfloat16, device=device)
        self.vg = torch.zeros((g.B, g.H, g.W, g.T // 8, g.D, 8), dtype=torch.bfloat16, device=device)
        self.desc = KVRing()
        _check("hf_ring_init", lib().hf_ring_init(ctypes.byref(g.dims()), self.k.data_ptr(), self.vg.data_ptr(),
                                                  ctypes.byref(self.desc)))

    @staticmethod
    def grouped(v: "torch.Tensor") -> "torch.Tensor":
        """Values [..., T, D] in the ring's value layout [..., T/8, D, 8]."""
        *lead, t, d = v.shape
        return v.reshape(*lead, t // 8, 8, d).transpose(-1, -2)

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
# Each wrapper checks its tensors against the geometry (dtype, contiguity, element count,
# device) before anything reaches the library, then passes the raw pointers.

_BF16, _F32, _F64, _I32 = torch.bfloat16, torch.float32, torch.float64, torch.int32


def _planes(g: Geometry) -> int:
    return g.B * g.H


def _state_args(fn: str, g: Geometry, S, z, optional: bool):
    BH, D = _planes(g), g.D
    if (S is None) != (z is None):
        raise ValueError(f"{fn}: give both S and z or neither")
    return (_arg(fn, "S", S, _F32, BH * D * D, optional), _arg(fn, "z", z, _F32, BH * D, optional))


def _events(events):
    if events is None:
        return None
    ev = StepEvents()
    for i, e in enumerate(events):
        ev.ev[i] = e
    return ctypes.byref(ev)


def hf_ring_append(g: Geometry, ring: Ring, k_cur, v_cur, stream=None) -> None:
    fn, n = "hf_ring_append", _planes(g) * g.Nq * g.D
    kp, vp = _arg(fn, "k_cur", k_cur, _BF16, n), _arg(fn, "v_cur", v_cur, _BF16, n)
    _call(fn, lib().hf_ring_append, ctypes.byref(g.dims()), ctypes.byref(ring.desc), kp, vp, _stream(stream))


def hf_block_select(g: Geometry, q, ring: Ring, top_k: int, idx, scores, ws, stream=None) -> None:
    fn, BH, nkb = "hf_block_select", _planes(g), g.n_kb(ring.n_committed)
    qp = _arg(fn, "q", q, _BF16, BH * g.Nq * g.D)
    ip = _arg(fn, "idx", idx, _I32, BH * g.n_qb * int(top_k))
    sp = _arg(fn, "scores", scores, _F64, BH * g.n_qb * nkb, optional=True)
    wp, wn = _ws(fn, ws)
    _call(fn, lib().hf_block_select, ctypes.byref(g.dims()), qp, ctypes.byref(ring.desc), int(top_k), ip, sp, wp, wn,
                                     _stream(stream))


def hf_block_select_hier(g: Geometry, q, ring: Ring, top_frames: int, top_k: int, idx, ws, frames=None,
                         scores=None, frame_scores=None, stream=None) -> None:
    fn, BH, nkb = "hf_block_select_hier", _planes(g), g.n_kb(ring.n_committed)
    nfr = ring.n_committed + g.C
    qp = _arg(fn, "q", q, _BF16, BH * g.Nq * g.D)
    ip = _arg(fn, "idx", idx, _I32, BH * g.n_qb * int(top_k))
    fp = _arg(fn, "frames", frames, _I32, BH * g.n_qb * int(top_frames), optional=True)
    sp = _arg(fn, "scores", scores, _F64, BH * g.n_qb * nkb, optional=True)
    fsp = _arg(fn, "frame_scores", frame_scores, _F64, BH * g.n_qb * nfr, optional=True)
    wp, wn = _ws(fn, ws)
    _call(fn, lib().hf_block_select_hier, ctypes.byref(g.dims()), qp, ctypes.byref(ring.desc), int(top_frames),
                                          int(top_k), ip, fp, sp, fsp, wp, wn, _stream(stream))


def _attn_args(fn: str, g: Geometry, q, idx, top_k: int, S, z, out):
    BH = _planes(g)
    qp = _arg(fn, "q", q, _BF16, BH * g.Nq * g.D)
    ip = _arg(fn, "idx", idx, _I32, BH * g.n_qb * int(top_k))
    Sp, zp = _state_args(fn, g, S, z, optional=True)
    op = _arg(fn, "out", out, _F32, BH * g.Nq * g.D)
    return qp, ip, Sp, zp, op


def hf_sparse_window_attn(g: Geometry, q, ring: Ring, idx, top_k: int, S, z, out, ws, eps=1e-6, stream=None) -> None:
    fn = "hf_sparse_window_attn"
    qp, ip, Sp, zp, op = _attn_args(fn, g, q, idx, top_k, S, z, out)
    wp, wn = _ws(fn, ws)
    _call(fn, lib().hf_sparse_window_attn, ctypes.byref(g.dims()), qp, ctypes.byref(ring.desc), ip, int(top_k), Sp,
                                           zp, float(eps), op, wp, wn, _stream(stream))


def hf_linear_absorb(g: Geometry, k_ev, v_ev, n_tok: int, S, z, ws, stream=None) -> None:
    fn, n = "hf_linear_absorb", _planes(g) * int(n_tok) * g.D
    opt = int(n_tok) == 0
    kp, vp = _arg(fn, "k_ev", k_ev, _BF16, n, opt), _arg(fn, "v_ev", v_ev, _BF16, n, opt)
    Sp, zp = _state_args(fn, g, S, z, optional=False)
    wp, wn = _ws(fn, ws)
    _call(fn, lib().hf_linear_absorb, ctypes.byref(g.dims()), kp, vp, int(n_tok), Sp, zp, wp, wn, _stream(stream))


def _step_args(fn: str, g: Geometry, q, k_cur, v_cur, top_k: int, S, z, idx, out):
    BH = _planes(g)
    n = BH * g.Nq * g.D
    qp = _arg(fn, "q", q, _BF16, n)
    if (k_cur is None) != (v_cur is None):
        raise ValueError(f"{fn}: give both k_cur and v_cur or neither")
    kp, vp = _arg(fn, "k_cur", k_cur, _BF16, n, True), _arg(fn, "v_cur", v_cur, _BF16, n, True)
    Sp, zp = _state_args(fn, g, S, z, optional=True)
    ip = _arg(fn, "idx", idx, _I32, BH * g.n_qb * int(top_k))
    op = _arg(fn, "out", out, _F32, n)
    return qp, kp, vp, Sp, zp, ip, op


def hf_hybrid_step(g: Geometry, q, k_cur, v_cur, ring: Ring, top_k: int, flags: int, S, z, idx, out, ws,
                   eps=1e-6, events=None, stream=None) -> None:
    """`events`: None or a sequence of 6 raw hipEvent_t handles (ints or None)."""
    fn = "hf_hybrid_step"
    qp, kp, vp, Sp, zp, ip, op = _step_args(fn, g, q, k_cur, v_cur, top_k, S, z, idx, out)
    wp, wn = _ws(fn, ws)
    _call(fn, lib().hf_hybrid_step, ctypes.byref(g.dims()), qp, kp, vp, ctypes.byref(ring.desc), int(top_k),
                                    int(flags), Sp, zp, float(eps), ip, op, wp, wn, _events(events), _stream(stream))


def hf_hybrid_step_noalloc(g: Geometry, q, k_cur, v_cur, ring: Ring, top_k: int, flags: int, S, z, idx, out,
                           eps=1e-6, events=None, stream=None) -> None:
    """hf_hybrid_step without a workspace: the library's fixed per-GPU scratch array holds the
    step's transient data (calls overlapping in time on one GPU race on it)."""
    fn = "hf_hybrid_step_noalloc"
    qp, kp, vp, Sp, zp, ip, op = _step_args(fn, g, q, k_cur, v_cur, top_k, S, z, idx, out)
    _call(fn, lib().hf_hybrid_step_noalloc, ctypes.byref(g.dims()), qp, kp, vp, ctypes.byref(ring.desc), int(top_k),
          int(flags), Sp, zp, float(eps), ip, op, _events(events), _stream(stream))


def hf_sparse_window_attn_rope(g: Geometry, q, ring: Ring, idx, top_k: int, S, z, out, ws, rope: Rope, eps=1e-6,
                               stream=None) -> None:
    fn = "hf_sparse_window_attn_rope"
    qp, ip, Sp, zp, op = _attn_args(fn, g, q, idx, top_k, S, z, out)
    wp, wn = _ws(fn, ws)
    _call(fn, lib().hf_sparse_window_attn_rope, ctypes.byref(g.dims()), qp, ctypes.byref(ring.desc), ip, int(top_k),
                                                Sp, zp, float(eps), ctypes.byref(rope) if rope is not None else None,
                                                op, wp, wn, _stream(stream))


def hf_hybrid_step_rope(g: Geometry, q, k_cur, v_cur, ring: Ring, top_k: int, flags: int, S, z, idx, out, ws,
                        rope: Rope, eps=1e-6, events=None, stream=None) -> None:
    fn = "hf_hybrid_step_rope"
    qp, kp, vp, Sp, zp, ip, op = _step_args(fn, g, q, k_cur, v_cur, top_k, S, z, idx, out)
    wp, wn = _ws(fn, ws)
    _call(fn, lib().hf_hybrid_step_rope, ctypes.byref(g.dims()), qp, kp, vp, ctypes.byref(ring.desc), int(top_k),
                                         int(flags), Sp, zp, float(eps),
                                         ctypes.byref(rope) if rope is not None else None, ip, op, wp, wn,
                                         _events(events), _stream(stream))


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
    fn = "hf_sparse_window_attn_lse"
    qp, ip, Sp, zp, op = _attn_args(fn, g, q, idx, top_k, S, z, out)
    lp = _arg(fn, "lse", lse, _F32, _planes(g) * g.Nq)
    wp, wn = _ws(fn, ws)
    _call(fn, lib().hf_sparse_window_attn_lse, ctypes.byref(g.dims()), qp, ctypes.byref(ring.desc), ip, int(top_k),
                                               Sp, zp, float(eps), op, lp, wp, wn, _stream(stream))


def hf_hybrid_attn_backward(g: Geometry, q, ring: Ring, idx, top_k: int, S, z, out, lse, dout, dq, dk, dv, dS, dz,
                            bws, eps=1e-6, stream=None) -> None:
    fn, BH = "hf_hybrid_attn_backward", _planes(g)
    nq, nk = BH * g.Nq * g.D, BH * (ring.n_committed + g.C) * g.T * g.D
    qp, ip, Sp, zp, op = _attn_args(fn, g, q, idx, top_k, S, z, out)
    if Sp.t is None:
        raise ValueError(f"{fn}: S and z are required")
    lp = _arg(fn, "lse", lse, _F32, BH * g.Nq)
    gp = _arg(fn, "dout", dout, _F32, nq)
    dqp = _arg(fn, "dq", dq, _F32, nq)
    dkp, dvp = _arg(fn, "dk", dk, _F32, nk), _arg(fn, "dv", dv, _F32, nk)
    dSp, dzp = _arg(fn, "dS", dS, _F32, BH * g.D * g.D), _arg(fn, "dz", dz, _F32, BH * g.D)
    wp, wn = _ws(fn, bws, "bws")
    _call(fn, lib().hf_hybrid_attn_backward, ctypes.byref(g.dims()), qp, ctypes.byref(ring.desc), ip, int(top_k), Sp,
                                             zp, float(eps), op, lp, gp, dqp, dkp, dvp, dSp, dzp, wp, wn,
                                             _stream(stream))


def hf_linear_absorb_backward(g: Geometry, k_ev, v_ev, n_tok: int, dS, dz, dk, dv, ws, stream=None) -> None:
    fn, BH = "hf_linear_absorb_backward", _planes(g)
    n = BH * int(n_tok) * g.D
    opt = int(n_tok) == 0
    kp, vp = _arg(fn, "k_ev", k_ev, _BF16, n, opt), _arg(fn, "v_ev", v_ev, _BF16, n, opt)
    dSp, dzp = _arg(fn, "dS", dS, _F32, BH * g.D * g.D), _arg(fn, "dz", dz, _F32, BH * g.D)
    dkp, dvp = _arg(fn, "dk", dk, _F32, n, opt), _arg(fn, "dv", dv, _F32, n, opt)
    wp, wn = _ws(fn, ws)
    _call(fn, lib().hf_linear_absorb_backward, ctypes.byref(g.dims()), kp, vp, int(n_tok), dSp, dzp, dkp, dvp, wp, wn,
                                               _stream(stream))
