"""The Python binding checks every tensor against the geometry before its pointer crosses
the C ABI (which cannot see dtypes, strides, sizes or devices).  These run on the CPU: a
tensor with the right dtype, layout and size but on the CPU is rejected last, by the
device check, so no call ever reaches the library's compute entry points here."""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf

G = hf.Geometry(B=1, H=2, D=64, T=64, C=1, W=4, bq=16, bk=16)
TOP_K = 3


def ring():
    r = hf.Ring(G, device="cpu")
    r.set_state(0, G.W - G.C)
    return r


def ws():
    return torch.zeros(1024, dtype=torch.uint8)


def q(dtype=torch.bfloat16):
    return torch.zeros((G.B, G.H, G.Nq, G.D), dtype=dtype)


def idx(k=TOP_K, dtype=torch.int32):
    return torch.zeros((G.B, G.H, G.n_qb, k), dtype=dtype)


def state():
    return torch.zeros((G.B, G.H, G.D, G.D)), torch.zeros((G.B, G.H, G.D))


def out():
    return torch.zeros((G.B, G.H, G.Nq, G.D))


def attn(**kw):
    S, z = state()
    args = dict(q=q(), idx=idx(), S=S, z=z, out=out(), ws=ws())
    args.update(kw)
    hf.hf_sparse_window_attn(G, args["q"], ring(), args["idx"], TOP_K, args["S"], args["z"], args["out"], args["ws"])


def test_wrong_dtype_rejected():
    with pytest.raises(TypeError, match="q must be bfloat16"):
        attn(q=q(torch.float32))
    with pytest.raises(TypeError, match="idx must be int32"):
        attn(idx=idx(dtype=torch.int64))
    with pytest.raises(TypeError, match="out must be float32"):
        attn(out=out().to(torch.bfloat16))
    with pytest.raises(TypeError, match="S must be float32"):
        attn(S=state()[0].double())
    with pytest.raises(TypeError, match="ws must be uint8"):
        attn(ws=torch.zeros(256, dtype=torch.float32))


def test_non_contiguous_rejected():
    qt = torch.zeros((G.B, G.H, G.D, G.Nq), dtype=torch.bfloat16).transpose(-1, -2)
    assert qt.shape == q().shape
    with pytest.raises(ValueError, match="q must be contiguous"):
        attn(q=qt)
    S, _ = state()
    with pytest.raises(ValueError, match="S must be contiguous"):
        attn(S=S.transpose(-1, -2))


def test_wrong_size_rejected():
    with pytest.raises(ValueError, match="out must hold"):
        attn(out=torch.zeros((G.B, G.H, G.Nq - 1, G.D)))
    with pytest.raises(ValueError, match="idx must hold"):
        attn(idx=idx(k=TOP_K + 1))
    with pytest.raises(ValueError, match="z must hold"):
        attn(z=torch.zeros((G.B, G.H, G.D + 1)))


def test_non_tensor_and_missing_rejected():
    with pytest.raises(TypeError, match="must be a torch.Tensor"):
        attn(q=np.zeros((G.B, G.H, G.Nq, G.D), dtype=np.uint16))
    with pytest.raises(ValueError, match="q is required"):
        attn(q=None)
    with pytest.raises(ValueError, match="both S and z"):
        attn(z=None)


def test_cpu_tensor_rejected_by_device_check():
    with pytest.raises(ValueError, match="must be on a GPU"):
        attn()


def test_select_and_step_checks():
    r = ring()
    nkb = G.n_kb(r.n_committed)
    with pytest.raises(ValueError, match="scores must hold"):
        hf.hf_block_select(G, q(), r, TOP_K, idx(), torch.zeros((G.B, G.H, G.n_qb, nkb + 1), dtype=torch.float64), ws())
    with pytest.raises(TypeError, match="scores must be float64"):
        hf.hf_block_select(G, q(), r, TOP_K, idx(), torch.zeros((G.B, G.H, G.n_qb, nkb)), ws())
    S, z = state()
    with pytest.raises(ValueError, match="both k_cur and v_cur"):
        hf.hf_hybrid_step(G, q(), q(), None, r, TOP_K, hf.HF_STEP_COMMIT, S, z, idx(), out(), ws())
    with pytest.raises(ValueError, match="k_cur must hold"):
        hf.hf_hybrid_step(G, q(), torch.zeros(7, dtype=torch.bfloat16), q(), r, TOP_K, 1, S, z, idx(), out(), ws())
    with pytest.raises(ValueError, match="must be on a GPU"):
        hf.hf_hybrid_step(G, q(), q(), q(), r, TOP_K, hf.HF_STEP_COMMIT, S, z, idx(), out(), ws())
    # the descriptor is untouched by a rejected call
    assert (r.head, r.n_committed) == (0, G.W - G.C)


def test_absorb_and_backward_checks():
    S, z = state()
    n_tok = 10
    kv = torch.zeros((G.B, G.H, n_tok, G.D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="v_ev must hold"):
        hf.hf_linear_absorb(G, kv, kv[:, :, :5].contiguous(), n_tok, S, z, ws())
    with pytest.raises(ValueError, match="S is required"):
        hf.hf_linear_absorb(G, kv, kv, n_tok, None, None, ws())
    r = ring()
    nk = (r.n_committed + G.C) * G.T
    lse = torch.zeros((G.B, G.H, G.Nq))
    grads = dict(dq=out(), dk=torch.zeros((G.B, G.H, nk, G.D)), dv=torch.zeros((G.B, G.H, nk, G.D)),
                 dS=torch.zeros_like(S), dz=torch.zeros_like(z))

    def bwd(**kw):
        a = dict(grads)
        a.update(kw)
        hf.hf_hybrid_attn_backward(G, q(), r, idx(), TOP_K, S, z, out(), lse, out(), a["dq"], a["dk"], a["dv"],
                                   a["dS"], a["dz"], ws())

    with pytest.raises(ValueError, match="dk must hold"):
        bwd(dk=torch.zeros((G.B, G.H, nk - G.T, G.D)))
    with pytest.raises(TypeError, match="dv must be float32"):
        bwd(dv=torch.zeros((G.B, G.H, nk, G.D), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must be on a GPU"):
        bwd()
    with pytest.raises(ValueError, match="dk must hold"):
        hf.hf_linear_absorb_backward(G, kv, kv, n_tok, S, z, torch.zeros(3), torch.zeros(3), ws())
