"""GPU parity of the backward pass (hf_sparse_window_attn_lse, hf_hybrid_attn_backward,
hf_linear_absorb_backward, through the C ABI) against the fp64 oracle's backward, which is
itself pinned by finite differences (tests/test_oracle_bwd.py).

Bar (derived from the arithmetic): every matrix-core operand is bf16 (unit roundoff
2^-9 ~ 2e-3) and the softmax weights P and their gradients G are rounded to bf16 before
the products that use them, so each gradient term carries a relative error of a few
2^-9; sums of many such terms of both signs keep the relative error of each gradient at
a few 2^-9 as well (observed 1.5e-3 .. 6e-3).  Each gradient must reach relative
Frobenius error <= 1e-2 and max-abs error <= 2e-2 x max |oracle|; lse and the forward
output keep the forward's bar.
"""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf
import oracle
from hybrid_sparse_linear_hf_amd import synth

from gpu_helpers import StepInputs, assert_close, dev_bf16, fill_ring

pytestmark = pytest.mark.gpu

FRO_TOL = 1e-2
MAX_TOL = 2e-2


def grad_close(got, ref, what):
    got = got.astype(np.float64)
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300)
    print(f"{what}: fro {fro:.2e} max {mx:.2e}", flush=True)
    assert fro <= FRO_TOL and mx <= MAX_TOL, f"{what}: relative Frobenius {fro:.3e}, max {mx:.3e}"


def run_forward_backward(g, inp, ncom, top_k, S, z, dout, head=0, eps=1e-6):
    ring = hf.Ring(g)
    fill_ring(ring, inp.k_bits, inp.v_bits, ncom + g.C, head)
    ring.set_state(head, ncom)
    ws = hf.new_workspace(g)
    bws = hf.new_backward_workspace(g, top_k)
    q = dev_bf16(inp.q_bits)
    Nk = (ncom + g.C) * g.T
    idx = torch.empty((g.B, g.H, g.n_qb, top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((g.B, g.H, g.Nq, g.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((g.B, g.H, g.Nq), dtype=torch.float32, device="cuda")
    Sd = torch.from_numpy(S.astype(np.float32)).cuda()
    zd = torch.from_numpy(z.astype(np.float32)).cuda()
    dO = torch.from_numpy(dout.astype(np.float32)).cuda()
    dq = torch.full((g.B, g.H, g.Nq, g.D), float("nan"), device="cuda")
    dk = torch.full((g.B, g.H, Nk, g.D), float("nan"), device="cuda")
    dv = torch.full((g.B, g.H, Nk, g.D), float("nan"), device="cuda")
    dS = torch.full((g.B, g.H, g.D, g.D), float("nan"), device="cuda")
    dz = torch.full((g.B, g.H, g.D), float("nan"), device="cuda")
    hf.hf_block_select(g, q, ring, top_k, idx, None, ws)
    hf.hf_sparse_window_attn_lse(g, q, ring, idx, top_k, Sd, zd, out, lse, ws, eps=eps)
    hf.hf_hybrid_attn_backward(g, q, ring, idx, top_k, Sd, zd, out, lse, dO, dq, dk, dv, dS, dz, bws, eps=eps)
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in (idx, out, lse, dq, dk, dv, dS, dz))


def oracle_lse(Q, K, idx, bq, bk):
    """log2 of each query's softmax denominator over its kept keys (base-2 logits)."""
    B, H, Nq, D = Q.shape
    Nk = K.shape[2]
    L = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for t in range(Nq):
                keys = np.concatenate([np.arange(j * bk, min((j + 1) * bk, Nk)) for j in idx[b, h, t // bq]])
                s = K[b, h, keys] @ Q[b, h, t] / np.sqrt(D)
                m = s.max()
                L[b, h, t] = (m + np.log(np.exp(s - m).sum())) / np.log(2.0)
    return L


CASES = [
    # B, H, D, T, C, W, bq, bk, n_committed, top_k, seed
    (1, 1, 64, 64, 1, 4, 16, 16, 3, 2, 0),        # the tiny shapes
    (1, 2, 128, 200, 1, 3, 64, 64, 2, 3, 1),      # ragged query and key blocks
    (2, 1, 64, 96, 2, 4, 32, 16, 2, 5, 2),        # B=2, bq=32, bk=16, frames across blocks
    (1, 1, 128, 104, 1, 5, 16, 128, 1, 1, 3),     # bq=16, bk=128 (last block partial)
    (1, 2, 128, 136, 1, 4, 64, 64, 3, 4, 4),      # odd number of query blocks
    (1, 1, 64, 48, 4, 6, 64, 32, 2, 6, 5),        # D=64, T=48
    # 200 query blocks x 1400 key blocks: the selection's transpose is too large for its
    # LDS bitmap and takes the ordered fill
    (1, 1, 64, 800, 4, 28, 16, 16, 24, 3, 6),
]


@pytest.mark.parametrize("B,H,D,T,C,W,bq,bk,ncom,top_k,seed", CASES)
def test_backward_parity(B, H, D, T, C, W, bq, bk, ncom, top_k, seed):
    print(f"case: backward B={B} H={H} D={D} T={T} C={C} W={W} bq={bq} bk={bk} n_committed={ncom} k={top_k}",
          flush=True)
    g = hf.Geometry(B, H, D, T, C, W, bq, bk)
    rng = np.random.default_rng(100 + seed)
    nfr = ncom + C
    b = synth.bf16_bits_from_f32
    mk = lambda n: b(rng.standard_normal((B, H, n, D)).astype(np.float32))
    inp = StepInputs(mk(C * T), mk(nfr * T), mk(nfr * T))
    S = rng.standard_normal((B, H, D, D)) * 0.05
    z = rng.random((B, H, D)) * 10 + 1
    dout = rng.standard_normal((B, H, C * T, D))
    # the device takes fp32 state and gradient: give the oracle the same values
    S, z, dout = (x.astype(np.float32).astype(np.float64) for x in (S, z, dout))
    idx, out, lse, dq, dk, dv, dS, dz = run_forward_backward(g, inp, ncom, top_k, S, z, dout)
    ref_out = oracle.sparse_attn(inp.Q, inp.K, inp.V, idx, bq, bk) + oracle.linear_readout(inp.Q, S, z, bq=bq)
    assert_close(out, ref_out, "forward")
    L = oracle_lse(inp.Q, inp.K, idx, bq, bk)
    assert np.abs(lse - L).max() <= 1e-3 * max(1.0, np.abs(L).max()), np.abs(lse - L).max()
    rq, rk, rv, rS, rz = oracle.hybrid_step_bwd(inp.Q, inp.K, inp.V, S, z, idx, bq, bk, dout)
    for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv"), (dS, rS, "dS"), (dz, rz, "dz")):
        grad_close(got, ref, what)


def test_backward_832x480_two_heads():
    """The layer shapes (T=1560, C=3, W=6, 64x64 blocks, top-37) on two heads of the
    synthetic field, with the state built from 18 frames."""
    print("case: backward 832x480 layer, heads 0-1", flush=True)
    cfg = synth.LAYER_832x480
    heads = [0, 1]
    inp_d = synth.field_step_inputs(cfg, heads=heads)
    g = hf.Geometry(cfg.B, len(heads), cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    inp = StepInputs(inp_d["q"], inp_d["k_win"], inp_d["v_win"], inp_d["k_ev"], inp_d["v_ev"])
    S, z = oracle.absorb(inp.Kev, inp.Vev)
    rng = np.random.default_rng(11)
    dout = rng.standard_normal(inp.Q.shape).astype(np.float32).astype(np.float64)
    S, z = S.astype(np.float32).astype(np.float64), z.astype(np.float32).astype(np.float64)
    top_k = cfg.top_k()
    idx, out, lse, dq, dk, dv, dS, dz = run_forward_backward(g, inp, cfg.W - cfg.C, top_k, S, z, dout)
    rq, rk, rv, rS, rz = oracle.hybrid_step_bwd(inp.Q, inp.K, inp.V, S, z, idx, cfg.bq, cfg.bk, dout)
    for got, ref, what in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv"), (dS, rS, "dS"), (dz, rz, "dz")):
        grad_close(got, ref, what)


@pytest.mark.parametrize("n_tok", [1, 63, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_absorb_backward_parity(n_tok, D):
    print(f"case: absorb backward D={D} n_tok={n_tok}", flush=True)
    B, H = 1, 2
    g = hf.Geometry(B, H, D, 64, 1, 2, 64, 64)
    rng = np.random.default_rng(n_tok + D)
    b = synth.bf16_bits_from_f32
    kb = b(rng.standard_normal((B, H, n_tok, D)).astype(np.float32))
    vb = b(rng.standard_normal((B, H, n_tok, D)).astype(np.float32))
    dS = rng.standard_normal((B, H, D, D)).astype(np.float32).astype(np.float64)
    dz = rng.standard_normal((B, H, D)).astype(np.float32).astype(np.float64)
    ws = hf.new_workspace(g)
    dk = torch.full((B, H, n_tok, D), float("nan"), device="cuda")
    dv = torch.full((B, H, n_tok, D), float("nan"), device="cuda")
    hf.hf_linear_absorb_backward(g, dev_bf16(kb), dev_bf16(vb), n_tok, torch.from_numpy(dS.astype(np.float32)).cuda(),
                                 torch.from_numpy(dz.astype(np.float32)).cuda(), dk, dv, ws)
    torch.cuda.synchronize()
    rk, rv = oracle.absorb_bwd(synth.f64_from_bf16_bits(kb), synth.f64_from_bf16_bits(vb), dS, dz)
    grad_close(dk.cpu().numpy(), rk, "dk")
    grad_close(dv.cpu().numpy(), rv, "dv")
