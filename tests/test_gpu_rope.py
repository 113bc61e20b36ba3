"""GPU parity of the attention with the relative temporal rotary embedding (called through
the C ABI) against the fp64 oracle: block indices bit-exact (the selection is unchanged by
the rotation), outputs within max-abs 1e-2 and mean-relative 2e-3.  The turned query is a
bf16 matrix-core operand on the GPU and exact in the oracle; that rounding is inside the
bar."""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf
import oracle
from hybrid_sparse_linear_hf_amd import synth

from gpu_helpers import StepInputs, assert_close, dev_bf16, fill_ring, rows_of_blocks

pytestmark = pytest.mark.gpu

BASE = 10000.0


def state_of(g, inp, ws):
    S = torch.zeros((g.B, g.H, g.D, g.D), dtype=torch.float32, device="cuda")
    z = torch.zeros((g.B, g.H, g.D), dtype=torch.float32, device="cuda")
    hf.hf_linear_absorb(g, dev_bf16(inp.kev_bits), dev_bf16(inp.vev_bits), inp.kev_bits.shape[2], S, z, ws)
    return S, z


def random_inputs(B, H, D, T, C, ncom, seed):
    rng = np.random.default_rng(seed)
    b = synth.bf16_bits_from_f32
    mk = lambda n: b(rng.standard_normal((B, H, n, D)).astype(np.float32))
    nfr = ncom + C
    return StepInputs(mk(C * T), mk(nfr * T), mk(nfr * T), mk(2 * T + 8), mk(2 * T + 8))


CASES = [
    # B, H, D, T, C, W, bq, bk, n_committed, top_k, temporal_dims, cap
    (1, 2, 128, 200, 1, 3, 64, 64, 2, 3, 32, 1),     # ragged blocks; the cap binds at offset 2
    (2, 1, 64, 96, 2, 4, 32, 16, 2, 5, 16, 3),       # D=64, bq=32, bk=16 (online path)
    (1, 1, 128, 104, 1, 5, 16, 128, 1, 1, 32, 0),    # cap 0: plain scores
    (1, 2, 128, 24, 3, 8, 64, 32, 5, 4, 32, 2),      # 24-token frames: subtiles over two or three frames
    (1, 1, 64, 48, 4, 6, 64, 64, 2, 4, 16, 2),       # negative offsets inside a 4-frame chunk
    (1, 2, 128, 136, 3, 6, 64, 32, 3, 9, 32, 10),    # cap beyond the window: unclamped rotary
    (1, 3, 64, 40, 3, 7, 32, 128, 4, 3, 32, 1),      # key blocks longer than a frame
    (1, 2, 128, 96, 2, 5, 64, 64, 3, 7, 16, 4),      # full 32-key subtiles crossing frames
]


@pytest.mark.parametrize("B,H,D,T,C,W,bq,bk,ncom,top_k,dt,cap", CASES)
def test_rope_attention_parity(B, H, D, T, C, W, bq, bk, ncom, top_k, dt, cap):
    print(f"case: rope B={B} H={H} D={D} T={T} C={C} W={W} bq={bq} bk={bk} ncom={ncom} k={top_k} dt={dt} cap={cap}",
          flush=True)
    g = hf.Geometry(B, H, D, T, C, W, bq, bk)
    inp = random_inputs(B, H, D, T, C, ncom, seed=B * 7919 + T * 31 + cap)
    head = min(2, W - 1)
    ring = hf.Ring(g)
    fill_ring(ring, inp.k_bits, inp.v_bits, ncom + C, head)
    ring.set_state(head, ncom)
    ws = hf.new_workspace(g)
    S, z = state_of(g, inp, ws)
    q = dev_bf16(inp.q_bits)
    idx = torch.empty((B, H, g.n_qb, top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, g.Nq, D), dtype=torch.float32, device="cuda")
    hf.hf_block_select(g, q, ring, top_k, idx, None, ws)
    hf.hf_sparse_window_attn_rope(g, q, ring, idx, top_k, S, z, out, ws, hf.Rope(dt, cap, BASE))
    torch.cuda.synchronize()
    So, zo = oracle.absorb(inp.Kev, inp.Vev)
    ref, idx_o = oracle.hybrid_step_rope(inp.Q, inp.K, inp.V, So, zo, bq, bk, top_k, T, dt, cap, BASE)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    mx, mr = assert_close(out.cpu().numpy(), ref, "rope")
    print(f"rope: max-abs {mx:.2e} mean-rel {mr:.2e}")


def test_rope_changes_the_output():
    """The rotated path is not the plain one on the same inputs (offsets within the cap)."""
    g = hf.Geometry(1, 1, 128, 96, 2, 5, 64, 64)
    inp = random_inputs(1, 1, 128, 96, 2, 3, seed=3)
    ring = hf.Ring(g)
    fill_ring(ring, inp.k_bits, inp.v_bits, 5, 0)
    ring.set_state(0, 3)
    ws = hf.new_workspace(g)
    q = dev_bf16(inp.q_bits)
    idx = torch.empty((1, 1, g.n_qb, 8), dtype=torch.int32, device="cuda")
    hf.hf_block_select(g, q, ring, 8, idx, None, ws)
    a = torch.empty((1, 1, g.Nq, 128), dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    hf.hf_sparse_window_attn(g, q, ring, idx, 8, None, None, a, ws)
    hf.hf_sparse_window_attn_rope(g, q, ring, idx, 8, None, None, b, ws, hf.Rope(32, 8, BASE))
    torch.cuda.synchronize()
    ref = oracle.sparse_attn_rope(inp.Q, inp.K, inp.V, idx.cpu().numpy(), 64, 64, 96, 32, 8, BASE)
    assert_close(b.cpu().numpy(), ref, "rope, sparse part only")
    assert float((a - b).abs().max()) > 0.05


def test_rope_step_layer_832x480():
    """The step with the rotation at the 832x480 layer shape (heads 0 and 7 of 12), in the
    launch configuration the benchmark times, on sampled query blocks."""
    print("case: rope step 832x480 (H=2 of 12, dt=32, cap=3)", flush=True)
    cfg = synth.LAYER_832x480
    d = synth.field_step_inputs(cfg, heads=[0, 7])
    inp = StepInputs(d["q"], d["k_win"], d["v_win"], d["k_ev"], d["v_ev"])
    g = hf.Geometry(cfg.B, 2, cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    ncom, k = cfg.W - cfg.C, cfg.top_k()
    ring = hf.Ring(g)
    fill_ring(ring, inp.k_bits, inp.v_bits, ncom + cfg.C, 1)
    ring.set_state(1, ncom)
    ws = hf.new_workspace(g)
    S, z = state_of(g, inp, ws)
    idx = torch.empty((1, 2, g.n_qb, k), dtype=torch.int32, device="cuda")
    out = torch.empty((1, 2, g.Nq, cfg.D), dtype=torch.float32, device="cuda")
    hf.hf_hybrid_step_rope(g, dev_bf16(inp.q_bits), None, None, ring, k, 0, S, z, idx, out, ws, hf.Rope(32, 3, BASE))
    torch.cuda.synchronize()
    blocks = sorted({(p, i) for p in range(2) for i in range(p % 7, g.n_qb, 7)} | {(p, g.n_qb - 1) for p in range(2)})
    So, zo = oracle.absorb(inp.Kev, inp.Vev)
    ref, idx_o = oracle.hybrid_step_rope(inp.Q, inp.K, inp.V, So, zo, cfg.bq, cfg.bk, k, cfg.T, 32, 3, BASE,
                                         blocks=blocks)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    rows = rows_of_blocks(blocks, g.Nq, cfg.bq, (2, g.Nq))
    mx, mr = assert_close(out.cpu().numpy().reshape(2, g.Nq, -1)[rows], ref.reshape(2, g.Nq, -1)[rows],
                          "rope step 832x480")
    print(f"rope step 832x480: {len(blocks)} blocks, max-abs {mx:.2e} mean-rel {mr:.2e}")


def test_rope_step_commit_stream():
    """Three committed steps with the rotation: outputs and the state track the oracle's
    window (the rotation touches neither the ring nor the state)."""
    g = hf.Geometry(B=1, H=2, D=128, T=96, C=2, W=5, bq=64, bk=32)
    rope = hf.Rope(16, 2, 500.0)
    rng = np.random.default_rng(21)
    b = synth.bf16_bits_from_f32
    shape = (g.B, g.H, g.C * g.T, g.D)
    ring = hf.Ring(g)
    ws = hf.new_workspace(g)
    S = torch.zeros((g.B, g.H, g.D, g.D), dtype=torch.float32, device="cuda")
    z = torch.zeros((g.B, g.H, g.D), dtype=torch.float32, device="cuda")
    fk, fv = [], []
    So, zo = np.zeros((1, 2, 128, 128)), np.zeros((1, 2, 128))
    for step in range(4):
        q, k, v = (b(rng.standard_normal(shape).astype(np.float32)) for _ in range(3))
        top_k = max(1, g.n_kb(ring.n_committed) // 3)
        idx = torch.empty((1, 2, g.n_qb, top_k), dtype=torch.int32, device="cuda")
        out = torch.empty((1, 2, g.Nq, g.D), dtype=torch.float32, device="cuda")
        hf.hf_hybrid_step_rope(g, dev_bf16(q), dev_bf16(k), dev_bf16(v), ring, top_k, hf.HF_STEP_COMMIT, S, z, idx,
                               out, ws, rope)
        torch.cuda.synchronize()
        Q, Kc, Vc = (synth.f64_from_bf16_bits(x) for x in (q, k, v))
        K = np.concatenate(fk + [Kc], axis=2)
        V = np.concatenate(fv + [Vc], axis=2)
        ref, idx_o = oracle.hybrid_step_rope(Q, K, V, So, zo, g.bq, g.bk, top_k, g.T, 16, 2, 500.0)
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
        assert_close(out.cpu().numpy(), ref, f"rope stream step {step}")
        for c in range(g.C):
            fk.append(Kc[:, :, c * g.T:(c + 1) * g.T])
            fv.append(Vc[:, :, c * g.T:(c + 1) * g.T])
        excess = len(fk) - (g.W - g.C)
        if excess > 0:
            So, zo = oracle.absorb(np.concatenate(fk[:excess], axis=2), np.concatenate(fv[:excess], axis=2), So, zo)
            del fk[:excess], fv[:excess]
    Sg = S.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(Sg - So) / np.linalg.norm(So) < 2e-3
