"""GPU parity of the HIP path (called through the C ABI) against the fp64 oracle.

Bar: block indices bit-exact (the GPU pools and scores in fp64 in the oracle's summation
order, so near-ties are resolved identically); outputs within max-abs 1e-2 and
mean-relative 2e-3 of the oracle; the state within a relative Frobenius error of 2e-3.
"""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf
import oracle
from hybrid_sparse_linear_hf_amd import synth

from gpu_helpers import StepInputs, assert_close, compare, dev_bf16, f64, fill_ring, rows_of_blocks

pytestmark = pytest.mark.gpu


def run_select_attn(g, inp, n_committed, top_k, head=0, with_state=True, S=None, z=None):
    """Fill a ring with the window, run select + sparse attention (+ readout).  Returns
    (idx, scores, out, S, z) as numpy."""
    ring = hf.Ring(g)
    nfr = n_committed + g.C
    fill_ring(ring, inp.k_bits, inp.v_bits, nfr, head)
    ring.set_state(head, n_committed)
    ws = hf.new_workspace(g)
    q = dev_bf16(inp.q_bits)
    nkb = g.n_kb(n_committed)
    idx = torch.empty((g.B, g.H, g.n_qb, top_k), dtype=torch.int32, device="cuda")
    scores = torch.empty((g.B, g.H, g.n_qb, nkb), dtype=torch.float64, device="cuda")
    out = torch.empty((g.B, g.H, g.Nq, g.D), dtype=torch.float32, device="cuda")
    if with_state and S is None:
        S = torch.zeros((g.B, g.H, g.D, g.D), dtype=torch.float32, device="cuda")
        z = torch.zeros((g.B, g.H, g.D), dtype=torch.float32, device="cuda")
        if inp.kev_bits is not None:
            n_ev = inp.kev_bits.shape[2]
            hf.hf_linear_absorb(g, dev_bf16(inp.kev_bits), dev_bf16(inp.vev_bits), n_ev, S, z, ws)
    hf.hf_block_select(g, q, ring, top_k, idx, scores, ws)
    hf.hf_sparse_window_attn(g, q, ring, idx, top_k, S if with_state else None, z if with_state else None, out, ws)
    torch.cuda.synchronize()
    res = (idx.cpu().numpy(), scores.cpu().numpy(), out.cpu().numpy())
    st = (S.cpu().numpy().astype(np.float64), z.cpu().numpy().astype(np.float64)) if with_state else (None, None)
    return res + st


def tiny_inputs():
    cfg = synth.TINY
    st = synth.tiny_stream(seed=0)
    T, ev = cfg.T, cfg.n_evicted
    b = synth.bf16_bits_from_f32
    return cfg, StepInputs(b(st.q), b(st.k_all[:, :, ev * T:]), b(st.v_all[:, :, ev * T:]),
                           b(st.k_all[:, :, :ev * T]), b(st.v_all[:, :, :ev * T]))


def geometry(cfg):
    return hf.Geometry(cfg.B, cfg.H, cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)


def test_tiny_step_parity():
    print("case: tiny config (D=64, T=64, W=4, block 16, top-2)", flush=True)
    cfg, inp = tiny_inputs()
    g = geometry(cfg)
    k = cfg.top_k()
    idx, sc, out, S, z = run_select_attn(g, inp, cfg.W - cfg.C, k)
    So, zo = oracle.absorb(inp.Kev, inp.Vev)
    ref, idx_o, sc_o = oracle.hybrid_step(inp.Q, inp.K, inp.V, So, zo, cfg.bq, cfg.bk, k, want_scores=True)
    np.testing.assert_array_equal(sc, sc_o)
    np.testing.assert_array_equal(idx, idx_o)
    assert np.linalg.norm(S - So) / np.linalg.norm(So) < 1e-5
    assert np.linalg.norm(z - zo) / np.linalg.norm(zo) < 1e-6
    mx, mr = assert_close(out, ref, "tiny step")
    print(f"tiny: max-abs {mx:.2e} mean-rel {mr:.2e}")


def test_tiny_sparse_only_and_keep_all():
    print("case: tiny config, sparse part only and keep-all", flush=True)
    cfg, inp = tiny_inputs()
    g = geometry(cfg)
    for k in (cfg.top_k(), 16):
        idx, _, out, _, _ = run_select_attn(g, inp, cfg.W - cfg.C, k, with_state=False)
        ref = oracle.sparse_attn(inp.Q, inp.K, inp.V, idx, cfg.bq, cfg.bk)
        assert_close(out, ref, f"sparse k={k}")
    np.testing.assert_array_equal(idx[0, 0, 0], np.arange(16))


def layer_inputs(cfg, heads=None):
    d = synth.field_step_inputs(cfg, heads=heads)
    return StepInputs(d["q"], d["k_win"], d["v_win"], d["k_ev"], d["v_ev"])


def sample_blocks(BH, nqb, stride=9):
    blocks = [(p, i) for p in range(BH) for i in range(p % stride, nqb, stride)]
    blocks += [(p, nqb - 1) for p in range(BH)]  # the ragged last block of every plane
    return sorted(set(blocks))


def test_layer_832x480_parity():
    """12 heads x 128, 4680 queries, 9360-key window, 64x64 blocks, 37 of 147 kept, state of 18
    frames: every score, kept list and output row."""
    print("case: 832x480 layer (H=12, D=128, T=1560, C=3, W=6, top-37)", flush=True)
    cfg = synth.LAYER_832x480
    g = geometry(cfg)
    inp = layer_inputs(cfg)
    k = cfg.top_k()
    idx, sc, out, S, z = run_select_attn(g, inp, cfg.W - cfg.C, k)
    So, zo = oracle.absorb(inp.Kev, inp.Vev)
    assert np.linalg.norm(S - So) / np.linalg.norm(So) < 2e-3
    assert np.linalg.norm(z - zo) / np.linalg.norm(zo) < 2e-3
    ref, idx_o, sc_o = oracle.hybrid_step(inp.Q, inp.K, inp.V, So, zo, cfg.bq, cfg.bk, k, want_scores=True)
    np.testing.assert_array_equal(sc, sc_o)
    np.testing.assert_array_equal(idx, idx_o)
    mx, mr = assert_close(out, ref, "832x480 layer")
    print(f"832x480: every row, max-abs {mx:.2e} mean-rel {mr:.2e}")



@pytest.mark.parametrize("keep", [1.0, 0.5, 0.25, 0.125])
def test_window21_keep_sweep(keep):
    """832x480 shapes with a 21-frame window (32760 keys, 512 key blocks), keep ratio swept
    from keep-all down to 1/8; heads 0 and 5, sampled query blocks."""
    cfg = synth.LAYER_832x480_W21
    heads = [0, 5]
    k = int(np.ceil(keep * cfg.n_kb))
    print(f"case: 21-frame window, heads {heads}, top-{k} of {cfg.n_kb}", flush=True)
    g = hf.Geometry(cfg.B, len(heads), cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    inp = layer_inputs(cfg, heads=heads)
    idx, sc, out, S, z = run_select_attn(g, inp, cfg.W - cfg.C, k, head=4)
    So, zo = oracle.absorb(inp.Kev, inp.Vev)
    blocks = sample_blocks(len(heads), cfg.n_qb, stride=17)
    ref, idx_o, sc_o = oracle.hybrid_step(inp.Q, inp.K, inp.V, So, zo, cfg.bq, cfg.bk, k, blocks=blocks,
                                          want_scores=True)
    np.testing.assert_array_equal(sc, sc_o)
    np.testing.assert_array_equal(idx, idx_o)
    if k == cfg.n_kb:
        np.testing.assert_array_equal(idx[0, 0, 0], np.arange(cfg.n_kb))
    rows = rows_of_blocks(blocks, cfg.Nq, cfg.bq, (len(heads), cfg.Nq))
    mx, mr = assert_close(out.reshape(-1, cfg.Nq, cfg.D)[rows], ref.reshape(-1, cfg.Nq, cfg.D)[rows], "W=21")
    print(f"W=21 top-{k}: {len(blocks)} blocks checked, max-abs {mx:.2e} mean-rel {mr:.2e}")


@pytest.mark.timeout(900)
def test_four_streams_per_layer_seeds():
    """Four independent streams batched (B=4) at 832x480 shapes on all 12 heads, for layers
    0, 15 and 29 of a stack (each layer seeds its own Q/K/V and state): every block's
    scores and kept list, every output row, and the absorbed state."""
    base = synth.LAYER_832x480
    cfg = synth.StepConfig("832x480_4streams", B=4, H=base.H, D=base.D, T=base.T, C=base.C, W=base.W,
                           bq=base.bq, bk=base.bk, keep=base.keep, n_evicted=base.n_evicted)
    heads = list(range(cfg.H))
    k = cfg.top_k()
    g = hf.Geometry(cfg.B, len(heads), cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    for layer in (0, 15, 29):
        print(f"case: 4 streams, layer {layer}, all heads, top-{k}", flush=True)
        d = synth.field_step_inputs(cfg, layer=layer, heads=heads)
        inp = StepInputs(d["q"], d["k_win"], d["v_win"], d["k_ev"], d["v_ev"])
        idx, sc, out, S, z = run_select_attn(g, inp, cfg.W - cfg.C, k, head=layer % cfg.W)
        So, zo = oracle.absorb(inp.Kev, inp.Vev)
        assert np.linalg.norm(S - So) / np.linalg.norm(So) < 2e-3
        ref, idx_o, sc_o = oracle.hybrid_step(inp.Q, inp.K, inp.V, So, zo, cfg.bq, cfg.bk, k, want_scores=True)
        np.testing.assert_array_equal(sc, sc_o)
        np.testing.assert_array_equal(idx, idx_o)
        mx, mr = assert_close(out, ref, f"layer {layer}")
        print(f"layer {layer}: every row, max-abs {mx:.2e} mean-rel {mr:.2e}", flush=True)

EDGE = [
    # B, H, D, T, C, W, bq, bk, n_committed, top_k
    (1, 2, 128, 200, 1, 3, 64, 64, 2, 3),     # ragged query block (200 = 3*64 + 8), ragged key block
    (2, 1, 64, 96, 2, 4, 32, 16, 2, 5),       # B=2, D=64, bq=32, bk=16
    (1, 1, 128, 104, 1, 5, 16, 128, 1, 1),    # bq=16, bk=128 (4 subtiles, last partial), top-1
    (1, 3, 64, 72, 1, 4, 64, 32, 0, 3),       # window not yet full (chunk only), keep-all
    (1, 1, 128, 64, 2, 2, 64, 64, 0, 1),      # W == C
    (1, 2, 128, 136, 1, 4, 64, 64, 3, 2),     # odd number of query blocks (last pair has one), 32-key last block
    (1, 1, 64, 48, 4, 6, 64, 64, 2, 4),       # D=64, odd number of query blocks, frames of 48 tokens
    (1, 1, 64, 512, 1, 48, 64, 16, 47, 1536), # the largest window: 1536 key blocks, all kept
    (1, 2, 128, 512, 1, 48, 64, 16, 47, 700), # 1536 key blocks, 700 kept
]


@pytest.mark.parametrize("B,H,D,T,C,W,bq,bk,ncom,top_k", EDGE)
def test_edge_shapes(B, H, D, T, C, W, bq, bk, ncom, top_k):
    print(f"case: edge B={B} H={H} D={D} T={T} C={C} W={W} bq={bq} bk={bk} n_committed={ncom} k={top_k}", flush=True)
    g = hf.Geometry(B, H, D, T, C, W, bq, bk)
    rng = np.random.default_rng(B * 1000 + T)
    nfr = ncom + C
    b = synth.bf16_bits_from_f32
    mk = lambda n: b(rng.standard_normal((B, H, n, D)).astype(np.float32))
    inp = StepInputs(mk(C * T), mk(nfr * T), mk(nfr * T), mk(2 * T + 24), mk(2 * T + 24))
    idx, sc, out, S, z = run_select_attn(g, inp, ncom, top_k, head=min(1, W - 1))
    So, zo = oracle.absorb(inp.Kev, inp.Vev)
    ref, idx_o, sc_o = oracle.hybrid_step(inp.Q, inp.K, inp.V, So, zo, bq, bk, top_k, want_scores=True)
    np.testing.assert_array_equal(sc, sc_o)
    np.testing.assert_array_equal(idx, idx_o)
    assert np.linalg.norm(S - So) / np.linalg.norm(So) < 1e-5
    assert_close(out, ref, "edge")


def test_exact_ties_take_lower_block():
    print("case: duplicated key blocks (exact score ties)", flush=True)
    B, H, D, T, C, W, bq, bk = 1, 1, 64, 64, 1, 4, 16, 16
    g = hf.Geometry(B, H, D, T, C, W, bq, bk)
    rng = np.random.default_rng(7)
    b = synth.bf16_bits_from_f32
    K = rng.standard_normal((1, 1, 4 * T, D)).astype(np.float32)
    K[0, 0, 9 * 16:10 * 16] = K[0, 0, 2 * 16:3 * 16]    # block 9 duplicates block 2
    K[0, 0, 13 * 16:14 * 16] = K[0, 0, 2 * 16:3 * 16]   # block 13 too
    Q = np.broadcast_to(K[0, 0, 2 * 16:3 * 16].mean(axis=0) * 4, (1, 1, T, D)).astype(np.float32)
    inp = StepInputs(b(Q), b(K), b(rng.standard_normal((1, 1, 4 * T, D)).astype(np.float32)))
    idx, sc, out, _, _ = run_select_attn(g, inp, 3, 2, with_state=False)
    assert sc[0, 0, 0, 2] == sc[0, 0, 0, 9] == sc[0, 0, 0, 13]
    _, idx_o, _ = oracle.hybrid_step(inp.Q, inp.K, inp.V, np.zeros((1, 1, D, D)), np.zeros((1, 1, D)), bq, bk, 2)
    np.testing.assert_array_equal(idx, idx_o)
    assert 2 in idx[0, 0, 0] and 13 not in idx[0, 0, 0]


@pytest.mark.parametrize("n_tok", [0, 1, 63, 64, 200, 1560 * 3])
def test_absorb_parity(n_tok):
    print(f"case: absorb n_tok={n_tok}", flush=True)
    g = hf.Geometry(1, 3, 128, 1560, 3, 6, 64, 64)
    rng = np.random.default_rng(n_tok)
    b = synth.bf16_bits_from_f32
    k = b(rng.standard_normal((1, 3, n_tok, 128)).astype(np.float32))
    v = b(rng.standard_normal((1, 3, n_tok, 128)).astype(np.float32))
    S0 = rng.standard_normal((1, 3, 128, 128)).astype(np.float32)
    z0 = np.abs(rng.standard_normal((1, 3, 128))).astype(np.float32)
    S = torch.from_numpy(S0).cuda()
    z = torch.from_numpy(z0).cuda()
    ws = hf.new_workspace(g)
    hf.hf_linear_absorb(g, dev_bf16(k), dev_bf16(v), n_tok, S, z, ws)
    torch.cuda.synchronize()
    So, zo = oracle.absorb(f64(k), f64(v), S0.astype(np.float64), z0.astype(np.float64))
    Sg, zg = S.cpu().numpy(), z.cpu().numpy()
    if n_tok == 0:
        np.testing.assert_array_equal(Sg, S0)
        np.testing.assert_array_equal(zg, z0)
    assert np.abs(Sg - So).max() <= 1e-4 * max(1.0, np.abs(So).max())
    assert np.abs(zg - zo).max() <= 1e-5 * max(1.0, np.abs(zo).max())


@pytest.mark.parametrize("D,bq", [(128, 64), (64, 64), (128, 32)])
@pytest.mark.parametrize("top_k", [1, 2, 3, 4, 5, 6, 7, 8, 11])
def test_fast_path_step_counts(D, bq, top_k):
    """32-key blocks, every one full, so a query block walks exactly top_k fast-path steps:
    covers the step loop's body (six steps at a time where it is unrolled by six) and
    every remainder, for the unrolled (two waves, no rotation) and the two-step (one
    wave) instances."""
    B, H, T, C, W, bk, ncom = 1, 2, 96, 1, 4, 32, 3
    print(f"case: fast path D={D} bq={bq} top_k={top_k}", flush=True)
    g = hf.Geometry(B, H, D, T, C, W, bq, bk)
    rng = np.random.default_rng(500 + 10 * top_k + D + bq)
    b = synth.bf16_bits_from_f32
    mk = lambda n: b(rng.standard_normal((B, H, n, D)).astype(np.float32))
    nfr = ncom + C
    inp = StepInputs(mk(C * T), mk(nfr * T), mk(nfr * T), mk(T), mk(T))
    idx, sc, out, S, z = run_select_attn(g, inp, ncom, top_k, head=2)
    So, zo = oracle.absorb(inp.Kev, inp.Vev)
    ref, idx_o, sc_o = oracle.hybrid_step(inp.Q, inp.K, inp.V, So, zo, bq, bk, top_k, want_scores=True)
    np.testing.assert_array_equal(idx, idx_o)
    assert_close(out, ref, f"fast path D={D} bq={bq} top_k={top_k}")
