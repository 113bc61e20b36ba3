"""GPU parity of the hierarchical coarse-to-fine block selection ([LF-de] §2.2),
hf_block_select_hier, against the fp64 oracle: frame and block scores bit-exact, kept
frames and blocks bit-exact, and the attention output over the selected blocks within
max-abs 1e-2 and mean-relative 2e-3."""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf
import oracle
from hybrid_sparse_linear_hf_amd import synth

from gpu_helpers import StepInputs, assert_close, dev_bf16, fill_ring, rows_of_blocks

pytestmark = pytest.mark.gpu


def run_hier(g, inp, n_committed, top_frames, top_k, head=0):
    ring = hf.Ring(g)
    nfr = n_committed + g.C
    fill_ring(ring, inp.k_bits, inp.v_bits, nfr, head)
    ring.set_state(head, n_committed)
    ws = hf.new_workspace(g)
    q = dev_bf16(inp.q_bits)
    nkb = g.n_kb(n_committed)
    dev = "cuda"
    idx = torch.empty((g.B, g.H, g.n_qb, top_k), dtype=torch.int32, device=dev)
    frames = torch.empty((g.B, g.H, g.n_qb, top_frames), dtype=torch.int32, device=dev)
    scores = torch.empty((g.B, g.H, g.n_qb, nkb), dtype=torch.float64, device=dev)
    fscores = torch.empty((g.B, g.H, g.n_qb, nfr), dtype=torch.float64, device=dev)
    hf.hf_block_select_hier(g, q, ring, top_frames, top_k, idx, ws, frames=frames, scores=scores, frame_scores=fscores)
    S = torch.zeros((g.B, g.H, g.D, g.D), dtype=torch.float32, device=dev)
    z = torch.zeros((g.B, g.H, g.D), dtype=torch.float32, device=dev)
    if inp.kev_bits is not None:
        hf.hf_linear_absorb(g, dev_bf16(inp.kev_bits), dev_bf16(inp.vev_bits), inp.kev_bits.shape[2], S, z, ws)
    out = torch.empty((g.B, g.H, g.Nq, g.D), dtype=torch.float32, device=dev)
    hf.hf_sparse_window_attn(g, q, ring, idx, top_k, S, z, out, ws)
    # the flat selection on the same ring, for the all-frames case
    idx_flat = torch.empty_like(idx)
    hf.hf_block_select(g, q, ring, top_k, idx_flat, None, ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in dict(idx=idx, frames=frames, scores=scores, fscores=fscores, out=out,
                                                 idx_flat=idx_flat).items()}


def check(g, inp, res, top_frames, top_k, blocks=None):
    idx_o, fr_o, sc_o, sf_o = oracle.hier_select(inp.Q, inp.K, g.bq, g.bk, g.T, top_frames, top_k)
    np.testing.assert_array_equal(res["fscores"], sf_o)
    np.testing.assert_array_equal(res["scores"], sc_o)
    np.testing.assert_array_equal(res["frames"], fr_o)
    np.testing.assert_array_equal(res["idx"], idx_o)
    So, zo = oracle.absorb(inp.Kev, inp.Vev) if inp.Kev is not None else (
        np.zeros((g.B, g.H, g.D, g.D)), np.zeros((g.B, g.H, g.D)))
    ref = oracle.sparse_attn(inp.Q, inp.K, inp.V, idx_o, g.bq, g.bk, blocks=blocks) + \
        oracle.linear_readout(inp.Q, So, zo, g.bq, blocks=blocks)
    out = res["out"]
    if blocks is not None:
        rows = rows_of_blocks(blocks, g.Nq, g.bq, (g.B * g.H, g.Nq))
        out = out.reshape(-1, g.Nq, g.D)[rows]
        ref = ref.reshape(-1, g.Nq, g.D)[rows]
    return assert_close(out, ref, "hierarchical")


def random_inputs(g, nfr, seed):
    rng = np.random.default_rng(seed)
    b = synth.bf16_bits_from_f32
    mk = lambda n: b(rng.standard_normal((g.B, g.H, n, g.D)).astype(np.float32))
    return StepInputs(mk(g.C * g.T), mk(nfr * g.T), mk(nfr * g.T), mk(2 * g.T), mk(2 * g.T))


HIER_EDGE = [
    # B, H, D, T, C, W, bq, bk, n_committed, top_frames, top_k
    (1, 2, 64, 64, 1, 6, 16, 16, 5, 2, 5),       # blocks inside frames
    (2, 1, 128, 40, 2, 7, 32, 16, 5, 3, 6),      # blocks straddling frames (40 = 2.5 blocks)
    (1, 1, 128, 64, 1, 5, 64, 64, 4, 1, 1),      # blocks as long as a frame, top-1
    (1, 3, 64, 72, 2, 4, 64, 32, 1, 3, 4),       # window not yet full
]


@pytest.mark.parametrize("B,H,D,T,C,W,bq,bk,ncom,top_frames,top_k", HIER_EDGE)
def test_hier_edge_shapes(B, H, D, T, C, W, bq, bk, ncom, top_frames, top_k):
    print(f"case: hier B={B} H={H} D={D} T={T} C={C} W={W} bq={bq} bk={bk} n_committed={ncom} "
          f"frames={top_frames} k={top_k}", flush=True)
    g = hf.Geometry(B, H, D, T, C, W, bq, bk)
    inp = random_inputs(g, ncom + C, seed=T * 10 + W)
    res = run_hier(g, inp, ncom, top_frames, top_k, head=min(2, W - 1))
    check(g, inp, res, top_frames, top_k)


def test_hier_all_frames_equals_flat():
    print("case: hier with every frame kept equals the flat selection", flush=True)
    g = hf.Geometry(1, 2, 128, 96, 2, 5, 64, 32, )
    inp = random_inputs(g, 5, seed=3)
    res = run_hier(g, inp, 3, 5, 7)
    np.testing.assert_array_equal(res["idx"], res["idx_flat"])
    check(g, inp, res, 5, 7)


@pytest.mark.parametrize("top_frames,top_k", [(6, 128), (3, 64)])
def test_hier_window21(top_frames, top_k):
    """832x480 shapes with a 21-frame window (512 key blocks): each query block keeps
    top_frames frames, then top_k blocks inside them; heads 0 and 5, sampled query blocks
    for the output."""
    cfg = synth.LAYER_832x480_W21
    heads = [0, 5]
    print(f"case: hier 21-frame window, heads {heads}, frames {top_frames}, top-{top_k}", flush=True)
    g = hf.Geometry(cfg.B, len(heads), cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    d = synth.field_step_inputs(cfg, heads=heads)
    inp = StepInputs(d["q"], d["k_win"], d["v_win"], d["k_ev"], d["v_ev"])
    res = run_hier(g, inp, cfg.W - cfg.C, top_frames, top_k, head=7)
    from test_gpu_parity import sample_blocks
    blocks = sample_blocks(len(heads), cfg.n_qb, stride=17)
    mx, mr = check(g, inp, res, top_frames, top_k, blocks=blocks)
    print(f"hier W=21 frames {top_frames} top-{top_k}: max-abs {mx:.2e} mean-rel {mr:.2e}")
