"""Streaming behaviour of hf_hybrid_step on the KV ring, against an fp64 oracle that keeps
its own window (a list of frames) and its own state (S, z)."""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf
import oracle
from hybrid_sparse_linear_hf_amd import synth

from gpu_helpers import (OracleStream, assert_close, compare, dev_bf16, f64, field_frames_par, random_chunks,
                         rows_of_blocks, run_gpu_stream)

pytestmark = pytest.mark.gpu


SMALL = hf.Geometry(B=1, H=2, D=128, T=96, C=2, W=5, bq=64, bk=32)


STREAMS = [
    # geometry, steps, keep: frames of 96 tokens (chunks cross frames), D=64 (the four-wave
    # absorb), frames shorter than a 64-token absorb chunk (several frames per chunk)
    (SMALL, 7, 0.3),
    (hf.Geometry(B=2, H=1, D=64, T=64, C=1, W=4, bq=16, bk=16), 6, 0.25),
    (hf.Geometry(B=1, H=3, D=128, T=40, C=3, W=7, bq=32, bk=16), 5, 0.4),
]


@pytest.mark.parametrize("g,n_steps,keep", STREAMS)
def test_stream_commit_matches_oracle(g, n_steps, keep):
    print(f"case: {n_steps}-step stream, B={g.B} H={g.H} D={g.D} T={g.T} C={g.C} W={g.W} bq={g.bq} bk={g.bk}, "
          "empty window at start", flush=True)
    chunks = random_chunks(g, n_steps, seed=11)
    outs, idxs, S, z, ring = run_gpu_stream(g, chunks, keep)
    ref = OracleStream(g.B, g.H, g.D, g.T, g.C, g.W)
    n_committed = 0
    for s, (q, k, v) in enumerate(chunks):
        top_k = max(1, int(np.ceil(keep * g.n_kb(n_committed))))
        o_ref, idx_ref = ref.step(f64(q), f64(k), f64(v), g.bq, g.bk, top_k)
        np.testing.assert_array_equal(idxs[s], idx_ref, err_msg=f"step {s}")
        assert_close(outs[s], o_ref, f"step {s}")
        n_committed = min(n_committed + g.C, g.W - g.C)
    assert np.linalg.norm(S - ref.S) / np.linalg.norm(ref.S) < 1e-5
    assert np.linalg.norm(z - ref.z) / np.linalg.norm(ref.z) < 1e-6
    # every step commits C frames and W - C committed frames are kept
    total = n_steps * g.C
    assert (ring.head, ring.n_committed) == ((total - (g.W - g.C)) % g.W, g.W - g.C)


def test_ring_offset_invariance_and_determinism():
    print("case: same stream at two ring offsets, and twice", flush=True)
    g = SMALL
    chunks = random_chunks(g, 5, seed=12)
    a = run_gpu_stream(g, chunks, 0.3, head0=0)
    b = run_gpu_stream(g, chunks, 0.3, head0=3)
    c = run_gpu_stream(g, chunks, 0.3, head0=0)
    for s in range(5):
        np.testing.assert_array_equal(a[0][s], b[0][s])
        np.testing.assert_array_equal(a[0][s], c[0][s])
        np.testing.assert_array_equal(a[1][s], b[1][s])
    np.testing.assert_array_equal(a[2], b[2])
    np.testing.assert_array_equal(a[2], c[2])
    np.testing.assert_array_equal(a[3], b[3])


def test_ring_append_layout():
    print("case: ring append layout", flush=True)
    g = hf.Geometry(B=2, H=3, D=64, T=136, C=2, W=4, bq=64, bk=64)
    ring = hf.Ring(g)
    ring.set_state(3, 1)   # current chunk -> logical frames 1, 2 -> slots 0, 1
    q, k, v = random_chunks(g, 1, seed=13)[0]
    hf.hf_ring_append(g, ring, dev_bf16(k), dev_bf16(v))
    torch.cuda.synchronize()
    K = dev_bf16(k).view(g.B, g.H, g.C, g.T, g.D)
    V = dev_bf16(v).view(g.B, g.H, g.C, g.T, g.D)
    for c, slot in enumerate((0, 1)):
        assert torch.equal(ring.k[:, :, slot], K[:, :, c])
        # value feature f of token 8 gi + j at [gi][f][j]
        Vc = V[:, :, c]
        assert torch.equal(ring.vg[:, :, slot], torch.stack([Vc[:, :, 8 * gi:8 * gi + 8].transpose(-1, -2)
                                                             for gi in range(g.T // 8)], dim=2))
    assert torch.count_nonzero(ring.k[:, :, 2:]) == 0


@pytest.mark.parametrize("g,head,ncom", [
    # frames of 200 tokens (a ragged 8-token tail of 64-token tiles), the chunk wrapping round
    # the ring; D = 64; a 1560-token frame at the layer shapes
    (hf.Geometry(B=1, H=2, D=128, T=200, C=2, W=5, bq=64, bk=64), 4, 3),
    (hf.Geometry(B=2, H=1, D=64, T=136, C=1, W=4, bq=32, bk=32), 1, 2),
    (hf.Geometry(B=1, H=2, D=128, T=1560, C=3, W=6, bq=64, bk=64), 5, 3),
])
def test_step_appends_chunk_to_ring(g, head, ncom):
    """A committed hf_hybrid_step leaves the chunk in its ring slots bit for bit (keys as
    rows, values in 8-token groups; written by extra workgroups of the selection's score
    launch, while its pool launch reads the chunk's keys from the input); the other slots
    keep their contents."""
    print(f"case: step append, D={g.D} T={g.T} C={g.C} W={g.W} head={head} ncom={ncom}", flush=True)
    rng = np.random.default_rng(14)
    ring = hf.Ring(g)
    before_k = torch.from_numpy(rng.integers(0, 1 << 14, ring.k.shape, dtype=np.int16)).cuda().view(torch.bfloat16)
    before_v = torch.from_numpy(rng.integers(0, 1 << 14, ring.vg.shape, dtype=np.int16)).cuda().view(torch.bfloat16)
    ring.k.copy_(before_k)
    ring.vg.copy_(before_v)
    ring.set_state(head, ncom)
    q, k, v = random_chunks(g, 1, seed=15)[0]
    top_k = max(1, g.n_kb(ncom) // 4)
    idx = torch.empty((g.B, g.H, g.n_qb, top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((g.B, g.H, g.Nq, g.D), dtype=torch.float32, device="cuda")
    S = torch.zeros((g.B, g.H, g.D, g.D), dtype=torch.float32, device="cuda")
    z = torch.zeros((g.B, g.H, g.D), dtype=torch.float32, device="cuda")
    hf.hf_hybrid_step(g, dev_bf16(q), dev_bf16(k), dev_bf16(v), ring, top_k, hf.HF_STEP_COMMIT, S, z, idx, out,
                      hf.new_workspace(g))
    torch.cuda.synchronize()
    K = dev_bf16(k).view(g.B, g.H, g.C, g.T, g.D)
    V = dev_bf16(v).view(g.B, g.H, g.C, g.T, g.D)
    slots = [(head + ncom + c) % g.W for c in range(g.C)]
    for c, slot in enumerate(slots):
        assert torch.equal(ring.k[:, :, slot], K[:, :, c]), f"keys of chunk frame {c}"
        Vc = V[:, :, c]
        want = torch.stack([Vc[:, :, 8 * gi:8 * gi + 8].transpose(-1, -2) for gi in range(g.T // 8)], dim=2)
        assert torch.equal(ring.vg[:, :, slot], want), f"values of chunk frame {c}"
    for slot in set(range(g.W)) - set(slots):
        assert torch.equal(ring.k[:, :, slot], before_k[:, :, slot])
        assert torch.equal(ring.vg[:, :, slot], before_v[:, :, slot])


@pytest.mark.timeout(900)
def test_long_horizon_832x480_all_heads():
    """The long-horizon stream at the 832x480 layer shapes (12 heads x 128, T=1560, C=3, W=6,
    64x64 blocks, keep 25%): 200 committed hf_hybrid_step calls, each evicting 3 frames
    (4680 tokens per head) into the fp32 state through the ring absorb.  Every step: indices
    on every query block, the output on two sampled query blocks per head plus the ragged
    last one; steps 0, 100 and 199: the output on every row.  At the end: the state (S
    12x128x128, z 12x128) against the fp64 recurrence, and the readout alone (output with
    the state minus output without it) against the oracle's readout from its state."""
    print("case: 200-step stream at 832x480 shapes, all 12 heads", flush=True)
    cfg = synth.LAYER_832x480
    heads = list(range(cfg.H))
    H, T, D, Nq = cfg.H, cfg.T, cfg.D, cfg.Nq
    g = hf.Geometry(1, H, D, T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    frames = lambda tid, f0, n: field_frames_par(tid, f0, n, heads)
    ev = cfg.n_evicted
    k_ev, v_ev = frames(synth.K_ID, 0, ev), frames(synth.V_ID, 0, ev)
    ring = hf.Ring(g)
    ws = hf.new_workspace(g)
    S = torch.zeros((1, H, D, D), dtype=torch.float32, device="cuda")
    z = torch.zeros((1, H, D), dtype=torch.float32, device="cuda")
    hf.hf_linear_absorb(g, dev_bf16(k_ev), dev_bf16(v_ev), ev * T, S, z, ws)
    ref = OracleStream(1, H, D, T, cfg.C, cfg.W)
    ref.S, ref.z = oracle.absorb(f64(k_ev), f64(v_ev))
    # the window's history: frames ev .. ev+2 committed through the ring
    first = ev + cfg.W - cfg.C
    kc, vc = frames(synth.K_ID, ev, 3), frames(synth.V_ID, ev, 3)
    hf.hf_ring_append(g, ring, dev_bf16(kc), dev_bf16(vc))
    ring.set_state(0, 3)
    ref.frames_k = [f64(kc)[:, :, i * T:(i + 1) * T] for i in range(3)]
    ref.frames_v = [f64(vc)[:, :, i * T:(i + 1) * T] for i in range(3)]
    top_k = cfg.top_k()
    idx = torch.empty((1, H, cfg.n_qb, top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((1, H, Nq, D), dtype=torch.float32, device="cuda")
    worst = (0.0, 0.0)
    full_steps = (0, 100, 199)
    nxt = [frames(t, first, 3) for t in (synth.Q_ID, synth.K_ID, synth.V_ID)]
    for s in range(200):
        q, k, v = nxt
        hf.hf_hybrid_step(g, dev_bf16(q), dev_bf16(k), dev_bf16(v), ring, top_k, hf.HF_STEP_COMMIT, S, z, idx, out, ws)
        if s + 1 < 200:   # draw the next chunk while the GPU works
            nxt = [frames(t, first + 3 * (s + 1), 3) for t in (synth.Q_ID, synth.K_ID, synth.V_ID)]
        if s in full_steps:
            blocks = None
        else:
            blocks = sorted({(p, (7 * s + 31 * p + j * 37) % cfg.n_qb) for p in range(H) for j in range(2)}
                            | {(p, cfg.n_qb - 1) for p in range(H)})
        o_ref, idx_ref = ref.step(f64(q), f64(k), f64(v), cfg.bq, cfg.bk, top_k, blocks=blocks)
        o = out.cpu().numpy()
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref, err_msg=f"step {s}")
        if blocks is None:
            mx, mr = assert_close(o, o_ref, f"step {s}, every row")
        else:
            rows = rows_of_blocks(blocks, Nq, cfg.bq, (H, Nq))
            mx, mr = assert_close(o.reshape(H, Nq, D)[rows], o_ref.reshape(H, Nq, D)[rows], f"step {s}")
        worst = (max(worst[0], mx), max(worst[1], mr))
        if s % 25 == 0 or blocks is None:
            print(f"step {s}: max-abs {mx:.2e} mean-rel {mr:.2e}" + (" (every row)" if blocks is None else ""),
                  flush=True)
    torch.cuda.synchronize()
    Sg = S.cpu().numpy().astype(np.float64)
    zg = z.cpu().numpy().astype(np.float64)
    eS = np.linalg.norm(Sg - ref.S) / np.linalg.norm(ref.S)
    ez = np.linalg.norm(zg - ref.z) / np.linalg.norm(ref.z)
    # the readout alone from the state after 200 steps (618 absorbed frames), on the last
    # chunk's queries: attention with the state minus attention without it, on the same ring
    # and kept lists (the sparse parts are bit-identical, so the difference is the readout)
    out_sp = torch.empty_like(out)
    qd = dev_bf16(q)
    hf.hf_sparse_window_attn(g, qd, ring, idx, top_k, S, z, out, ws)
    hf.hf_sparse_window_attn(g, qd, ring, idx, top_k, None, None, out_sp, ws)
    r = out.cpu().numpy().astype(np.float64) - out_sp.cpu().numpy()
    lin = oracle.linear_readout(f64(q), ref.S, ref.z, cfg.bq)
    rmx, rmr = compare(r, lin)
    print(f"200 steps: worst max-abs {worst[0]:.2e}, worst mean-rel {worst[1]:.2e}; state rel err S {eS:.2e} "
          f"z {ez:.2e}; readout alone after 618 absorbed frames: max-abs {rmx:.2e} rel {rmr:.2e}")
    assert eS < 2e-3 and ez < 2e-3
    assert rmr < 2e-3
