"""The benched call itself, hf_hybrid_step with commit, against the fp64 oracle at full
size; the ring absorb in its steady state (several 64-token chunks per split); the
attention's recomputation with the online softmax when a later kept block's logits far
exceed the first subtile's; and a stream on the chunk-aware keep schedule.

Bar: block indices bit-exact; outputs max-abs 1e-2 and mean-relative 2e-3 against the
oracle; the state after a commit within a relative Frobenius error of 1e-5 (hi/lo split of
phi(K), fp32 accumulation)."""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf
import oracle
from hybrid_sparse_linear_hf_amd import synth

from gpu_helpers import (OracleStream, assert_close, compare, dev_bf16, f64, field_frames_par, fill_ring,
                         random_chunks, rows_of_blocks, run_gpu_stream)

pytestmark = pytest.mark.gpu


def rel_fro(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_step_commit_832x480_all_heads():
    """The 832x480 layer with all 12 heads (T=1560, C=3, W=6, D=128, 64x64 blocks, 37 of 147
    kept): the state absorbs frames 0..17, the ring holds frames 18..20, and one committed
    hf_hybrid_step takes frames 21..23 -- the same call the benchmark times.  Indices on every
    query block, the output on every row, the readout alone, and the state after the commit
    (frames 18..20 absorbed by the ring absorb) against the oracle."""
    print("case: hf_hybrid_step + commit, 832x480 layer, all 12 heads, every row", flush=True)
    cfg = synth.LAYER_832x480
    g = hf.Geometry(cfg.B, cfg.H, cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    heads = list(range(cfg.H))
    T, ev, top_k = cfg.T, cfg.n_evicted, cfg.top_k()
    frames = lambda tid, f0, n: field_frames_par(tid, f0, n, heads)
    k_ev, v_ev = frames(synth.K_ID, 0, ev), frames(synth.V_ID, 0, ev)
    k_hist, v_hist = frames(synth.K_ID, ev, 3), frames(synth.V_ID, ev, 3)
    q, k, v = frames(synth.Q_ID, ev + 3, 3), frames(synth.K_ID, ev + 3, 3), frames(synth.V_ID, ev + 3, 3)

    ring = hf.Ring(g)
    ws = hf.new_workspace(g)
    S = torch.zeros((1, cfg.H, cfg.D, cfg.D), dtype=torch.float32, device="cuda")
    z = torch.zeros((1, cfg.H, cfg.D), dtype=torch.float32, device="cuda")
    hf.hf_linear_absorb(g, dev_bf16(k_ev), dev_bf16(v_ev), ev * T, S, z, ws)
    hf.hf_ring_append(g, ring, dev_bf16(k_hist), dev_bf16(v_hist))
    ring.set_state(0, cfg.W - cfg.C)
    idx = torch.empty((1, cfg.H, cfg.n_qb, top_k), dtype=torch.int32, device="cuda")
    out_sp = torch.empty((1, cfg.H, cfg.Nq, cfg.D), dtype=torch.float32, device="cuda")
    out = torch.empty_like(out_sp)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    # the sparse part alone (no state, no commit), then the benched call
    hf.hf_hybrid_step(g, qd, kd, vd, ring, top_k, 0, None, None, idx, out_sp, ws)
    assert (ring.head, ring.n_committed) == (0, cfg.W - cfg.C)
    hf.hf_hybrid_step(g, qd, kd, vd, ring, top_k, hf.HF_STEP_COMMIT, S, z, idx, out, ws)
    torch.cuda.synchronize()
    assert (ring.head, ring.n_committed) == (cfg.C, cfg.W - cfg.C)

    So, zo = oracle.absorb(f64(k_ev), f64(v_ev))
    Q = f64(q)
    K = np.concatenate([f64(k_hist), f64(k)], axis=2)
    V = np.concatenate([f64(v_hist), f64(v)], axis=2)
    ref, idx_o, _ = oracle.hybrid_step(Q, K, V, So, zo, cfg.bq, cfg.bk, top_k)
    lin = oracle.linear_readout(Q, So, zo, cfg.bq)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    o, osp = out.cpu().numpy(), out_sp.cpu().numpy()
    mx, mr = assert_close(o, ref, "step output, every row")
    mxs, mrs = assert_close(osp, ref - lin, "sparse part, every row")
    # the readout alone: its own error, and its share of the output's error budget
    r = o.astype(np.float64) - osp
    rmx, rmr = compare(r, lin)
    share = float(np.abs(r - lin).sum() / np.abs(ref).sum())
    print(f"832x480 step: out max-abs {mx:.2e} mean-rel {mr:.2e}; sparse part {mxs:.2e} / {mrs:.2e}; "
          f"readout alone max-abs {rmx:.2e} rel {rmr:.2e}, share of output {share:.2e}")
    assert share <= 1e-3, f"readout error uses {share:.2e} of the 2e-3 mean-relative budget"
    # the commit evicted frames 18..20 (the oldest window frames) into the state
    So2, zo2 = oracle.absorb(f64(k_hist), f64(v_hist), So, zo)
    eS = rel_fro(S.cpu().numpy().astype(np.float64), So2)
    ez = rel_fro(z.cpu().numpy().astype(np.float64), zo2)
    print(f"state after commit: rel err S {eS:.2e} z {ez:.2e}")
    assert eS < 1e-5 and ez < 1e-5


RING_ABSORB = [
    # B, H, D, T, C, W, bq, bk, top_k: evictions of thousands of tokens per plane over many
    # planes, so every absorb split walks several 64-token chunks (the LDS ring wraps)
    (1, 16, 128, 1560, 3, 6, 64, 64, 37),   # 4680 tokens per plane, chunks straddle frames
    (2, 16, 64, 96, 32, 64, 64, 64, 4),     # D=64, 3072 tokens per plane
    (1, 32, 64, 40, 80, 160, 64, 64, 3),    # frames shorter than a chunk, 3200 tokens per plane
    (1, 2, 128, 1024, 8, 16, 64, 64, 8),    # 8192 tokens per plane: the most splits
    (1, 3, 128, 1560, 3, 6, 32, 64, 37),    # one-wave attention workgroups (bq = 32)
]


@pytest.mark.parametrize("B,H,D,T,C,W,bq,bk,top_k", RING_ABSORB)
def test_ring_absorb_steady_state(B, H, D, T, C, W, bq, bk, top_k):
    """Two committed steps on a full window (the second at another ring offset): each evicts
    C frames through the ring absorb.  Indices, outputs (sampled blocks) and the state after
    each step against the oracle's window and recurrence."""
    print(f"case: ring absorb B={B} H={H} D={D} T={T} C={C} W={W}, {C * T} tokens evicted per plane per step",
          flush=True)
    g = hf.Geometry(B, H, D, T, C, W, bq, bk)
    rng = np.random.default_rng(D * 7 + T)
    b = synth.bf16_bits_from_f32
    mk = lambda n: b(rng.standard_normal((B, H, n, D)).astype(np.float32))
    nhist = W - C
    k_hist, v_hist = mk(nhist * T), mk(nhist * T)
    S0 = rng.standard_normal((B, H, D, D)).astype(np.float32)
    z0 = np.abs(rng.standard_normal((B, H, D))).astype(np.float32) * 100
    ring = hf.Ring(g)
    fill_ring(ring, k_hist, v_hist, nhist, head=5 % W)
    ring.set_state(5 % W, nhist)
    ws = hf.new_workspace(g)
    S, z = torch.from_numpy(S0).cuda(), torch.from_numpy(z0).cuda()
    ref = OracleStream(B, H, D, T, C, W, S0.astype(np.float64), z0.astype(np.float64))
    ref.frames_k = [f64(k_hist)[:, :, f * T:(f + 1) * T] for f in range(nhist)]
    ref.frames_v = [f64(v_hist)[:, :, f * T:(f + 1) * T] for f in range(nhist)]
    nqb = -(-C * T // bq)
    for step in range(2):
        q, k, v = mk(C * T), mk(C * T), mk(C * T)
        idx = torch.empty((B, H, nqb, top_k), dtype=torch.int32, device="cuda")
        out = torch.empty((B, H, C * T, D), dtype=torch.float32, device="cuda")
        hf.hf_hybrid_step(g, dev_bf16(q), dev_bf16(k), dev_bf16(v), ring, top_k, hf.HF_STEP_COMMIT, S, z, idx, out,
                          ws)
        torch.cuda.synchronize()
        blocks = sorted({(p, i) for p in range(B * H) for i in ((3 * p + step) % nqb, nqb - 1)})
        o_ref, idx_ref = ref.step(f64(q), f64(k), f64(v), bq, bk, top_k, blocks=blocks)
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref, err_msg=f"step {step}")
        rows = rows_of_blocks(blocks, C * T, bq, (B * H, C * T))
        mx, mr = assert_close(out.cpu().numpy().reshape(B * H, C * T, D)[rows],
                              o_ref.reshape(B * H, C * T, D)[rows], f"step {step}")
        eS = rel_fro(S.cpu().numpy().astype(np.float64), ref.S)
        ez = rel_fro(z.cpu().numpy().astype(np.float64), ref.z)
        print(f"step {step}: out max-abs {mx:.2e} mean-rel {mr:.2e}; state rel err S {eS:.2e} z {ez:.2e}", flush=True)
        assert eS < 1e-5 and ez < 1e-5
    assert (ring.head, ring.n_committed) == ((5 + 2 * C) % W, nhist)


FALLBACK = [(64, 32), (64, 64), (128, 32), (128, 64)]


@pytest.mark.parametrize("D,bq", FALLBACK)
@pytest.mark.parametrize("dt", [0, 16])
def test_attention_online_fallback_on_large_logits(D, bq, dt):
    """Kept key blocks whose logits exceed the first subtile's maximum by about 30 (natural
    units) for some queries of every query block: in the 16-key tail of the last key block for
    query block 0, in a full subtile of a middle key block of its own for every other one.  The attention's
    fixed per-row reference then overflows its bound and the block is recomputed with the
    online softmax; the result must still match the oracle.  dt = 16: the same through the
    instances with the relative temporal rotation (16 rotated features, offset cap 1)."""
    T, C, W, ncom, bk = 208, 1, 3, 2, 64        # window 624 keys: 9 full key blocks + 48 (32 + a 16-key tail)
    g = hf.Geometry(1, 2, D, T, C, W, bq, bk)
    Nq, Nk = C * T, (ncom + C) * T
    nqb, nkb = -(-Nq // bq), -(-Nk // bk)
    rng = np.random.default_rng(D + bq)
    Q = rng.standard_normal((1, 2, Nq, D)).astype(np.float32)
    K = rng.standard_normal((1, 2, Nk, D)).astype(np.float32)
    # values at half scale: the probabilities are bf16 matrix-core operands, so a weight near 1
    # errs by up to 2^-9 of the value it multiplies, and the unplanted queries of block 0 meet
    # the planted keys with logits spread by alpha
    V = 0.5 * rng.standard_normal((1, 2, Nk, D)).astype(np.float32)
    alpha = (30.0 if dt == 0 else 40.0) / np.sqrt(D)   # planted key = alpha * query -> logit ~ 30 (40)
    idx = np.zeros((1, 2, nqb, 3), dtype=np.int32)
    for i in range(nqb):
        q0, q1 = i * bq, min((i + 1) * bq, Nq)
        if i == 0:     # the 16-key tail subtile of the last key block (keys 608 .. 623)
            rows = (nkb - 1) * bk + 32 + np.arange(min(16, q1 - q0))
            idx[:, :, i] = [0, 5, nkb - 1]
        else:          # a full subtile of key block i (1 .. nqb-1 <= 6), its own
            rows = i * bk + np.arange(q1 - q0)
            idx[:, :, i] = [0, i, nkb - 1]
        K[:, :, rows] = alpha * Q[:, :, q0:q0 + len(rows)]
    b = synth.bf16_bits_from_f32
    qb, kb, vb = b(Q), b(K), b(V)
    Qd, Kd, Vd = f64(qb), f64(kb), f64(vb)
    # the inputs do what the test is about: for every query block, some query's best kept key
    # lies >= 32 base-2 units above its best key of the first 32-key subtile (with the
    # rotation: bounds from the unrotated features, the rotated pairs' part bounded by the
    # product of their norms, which a rotation keeps)
    c = np.log2(np.e) / np.sqrt(D)
    for p in range(2):
        for i in range(nqb):
            q0, q1 = i * bq, min((i + 1) * bq, Nq)
            keys = np.concatenate([np.arange(j * bk, min((j + 1) * bk, Nk)) for j in idx[0, p, i]])
            Qi, Kj = Qd[0, p, q0:q1], Kd[0, p, keys]
            sp = Qi[:, dt:] @ Kj[:, dt:].T * c
            tb = np.linalg.norm(Qi[:, :dt], axis=1)[:, None] * np.linalg.norm(Kj[:, :dt], axis=1)[None, :] * c
            lo, hi = sp - tb, sp + tb
            assert (lo.max(axis=1) - hi[:, :32].max(axis=1)).max() >= 34.0
    kev, vev = b(rng.standard_normal((1, 2, 300, D)).astype(np.float32)), b(rng.standard_normal((1, 2, 300, D)).astype(np.float32))
    ring = hf.Ring(g)
    fill_ring(ring, kb, vb, ncom + C, head=1)
    ring.set_state(1, ncom)
    ws = hf.new_workspace(g)
    S = torch.zeros((1, 2, D, D), dtype=torch.float32, device="cuda")
    z = torch.zeros((1, 2, D), dtype=torch.float32, device="cuda")
    hf.hf_linear_absorb(g, dev_bf16(kev), dev_bf16(vev), 300, S, z, ws)
    out = torch.empty((1, 2, Nq, D), dtype=torch.float32, device="cuda")
    idx_d = torch.from_numpy(idx).cuda()
    So, zo = oracle.absorb(f64(kev), f64(vev))
    if dt == 0:
        hf.hf_sparse_window_attn(g, dev_bf16(qb), ring, idx_d, 3, S, z, out, ws)
        ref = oracle.sparse_attn(Qd, Kd, Vd, idx, bq, bk)
    else:
        hf.hf_sparse_window_attn_rope(g, dev_bf16(qb), ring, idx_d, 3, S, z, out, ws, hf.Rope(dt, 1, 10000.0))
        ref = oracle.sparse_attn_rope(Qd, Kd, Vd, idx, bq, bk, T, dt, 1, 10000.0)
    torch.cuda.synchronize()
    ref = ref + oracle.linear_readout(Qd, So, zo, bq)
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    mx, mr = assert_close(o, ref, f"large logits D={D} bq={bq} dt={dt}")
    print(f"large logits D={D} bq={bq} dt={dt}: max-abs {mx:.2e} mean-rel {mr:.2e}")


def test_stream_on_chunk_aware_schedule():
    """hf_hybrid_step from an empty window with the per-chunk keep counts of hf_cag_schedule
    (Light Forcing, chunk-aware growth: the first chunk dense, later ones sparser); the keep
    counts equal the oracle schedule's, and every step matches the oracle stream."""
    g = hf.Geometry(B=1, H=3, D=128, T=96, C=2, W=8, bq=64, bk=32)
    n_steps = 8
    nkb = [g.n_kb(min(s * g.C, g.W - g.C)) for s in range(n_steps)]
    ks, _, beta = hf.hf_cag_schedule(nkb, 0.9, 0.6, 0.95)
    ks_o, _, beta_o = oracle.cag_schedule(nkb, 0.9, 0.6, 0.95)
    assert ks == ks_o and ks[0] == nkb[0] and abs(beta - beta_o) <= 1e-12 * max(1.0, beta_o)
    print(f"case: chunk-aware stream, n_kb {nkb}, keep {ks}", flush=True)
    chunks = random_chunks(g, n_steps, seed=21)
    outs, idxs, S, z, ring = run_gpu_stream(g, chunks, ks)
    ref = OracleStream(g.B, g.H, g.D, g.T, g.C, g.W)
    for s, (q, k, v) in enumerate(chunks):
        o_ref, idx_ref = ref.step(f64(q), f64(k), f64(v), g.bq, g.bk, ks[s])
        np.testing.assert_array_equal(idxs[s], idx_ref, err_msg=f"step {s}")
        assert_close(outs[s], o_ref, f"step {s}")
    assert rel_fro(S, ref.S) < 1e-5 and rel_fro(z, ref.z) < 1e-5
