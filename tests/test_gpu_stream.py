"""Streaming behaviour of hf_hybrid_step on the KV ring, against an fp64 oracle that keeps
its own window (a list of frames) and its own state (S, z)."""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf
import oracle
from hybrid_sparse_linear_hf_amd import synth

from gpu_helpers import assert_close, dev_bf16, f64, rows_of_blocks

pytestmark = pytest.mark.gpu


class OracleStream:
    """The method's streaming loop written plainly: a window of frames, the state, and
    eviction of the oldest frames into the state once more than W - C are committed."""

    def __init__(self, B, H, D, T, C, W, S=None, z=None):
        self.T, self.C, self.W = T, C, W
        self.frames_k, self.frames_v = [], []
        self.S = np.zeros((B, H, D, D)) if S is None else S
        self.z = np.zeros((B, H, D)) if z is None else z

    def step(self, Qc, Kc, Vc, bq, bk, top_k, blocks=None):
        """Qc, Kc, Vc: fp64 [B,H,C*T,D] of the current chunk.  Returns (out, idx)."""
        K = np.concatenate(self.frames_k + [Kc], axis=2)
        V = np.concatenate(self.frames_v + [Vc], axis=2)
        out, idx, _ = oracle.hybrid_step(Qc, K, V, self.S, self.z, bq, bk, top_k, blocks=blocks)
        T = self.T
        for c in range(self.C):
            self.frames_k.append(Kc[:, :, c * T:(c + 1) * T])
            self.frames_v.append(Vc[:, :, c * T:(c + 1) * T])
        excess = len(self.frames_k) - (self.W - self.C)
        if excess > 0:
            Kev = np.concatenate(self.frames_k[:excess], axis=2)
            Vev = np.concatenate(self.frames_v[:excess], axis=2)
            self.S, self.z = oracle.absorb(Kev, Vev, self.S, self.z)
            del self.frames_k[:excess], self.frames_v[:excess]
        return out, idx


def random_chunks(g, n_steps, seed):
    rng = np.random.default_rng(seed)
    b = synth.bf16_bits_from_f32
    shape = (g.B, g.H, g.C * g.T, g.D)
    return [tuple(b(rng.standard_normal(shape).astype(np.float32)) for _ in range(3)) for _ in range(n_steps)]


def run_gpu_stream(g, chunks, keep, head0=0):
    ring = hf.Ring(g)
    ring.set_state(head0, 0)
    ws = hf.new_workspace(g)
    S = torch.zeros((g.B, g.H, g.D, g.D), dtype=torch.float32, device="cuda")
    z = torch.zeros((g.B, g.H, g.D), dtype=torch.float32, device="cuda")
    outs, idxs = [], []
    for (q, k, v) in chunks:
        top_k = max(1, int(np.ceil(keep * g.n_kb(ring.n_committed))))
        idx = torch.empty((g.B, g.H, g.n_qb, top_k), dtype=torch.int32, device="cuda")
        out = torch.empty((g.B, g.H, g.Nq, g.D), dtype=torch.float32, device="cuda")
        hf.hf_hybrid_step(g, dev_bf16(q), dev_bf16(k), dev_bf16(v), ring, top_k, hf.HF_STEP_COMMIT, S, z, idx, out, ws)
        outs.append(out.cpu().numpy())
        idxs.append(idx.cpu().numpy())
    torch.cuda.synchronize()
    return outs, idxs, S.cpu().numpy().astype(np.float64), z.cpu().numpy().astype(np.float64), ring


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
        assert torch.equal(ring.vt[:, :, slot], V[:, :, c].transpose(-1, -2))
    assert torch.count_nonzero(ring.k[:, :, 2:]) == 0


def test_long_horizon_832x480_two_heads():
    """832x480 layer shapes (T=1560, C=3, W=6, D=128, 64x64 blocks, keep 25%) on heads 0 and 7
    streamed for 200 chunk steps; every step evicts 3 frames into the fp32 state.  Each step's
    output is checked on sampled query blocks, the final state against the fp64 recurrence."""
    print("case: 200-step stream at 832x480 shapes, heads 0 and 7", flush=True)
    cfg = synth.LAYER_832x480
    heads = [0, 7]
    g = hf.Geometry(1, len(heads), cfg.D, cfg.T, cfg.C, cfg.W, cfg.bq, cfg.bk)
    kw = dict(B=1, D=cfg.D, gh=cfg.gh, gw=cfg.gw, heads=heads)
    ev = cfg.n_evicted
    k_ev, v_ev = synth.field_frames(synth.K_ID, 0, ev, **kw), synth.field_frames(synth.V_ID, 0, ev, **kw)
    ring = hf.Ring(g)
    ws = hf.new_workspace(g)
    S = torch.zeros((1, 2, 128, 128), dtype=torch.float32, device="cuda")
    z = torch.zeros((1, 2, 128), dtype=torch.float32, device="cuda")
    hf.hf_linear_absorb(g, dev_bf16(k_ev), dev_bf16(v_ev), ev * cfg.T, S, z, ws)
    ref = OracleStream(1, 2, cfg.D, cfg.T, cfg.C, cfg.W)
    ref.S, ref.z = oracle.absorb(f64(k_ev), f64(v_ev))
    # commit frames ev .. ev+2 (the window's history) through the ring with a dry step
    first = ev + cfg.W - cfg.C
    kc, vc = synth.field_frames(synth.K_ID, ev, 3, **kw), synth.field_frames(synth.V_ID, ev, 3, **kw)
    hf.hf_ring_append(g, ring, dev_bf16(kc), dev_bf16(vc))
    ring.set_state(0, 3)
    ref.frames_k = [f64(kc)[:, :, i * cfg.T:(i + 1) * cfg.T] for i in range(3)]
    ref.frames_v = [f64(vc)[:, :, i * cfg.T:(i + 1) * cfg.T] for i in range(3)]
    top_k = cfg.top_k()
    idx = torch.empty((1, 2, cfg.n_qb, top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((1, 2, cfg.Nq, cfg.D), dtype=torch.float32, device="cuda")
    worst = (0.0, 0.0)
    for s in range(200):
        f0 = first + 3 * s
        q = synth.field_frames(synth.Q_ID, f0, 3, **kw)
        k = synth.field_frames(synth.K_ID, f0, 3, **kw)
        v = synth.field_frames(synth.V_ID, f0, 3, **kw)
        hf.hf_hybrid_step(g, dev_bf16(q), dev_bf16(k), dev_bf16(v), ring, top_k, hf.HF_STEP_COMMIT, S, z, idx, out, ws)
        blocks = [(p, (7 * s + 31 * p) % cfg.n_qb) for p in range(2)] + [(s % 2, cfg.n_qb - 1)]
        o_ref, idx_ref = ref.step(f64(q), f64(k), f64(v), cfg.bq, cfg.bk, top_k, blocks=blocks)
        o = out.cpu().numpy()
        np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref, err_msg=f"step {s}")
        rows = rows_of_blocks(blocks, cfg.Nq, cfg.bq, (2, cfg.Nq))
        mx, mr = assert_close(o.reshape(2, cfg.Nq, cfg.D)[rows], o_ref.reshape(2, cfg.Nq, cfg.D)[rows], f"step {s}")
        worst = (max(worst[0], mx), max(worst[1], mr))
        if s % 50 == 0:
            print(f"step {s}: max-abs {mx:.2e} mean-rel {mr:.2e}", flush=True)
    Sg = S.cpu().numpy().astype(np.float64)
    zg = z.cpu().numpy().astype(np.float64)
    eS = np.linalg.norm(Sg - ref.S) / np.linalg.norm(ref.S)
    ez = np.linalg.norm(zg - ref.z) / np.linalg.norm(ref.z)
    print(f"200 steps: worst max-abs {worst[0]:.2e}, worst mean-rel {worst[1]:.2e}; state rel err S {eS:.2e} z {ez:.2e}")
    assert eS < 2e-3 and ez < 2e-3
