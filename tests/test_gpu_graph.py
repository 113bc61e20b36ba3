"""The hybrid step captured in a HIP graph (torch.cuda.CUDAGraph around the C-ABI calls):
two layers' committed steps in one graph, replayed three times with eager work between the
replays (the starting state restored by plain copies), every replay checked against the
eager steps from the same state.  The kernels are deterministic, so the check is bit-exact."""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf

pytestmark = pytest.mark.gpu


class Layer:
    def __init__(self, g, seed, ws):
        gen = torch.Generator(device="cuda").manual_seed(seed)
        rnd = lambda *shape: (torch.randn(shape, generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
        self.g = g
        self.ring = hf.Ring(g)
        hist = g.W - g.C
        for f in range(0, hist, g.C):      # the history, a chunk at a time
            kc, vc = rnd(g.B, g.H, g.C * g.T, g.D), rnd(g.B, g.H, g.C * g.T, g.D)
            self.ring.set_state(0, f)
            hf.hf_ring_append(g, self.ring, kc, vc)
        self.ring.set_state(0, hist)
        self.S = torch.zeros((g.B, g.H, g.D, g.D), dtype=torch.float32, device="cuda")
        self.z = torch.zeros((g.B, g.H, g.D), dtype=torch.float32, device="cuda")
        kev, vev = rnd(g.B, g.H, 2 * g.T + 8, g.D), rnd(g.B, g.H, 2 * g.T + 8, g.D)
        hf.hf_linear_absorb(g, kev, vev, 2 * g.T + 8, self.S, self.z, ws)
        self.q, self.k, self.v = (rnd(g.B, g.H, g.C * g.T, g.D) for _ in range(3))
        self.top_k = max(1, g.n_kb(hist) // 3)
        self.idx = torch.empty((g.B, g.H, g.n_qb, self.top_k), dtype=torch.int32, device="cuda")
        self.out = torch.empty((g.B, g.H, g.Nq, g.D), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        self.saved = [t.clone() for t in (self.ring.k, self.ring.vg, self.S, self.z)]
        self.desc = (self.ring.head, self.ring.n_committed)

    def restore(self):
        for dst, src in zip((self.ring.k, self.ring.vg, self.S, self.z), self.saved):
            dst.copy_(src)
        self.out.fill_(float("nan"))
        self.idx.fill_(-1)
        self.ring.set_state(*self.desc)

    def step(self, ws):
        hf.hf_hybrid_step(self.g, self.q, self.k, self.v, self.ring, self.top_k, hf.HF_STEP_COMMIT, self.S, self.z,
                          self.idx, self.out, ws)

    def snapshot(self):
        return [t.clone() for t in (self.out, self.idx, self.S, self.z, self.ring.k, self.ring.vg)]


@pytest.mark.parametrize("geom", [hf.Geometry(B=2, H=2, D=128, T=96, C=2, W=5, bq=64, bk=32),
                                  hf.Geometry(B=1, H=3, D=64, T=64, C=1, W=4, bq=16, bk=16)])
def test_graph_replays_match_eager(geom):
    print(f"case: graph {geom}", flush=True)
    ws = hf.new_workspace(geom)
    layers = [Layer(geom, 100 + i, ws) for i in range(2)]
    for L in layers:
        L.step(ws)
    torch.cuda.synchronize()
    ref = [L.snapshot() for L in layers]
    after = [(L.ring.head, L.ring.n_committed) for L in layers]

    for L in layers:
        L.restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for L in layers:
            L.step(ws)
    # the host descriptors advanced at capture, as an eager step would have
    assert [(L.ring.head, L.ring.n_committed) for L in layers] == after
    for rep in range(3):
        for L in layers:
            L.restore()            # eager copies and fills between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for li, L in enumerate(layers):
            for name, got, want in zip(("out", "idx", "S", "z", "ring K", "ring V^T"), L.snapshot(), ref[li]):
                assert torch.equal(got, want), f"replay {rep}, layer {li}: {name} differs"
    print("graph: 3 replays bit-exact", flush=True)
