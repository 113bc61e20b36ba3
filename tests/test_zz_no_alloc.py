"""hf_hybrid_step_noalloc -- the step for callers that cannot allocate, whose transient data
live in the library's fixed per-GPU scratch array -- against hf_hybrid_step with a caller
workspace, through the C ABI: two calls in a row, the second with a smaller input (the
array then holds the first call's data).  Indices, outputs, state and ring descriptor must
be identical (the same kernels run), which also meets the parity bar."""

import numpy as np
import pytest
import torch

import hybrid_sparse_linear_hf_amd as hf
from hybrid_sparse_linear_hf_amd import synth

from gpu_helpers import assert_close, dev_bf16, fill_ring

pytestmark = pytest.mark.gpu

BIG = hf.Geometry(B=1, H=12, D=128, T=1560, C=3, W=6, bq=64, bk=64)   # the 832x480 layer
SMALL = hf.Geometry(B=1, H=2, D=64, T=96, C=2, W=5, bq=32, bk=32)


def make_case(g, seed):
    rng = np.random.default_rng(seed)
    b = synth.bf16_bits_from_f32
    mk = lambda n: b((0.5 * rng.standard_normal((g.B, g.H, n, g.D))).astype(np.float32))
    nhist = g.W - g.C
    return dict(k_hist=mk(nhist * g.T), v_hist=mk(nhist * g.T), q=mk(g.Nq), k=mk(g.Nq), v=mk(g.Nq),
                S=rng.standard_normal((g.B, g.H, g.D, g.D)).astype(np.float32),
                z=(np.abs(rng.standard_normal((g.B, g.H, g.D))) * 50).astype(np.float32),
                top_k=max(1, g.n_kb(nhist) // 4))


def setup(g, c):
    ring = hf.Ring(g)
    fill_ring(ring, c["k_hist"], c["v_hist"], g.W - g.C, head=2)
    ring.set_state(2, g.W - g.C)
    S, z = torch.from_numpy(c["S"]).cuda(), torch.from_numpy(c["z"]).cuda()
    idx = torch.full((g.B, g.H, g.n_qb, c["top_k"]), -1, dtype=torch.int32, device="cuda")
    out = torch.full((g.B, g.H, g.Nq, g.D), float("nan"), dtype=torch.float32, device="cuda")
    return ring, S, z, idx, out


def test_noalloc_step_matches_workspace_step():
    cases = [(BIG, make_case(BIG, 1)), (SMALL, make_case(SMALL, 2))]
    ref = []
    for g, c in cases:
        print(f"case: workspace step B={g.B} H={g.H} D={g.D} T={g.T} C={g.C} W={g.W}", flush=True)
        ring, S, z, idx, out = setup(g, c)
        ws = hf.new_workspace(g)
        hf.hf_hybrid_step(g, dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"]), ring, c["top_k"],
                          hf.HF_STEP_COMMIT, S, z, idx, out, ws)
        torch.cuda.synchronize()
        ref.append((idx.cpu(), out.cpu(), S.cpu(), z.cpu(), (ring.head, ring.n_committed)))
        del ws
    # two allocation-free calls in a row: the 832x480 layer, then the smaller input
    for (g, c), (idx_r, out_r, S_r, z_r, desc_r) in zip(cases, ref):
        print(f"case: allocation-free step B={g.B} H={g.H} D={g.D} T={g.T} C={g.C} W={g.W}", flush=True)
        ring, S, z, idx, out = setup(g, c)
        q, k, v = dev_bf16(c["q"]), dev_bf16(c["k"]), dev_bf16(c["v"])
        torch.cuda.synchronize()
        hf.hf_hybrid_step_noalloc(g, q, k, v, ring, c["top_k"], hf.HF_STEP_COMMIT, S, z, idx, out)
        torch.cuda.synchronize()
        assert torch.equal(idx.cpu(), idx_r)
        assert (ring.head, ring.n_committed) == desc_r
        o = out.cpu()
        assert_close(o.numpy(), out_r.numpy().astype(np.float64), "noalloc vs workspace step")
        assert torch.equal(o, out_r)
        assert torch.equal(S.cpu(), S_r) and torch.equal(z.cpu(), z_r)
