"""The seeded input generator: determinism, bf16 rounding, per-frame reproducibility."""

import numpy as np
import torch

from hybrid_sparse_linear_hf_amd import synth


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100_000).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # exact halfway cases: ties to even
    bits = synth.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = synth.f32_from_bf16_bits(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_tiny_stream_is_seeded():
    a, b = synth.tiny_stream(seed=0), synth.tiny_stream(seed=0)
    np.testing.assert_array_equal(a.k_all, b.k_all)
    assert a.q.shape == (1, 1, 64, 64) and a.k_all.shape == (1, 1, 7 * 64, 64)
    assert not np.array_equal(a.q, synth.tiny_stream(seed=1).q)


def test_field_frames_are_per_frame_reproducible():
    src = synth.FieldSource(D=32, gh=6, gw=10, seed=0, layer=0, stream=0, head=3)
    whole = src.frames_bf16(synth.K_ID, 2, 3)
    again = np.concatenate([src.frames_bf16(synth.K_ID, f, 1) for f in (2, 3, 4)])
    np.testing.assert_array_equal(whole, again)
    assert whole.shape == (3 * 60, 32)
    # Q, K, V of one head differ; the same head in another stream differs
    assert not np.array_equal(src.frames_bf16(synth.Q_ID, 2, 1), src.frames_bf16(synth.K_ID, 2, 1))
    other = synth.FieldSource(D=32, gh=6, gw=10, seed=0, layer=0, stream=1, head=3)
    assert not np.array_equal(other.frames_bf16(synth.K_ID, 2, 1), src.frames_bf16(synth.K_ID, 2, 1))


def test_field_statistics():
    src = synth.FieldSource(D=128, seed=0, head=0)
    x = synth.f32_from_bf16_bits(src.frames_bf16(synth.V_ID, 0, 2))
    # N(0,1)*0.5 overall scale; a spatially structured (rank-8) component
    assert 0.15 < x.var() < 0.35
    sv = np.linalg.svd(x - x.mean(0), compute_uv=False)
    assert sv[:8].sum() / sv.sum() > 0.15


def test_layer_config_geometry():
    c = synth.LAYER_832x480
    assert (c.Nq, c.Nk, c.n_qb, c.n_kb, c.top_k()) == (4680, 9360, 74, 147, 37)
    w = synth.LAYER_832x480_W21
    assert (w.Nk, w.n_kb) == (32760, 512)
    t = synth.TINY
    assert (t.Nq, t.Nk, t.n_qb, t.n_kb, t.top_k()) == (64, 256, 4, 16, 2)
