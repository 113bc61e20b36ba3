"""Pins of the oracle's relative temporal rotary embedding (CPU).

The oracle rotates each query by the clamped frame offset to the key's frame.  Within
the cap that must equal the usual absolute-position form, written here independently
with complex arithmetic (feature pair (2i, 2i+1) as the complex number x_2i + j x_2i+1,
turned by exp(j a theta_i)) and fed to the oracle's plain sparse attention, which has
pins of its own.  The clamp is pinned by key frames whose offsets lie beyond the cap:
identical keys there must get identical weights."""
import numpy as np
import pytest

import oracle


def _idx(rng, B, H, nqb, nkb, k):
    return np.stack([np.stack([np.stack([np.sort(rng.choice(nkb, k, replace=False)) for _ in range(nqb)])
                               for _ in range(H)]) for _ in range(B)]).astype(np.int32)


def _rotate_absolute(X, pos, DT, base):
    """Rows of X [..., N, D] turned by absolute positions pos [N] (complex form)."""
    i = np.arange(DT // 2)
    theta = base ** (-2.0 * i / DT)
    z = X[..., 0:DT:2] + 1j * X[..., 1:DT:2]
    z = z * np.exp(1j * pos[:, None] * theta[None, :])
    out = X.copy()
    out[..., 0:DT:2] = z.real
    out[..., 1:DT:2] = z.imag
    return out


CASES = [
    # B, H, D, T, n_frames, C, bq, bk, k, DT, base
    (1, 2, 16, 8, 5, 2, 4, 4, 5, 8, 10000.0),
    (1, 1, 12, 6, 4, 2, 5, 3, 4, 12, 100.0),     # every feature temporal, blocks across frames
    (2, 1, 8, 5, 3, 1, 3, 4, 2, 4, 10.0),        # ragged blocks, one chunk frame
    (1, 2, 16, 12, 6, 3, 8, 8, 6, 16, 10000.0),
]


@pytest.mark.parametrize("case", CASES)
def test_within_cap_equals_absolute_positions(case):
    B, H, D, T, nfr, C, bq, bk, k, DT, base = case
    rng = np.random.default_rng(sum(case[:9]))
    Nq, Nk = C * T, nfr * T
    Q = rng.standard_normal((B, H, Nq, D))
    K = rng.standard_normal((B, H, Nk, D))
    V = rng.standard_normal((B, H, Nk, D))
    idx = _idx(rng, B, H, oracle.n_blocks(Nq, bq), oracle.n_blocks(Nk, bk), k)
    a0 = 37.0   # any common shift of the absolute positions
    kpos = a0 + np.arange(Nk) // T
    qpos = a0 + (Nk - Nq + np.arange(Nq)) // T
    want = oracle.sparse_attn(_rotate_absolute(Q, qpos, DT, base), _rotate_absolute(K, kpos, DT, base), V, idx,
                              bq, bk)
    for cap in (nfr - 1, nfr + 5):   # every offset within the cap
        got = oracle.sparse_attn_rope(Q, K, V, idx, bq, bk, T, DT, cap, base)
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)
    # the rotation is not a no-op here
    plain = oracle.sparse_attn(Q, K, V, idx, bq, bk)
    assert np.abs(plain - want).max() > 1e-3


def test_cap_zero_and_no_temporal_features_are_plain_attention():
    rng = np.random.default_rng(5)
    B, H, D, T, nfr, C, bq, bk, k = 1, 2, 8, 4, 4, 2, 4, 4, 3
    Q = rng.standard_normal((B, H, C * T, D))
    K = rng.standard_normal((B, H, nfr * T, D))
    V = rng.standard_normal((B, H, nfr * T, D))
    idx = _idx(rng, B, H, 2, 4, k)
    plain = oracle.sparse_attn(Q, K, V, idx, bq, bk)
    np.testing.assert_array_equal(oracle.sparse_attn_rope(Q, K, V, idx, bq, bk, T, 8, 0, 10000.0), plain)
    np.testing.assert_array_equal(oracle.sparse_attn_rope(Q, K, V, idx, bq, bk, T, 0, 3, 10000.0), plain)


@pytest.mark.parametrize("cap,beyond", [(2, (3, 4)), (1, (-2, -1))])
def test_offsets_beyond_the_cap_score_alike(cap, beyond):
    """One query; key frames at offsets `beyond` (both at or past the clamp) hold the same
    key row, with values e_0 and e_1: their weights, hence out[0] and out[1], agree exactly
    when clamped, and differ without the clamp."""
    T, D, DT = 1, 4, 4
    nfr, C = 5, 3
    Nk, Nq = nfr, C
    t = 0 if beyond[0] < 0 else C - 1          # query in the chunk's first or last frame
    fq = Nk - Nq + t
    rng = np.random.default_rng(11)
    q = rng.standard_normal(D)
    kr = rng.standard_normal(D)
    Q = np.zeros((1, 1, Nq, D))
    Q[0, 0, :] = q
    K = rng.standard_normal((1, 1, Nk, D))
    V = np.zeros((1, 1, Nk, D))
    V[0, 0, :, 3] = 1.0                        # other keys land in feature 3
    for e, off in enumerate(beyond):
        fk = fq - off
        K[0, 0, fk] = kr
        V[0, 0, fk] = 0.0
        V[0, 0, fk, e] = 1.0
    idx = np.zeros((1, 1, Nq, Nk), dtype=np.int32) + np.arange(Nk, dtype=np.int32)
    got = oracle.sparse_attn_rope(Q, K, V, idx, 1, 1, T, DT, cap, 3.0)[0, 0, t]
    assert got[0] == got[1]
    free = oracle.sparse_attn_rope(Q, K, V, idx, 1, 1, T, DT, 10, 3.0)[0, 0, t]
    assert abs(free[0] - free[1]) > 1e-6


def test_hybrid_step_rope_without_rotation_is_the_step():
    rng = np.random.default_rng(8)
    B, H, D, T, nfr, C, bq, bk, k = 1, 2, 8, 4, 4, 2, 4, 4, 3
    Q = rng.standard_normal((B, H, C * T, D))
    K = rng.standard_normal((B, H, nfr * T, D))
    V = rng.standard_normal((B, H, nfr * T, D))
    S = rng.random((B, H, D, D))
    z = rng.random((B, H, D)) + 1.0
    want, idx_want, _ = oracle.hybrid_step(Q, K, V, S, z, bq, bk, k)
    got, idx = oracle.hybrid_step_rope(Q, K, V, S, z, bq, bk, k, T, 0, 2)
    np.testing.assert_array_equal(idx, idx_want)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
