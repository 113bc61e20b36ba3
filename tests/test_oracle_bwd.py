"""Pins of the oracle's backward pass (CPU): every analytic gradient against central
finite differences of the oracle's own forward functions (a different computation: the
forward never forms a gradient), plus invariants the mathematics fixes.  The selection
is held fixed (it is piecewise constant in the inputs)."""
import numpy as np
import pytest

import oracle

H_FD = 1e-5


def _fd(f, x, h=H_FD):
    """Central differences of the scalar f() with respect to every entry of x (in place)."""
    g = np.zeros_like(x)
    flat, gf = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        flat[i] = keep + h
        fp = f()
        flat[i] = keep - h
        fm = f()
        flat[i] = keep
        gf[i] = (fp - fm) / (2 * h)
    return g


def _idx(rng, B, H, nqb, nkb, k):
    return np.stack([np.stack([np.stack([np.sort(rng.choice(nkb, k, replace=False)) for _ in range(nqb)])
                               for _ in range(H)]) for _ in range(B)]).astype(np.int32)


@pytest.mark.parametrize("Nq,Nk,bq,bk,k", [(6, 12, 3, 4, 2), (7, 11, 3, 4, 2), (4, 8, 4, 2, 4)])
def test_sparse_attn_bwd_finite_differences(Nq, Nk, bq, bk, k):
    rng = np.random.default_rng(Nq * 100 + Nk)
    B, H, D = 1, 2, 4
    Q = rng.standard_normal((B, H, Nq, D))
    K = rng.standard_normal((B, H, Nk, D))
    V = rng.standard_normal((B, H, Nk, D))
    dO = rng.standard_normal((B, H, Nq, D))
    idx = _idx(rng, B, H, -(-Nq // bq), -(-Nk // bk), k)
    loss = lambda: float((oracle.sparse_attn(Q, K, V, idx, bq, bk) * dO).sum())
    dQ, dK, dV = oracle.sparse_attn_bwd(Q, K, V, idx, bq, bk, dO)
    for ana, x in ((dQ, Q), (dK, K), (dV, V)):
        np.testing.assert_allclose(ana, _fd(loss, x), rtol=1e-6, atol=1e-8)


def test_sparse_attn_bwd_invariants():
    """Per plane: softmax weights sum to one, so sum_u dV_u = sum_t dO_t; each query's
    logit gradients sum to zero, so sum_u dK_u = 0 (over every key)."""
    rng = np.random.default_rng(7)
    B, H, D, Nq, Nk, bq, bk, k = 2, 2, 8, 10, 24, 4, 4, 3
    Q, K, V = (rng.standard_normal((B, H, n, D)) for n in (Nq, Nk, Nk))
    dO = rng.standard_normal((B, H, Nq, D))
    idx = _idx(rng, B, H, -(-Nq // bq), -(-Nk // bk), k)
    dQ, dK, dV = oracle.sparse_attn_bwd(Q, K, V, idx, bq, bk, dO)
    np.testing.assert_allclose(dV.sum(axis=2), dO.sum(axis=2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-12)
    # keys no block kept get no gradient
    kept = np.zeros((B, H, Nk), bool)
    for b in range(B):
        for h in range(H):
            for j in np.unique(idx[b, h]):
                kept[b, h, j * bk:(j + 1) * bk] = True
    assert np.all(dK[~kept] == 0) and np.all(dV[~kept] == 0)


def test_linear_readout_bwd_finite_differences():
    rng = np.random.default_rng(3)
    B, H, Nq, D, eps = 1, 2, 5, 4, 1e-3
    Q = rng.standard_normal((B, H, Nq, D))
    S = rng.standard_normal((B, H, D, D))
    z = rng.random((B, H, D)) + 0.5
    dO = rng.standard_normal((B, H, Nq, D))
    loss = lambda: float((oracle.linear_readout(Q, S, z, bq=2, eps=eps) * dO).sum())
    dQ, dS, dz = oracle.linear_readout_bwd(Q, S, z, dO, eps)
    for ana, x in ((dQ, Q), (dS, S), (dz, z)):
        np.testing.assert_allclose(ana, _fd(loss, x), rtol=1e-6, atol=1e-8)


def test_linear_readout_bwd_euler():
    """With eps = 0 the readout is homogeneous of degree 0 in (S, z) together, so
    sum(dS * S) + sum(dz * z) = 0 (Euler's relation)."""
    rng = np.random.default_rng(4)
    B, H, Nq, D = 1, 3, 9, 8
    Q = rng.standard_normal((B, H, Nq, D))
    S = rng.standard_normal((B, H, D, D))
    z = rng.random((B, H, D)) + 0.5
    dO = rng.standard_normal((B, H, Nq, D))
    _, dS, dz = oracle.linear_readout_bwd(Q, S, z, dO, 0.0)
    e = (dS * S).sum(axis=(2, 3)) + (dz * z).sum(axis=2)
    np.testing.assert_allclose(e, 0.0, atol=1e-10)


def test_absorb_bwd_finite_differences():
    rng = np.random.default_rng(5)
    B, H, n, D = 1, 2, 6, 4
    K = rng.standard_normal((B, H, n, D))
    V = rng.standard_normal((B, H, n, D))
    S0 = rng.standard_normal((B, H, D, D))
    z0 = rng.random((B, H, D))
    dS = rng.standard_normal((B, H, D, D))
    dz = rng.standard_normal((B, H, D))

    def loss():
        S, z = oracle.absorb(K, V, S0, z0)
        return float((S * dS).sum() + (z * dz).sum())

    dK, dV = oracle.absorb_bwd(K, V, dS, dz)
    for ana, x in ((dK, K), (dV, V)):
        np.testing.assert_allclose(ana, _fd(loss, x), rtol=1e-6, atol=1e-8)


def test_absorb_bwd_linear_in_values():
    """The state is linear in V, so sum_u dV_u . v_u = sum(dS * (S_after - S_before))."""
    rng = np.random.default_rng(6)
    B, H, n, D = 1, 2, 20, 8
    K, V = rng.standard_normal((B, H, n, D)), rng.standard_normal((B, H, n, D))
    dS, dz = rng.standard_normal((B, H, D, D)), rng.standard_normal((B, H, D))
    _, dV = oracle.absorb_bwd(K, V, dS, dz)
    S, _ = oracle.absorb(K, V)
    np.testing.assert_allclose((dV * V).sum(axis=(2, 3)), (dS * S).sum(axis=(2, 3)), rtol=1e-12)


def test_hybrid_step_bwd_finite_differences():
    """The step's output (sparse + linear, selection fixed) against the sum of both
    branches' gradients."""
    rng = np.random.default_rng(8)
    B, H, D, Nq, Nk, bq, bk, k, eps = 1, 1, 4, 6, 12, 3, 4, 2, 1e-3
    Q = rng.standard_normal((B, H, Nq, D))
    K, V = rng.standard_normal((B, H, Nk, D)), rng.standard_normal((B, H, Nk, D))
    S, z = rng.standard_normal((B, H, D, D)), rng.random((B, H, D)) + 0.5
    dO = rng.standard_normal((B, H, Nq, D))
    idx = _idx(rng, B, H, -(-Nq // bq), -(-Nk // bk), k)

    def loss():
        out = oracle.sparse_attn(Q, K, V, idx, bq, bk) + oracle.linear_readout(Q, S, z, bq=bq, eps=eps)
        return float((out * dO).sum())

    dQ, dK, dV, dS, dz = oracle.hybrid_step_bwd(Q, K, V, S, z, idx, bq, bk, dO, eps)
    for ana, x in ((dQ, Q), (dK, K), (dV, V), (dS, S), (dz, z)):
        np.testing.assert_allclose(ana, _fd(loss, x), rtol=1e-6, atol=1e-8)
