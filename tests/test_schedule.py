"""Chunk-aware growth schedule ([LF-de] §2.1): the oracle (exact enumeration of the
breakpoints of the kept-block total) pinned to hand-computed cases and invariants, and the
library's host implementation (hf_cag_schedule, a bisection, no GPU work) compared with it:
keep counts exactly, beta and the sparsities to 1e-12."""

import math

import numpy as np
import pytest

import hybrid_sparse_linear_hf_amd as hf
import oracle


def work(ks):
    return sum(ks)


def test_first_chunk_dense_and_zero_target_is_dense():
    k, s, beta = oracle.cag_schedule([147] * 6, 0.75, 0.0, 0.9)
    assert k == [147] * 6 and s[0] == 0.0      # (the last chunks may keep every block at s_i > 0)
    k, s, _ = oracle.cag_schedule([147, 147, 147], 0.8, 0.5, 0.9)
    assert k[0] == 147 and s[0] == 0.0


def test_hand_computed_two_chunks():
    # target 0.25 of 200 dense blocks: 150 kept; beta = 0 already keeps 100 + 50
    assert oracle.cag_schedule([100, 100], 0.5, 0.25, 0.9) == ([100, 50], [0.0, 0.5], 0.0)
    # target 0.1: 180 kept, so chunk 1 keeps 80, which needs (1 - s_1) * 100 > 79, i.e.
    # s_1 = 0.5 - beta / sqrt(2) < 0.21: the smallest beta is 0.29 sqrt(2)
    k, s, beta = oracle.cag_schedule([100, 100], 0.5, 0.1, 0.9)
    assert k == [100, 80]
    assert abs(beta - 0.29 * math.sqrt(2.0)) < 1e-12
    assert abs(s[1] - 0.21) < 1e-12


def test_cap_and_monotone_sparsity():
    n_kb = [147] * 12
    k, s, beta = oracle.cag_schedule(n_kb, 0.95, 0.45, 0.5)
    assert max(s) <= 0.5
    assert all(s[i] <= s[i + 1] for i in range(len(s) - 1))          # later chunks never denser
    assert all(k[i] >= k[i + 1] for i in range(len(k) - 1))


@pytest.mark.parametrize("seed", range(6))
def test_beta_is_minimal(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 20))
    n_kb = [int(x) for x in rng.integers(4, 600, n)]
    s_base, s_target, s_max = float(rng.uniform(0.3, 0.95)), float(rng.uniform(0.05, 0.5)), float(rng.uniform(0.5, 0.97))
    k, s, beta = oracle.cag_schedule(n_kb, s_base, s_target, s_max)
    goal = (1.0 - s_target) * sum(n_kb)
    assert work(k) >= goal
    if beta > 0:
        # a slightly smaller beta misses the goal
        lower = [min(max(math.ceil((1.0 - (0.0 if i == 0 else min(max(s_base - beta * (1 - 1e-9) / math.sqrt(i + 1), 0.0), s_max))) * n_kb[i]), 1), n_kb[i]) for i in range(n)]
        assert work(lower) < goal


@pytest.mark.parametrize("seed", range(10))
def test_library_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 40))
    n_kb = [int(x) for x in rng.integers(1, 1536, n)]
    args = (float(rng.uniform(0, 0.99)), float(rng.uniform(0, 0.9)), float(rng.uniform(0, 0.99)))
    got = hf.hf_cag_schedule(n_kb, *args)
    ref = oracle.cag_schedule(n_kb, *args)
    assert got[0] == ref[0]
    # the bisection stops within rounding of the breakpoint the oracle finds exactly
    assert abs(got[2] - ref[2]) <= 1e-12 * max(1.0, ref[2])
    assert np.allclose(got[1], ref[1], rtol=0, atol=1e-12)


def test_library_rejects_bad_arguments():
    with pytest.raises(hf.HFError):
        hf.hf_cag_schedule([], 0.5, 0.2, 0.9)
    with pytest.raises(hf.HFError):
        hf.hf_cag_schedule([10, 0], 0.5, 0.2, 0.9)
    for bad in ((1.0, 0.2, 0.9), (0.5, -0.1, 0.9), (0.5, 0.2, float("nan"))):
        with pytest.raises(hf.HFError):
            hf.hf_cag_schedule([10, 10], *bad)


def brute_keep(n_kb, s_base, s_max, beta):
    """The schedule's keep counts at one beta, straight from the definition."""
    ks = [n_kb[0]]
    for i in range(1, len(n_kb)):
        s = min(max(s_base - beta / math.sqrt(i + 1), 0.0), s_max)
        ks.append(int(min(max(math.ceil((1.0 - s) * n_kb[i]), 1), n_kb[i])))
    return ks


@pytest.mark.parametrize("seed", range(8))
def test_oracle_against_scan_of_beta(seed):
    """Scanning beta on a fine grid with the definition: the first grid point that reaches the
    goal lies just above the oracle's beta, and gives the oracle's keep counts."""
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(2, 7))
    n_kb = [int(x) for x in rng.integers(2, 40, n)]
    s_base, s_target, s_max = float(rng.uniform(0.3, 0.95)), float(rng.uniform(0.05, 0.4)), float(rng.uniform(0.5, 0.97))
    k, s, beta = oracle.cag_schedule(n_kb, s_base, s_target, s_max)
    goal = (1.0 - s_target) * sum(n_kb)
    step = 1e-4
    grid = np.arange(0.0, s_base * math.sqrt(n) + 1.0 + step, step)
    first = next(b for b in grid if sum(brute_keep(n_kb, s_base, s_max, b)) >= goal)
    assert beta <= first < beta + step + 1e-12
    if beta > 0 and first - beta > 1e-9:
        assert brute_keep(n_kb, s_base, s_max, first) == k
