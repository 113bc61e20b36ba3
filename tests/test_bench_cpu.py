"""Host-side pieces of the benchmark (no GPU): the kept-block flop count every TF/s figure
divides by, against a brute-force count of query-key pairs; the --gpus guard."""
import subprocess
import sys
from pathlib import Path

import numpy as np
import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


@pytest.mark.parametrize("Nq,Nk,bq,bk,D", [(200, 300, 64, 64, 128), (96, 400, 32, 16, 64), (64, 64, 64, 64, 128),
                                          (4680, 9360, 64, 64, 128)])
def test_kept_flops_brute_force(Nq, Nk, bq, bk, D):
    rng = np.random.default_rng(Nq + Nk)
    nqb, nkb = -(-Nq // bq), -(-Nk // bk)
    k = max(1, nkb // 3)
    idx = np.stack([np.sort(rng.choice(nkb, k, replace=False)) for _ in range(2 * nqb)]).reshape(1, 2, nqb, k)
    pairs = 0
    for h in range(2):
        for i in range(nqb):
            nq = min(bq, Nq - i * bq)
            nk = sum(min(bk, Nk - j * bk) for j in idx[0, h, i])
            pairs += nq * nk
    assert bench.kept_flops(idx, Nq, Nk, bq, bk, D) == 4.0 * D * pairs


def test_keep_all_flops_equal_dense():
    Nq, Nk, bq, bk, D = 4680, 9360, 64, 64, 128
    nqb, nkb = -(-Nq // bq), -(-Nk // bk)
    idx = np.broadcast_to(np.arange(nkb), (1, 12, nqb, nkb))
    assert bench.kept_flops(idx, Nq, Nk, bq, bk, D) == 4.0 * D * Nq * Nk * 12


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "not supported" in r.stderr
