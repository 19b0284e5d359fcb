"""Host-side pieces of bench.py (no GPU): the visible-pair count behind the
FLOP figures, and the one-GPU guard."""
import subprocess
import sys

import numpy as np
import pytest

import workloads as W
from _lib import ROOT
from oracle import ffa_oracle as O

sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [1, 2, 3])
def test_visible_pairs_match_oracle_mask(n):
    w = W.config(n)
    sl = O.normalise_slices(*w.slices(), w.Tq, w.Tk)
    assert bench.visible_pairs(w) == O.visible_count(sl, w.Tq, w.Tk)


def test_visible_pairs_random_slices():
    rng = np.random.default_rng(3)
    for _ in range(20):
        Tq, Tk = int(rng.integers(1, 200)), int(rng.integers(1, 200))
        qr, kr, ty = W.random_slices(rng, Tq, Tk, n_dummies=2)
        w = W.Workload("r", Tq, Tk, 1, 1, 64, tuple(map(tuple, qr.tolist())),
                       tuple(map(tuple, kr.tolist())), tuple(ty.tolist()))
        sl = O.normalise_slices(qr, kr, ty, Tq, Tk)
        assert bench.visible_pairs(w) == O.visible_count(sl, Tq, Tk)


def test_large_configs_closed_form():
    assert bench.visible_pairs(W.config(4)) == 8 * 8192 * 8193 // 2
    assert bench.visible_pairs(W.config(5)) == 125845504


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stdout
