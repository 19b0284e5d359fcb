"""ffa_block_slices (host C++ through the C ABI): a BlockMask-style block list
becomes disjoint FULL slices covering exactly the listed blocks, checked
against the oracle's block visibility (defined cell by cell)."""
import numpy as np
import pytest

from _lib import ensure_built, ffa
from oracle import ffa_oracle as O


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _random_blocks(rng, Tq, Tk, bq, bk, density):
    nqb, nkb = -(-Tq // bq), -(-Tk // bk)
    width = nkb + 2
    num = np.zeros(nqb, np.int32)
    idx = np.full((nqb, width), -5, np.int32)  # padding past the count is ignored
    for b in range(nqb):
        listed = np.nonzero(rng.random(nkb) < density)[0]
        rng.shuffle(listed)
        num[b] = listed.size
        idx[b, :listed.size] = listed
    return num, idx


def _check(num, idx, Tq, Tk, bq, bk):
    qr, kr, ty = ffa.ffa_block_slices(num, idx, Tq, Tk, bq, bk)
    assert np.all(ty == ffa.FULL)
    order = [(a[0], b[0]) for a, b in zip(qr.tolist(), kr.tolist())]
    assert order == sorted(order)
    M = O.visibility(O.normalise_slices(qr, kr, ty, Tq, Tk), np.arange(Tq), np.arange(Tk))
    assert M.max(initial=0) <= 1, "slices overlap"
    assert np.array_equal(M > 0, O.block_visibility(num, idx, bq, bk, Tq, Tk))
    return qr.shape[0]


@pytest.mark.parametrize("seed", range(6))
def test_random_block_lists(seed):
    rng = np.random.default_rng(seed)
    Tq, Tk = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    bq, bk = int(rng.choice([16, 32, 64, 128])), int(rng.choice([16, 32, 64, 128]))
    for density in (0.0, 0.2, 0.6, 1.0):
        _check(*_random_blocks(rng, Tq, Tk, bq, bk, density), Tq, Tk, bq, bk)


def test_merging_keeps_slices_few():
    n = 16
    Tq = Tk = 128 * n - 50  # ragged last block
    full = np.tile(np.arange(n, dtype=np.int32), (n, 1))
    assert _check(np.full(n, n, np.int32), full, Tq, Tk, 128, 128) == 1          # dense: one slice
    causal_num = np.arange(1, n + 1, dtype=np.int32)
    assert _check(causal_num, full, Tq, Tk, 128, 128) == n                        # one run per row
    # local-global: block 0 for everyone plus a 3-block window; the global
    # column continues over every row and becomes one slice
    num = np.zeros(n, np.int32)
    idx = np.zeros((n, 4), np.int32)
    for b in range(n):
        blocks = sorted({0} | set(range(max(0, b - 2), b + 1)))
        num[b] = len(blocks)
        idx[b, :len(blocks)] = blocks[::-1]
    R = _check(num, idx, Tq, Tk, 128, 128)
    assert R <= n + 1, R


def test_bad_lists_raise():
    with pytest.raises(ffa.FfaError, match="count"):
        ffa.ffa_block_slices([3], [[0, 1]], 100, 100, 128, 64)
    with pytest.raises(ffa.FfaError, match="listed twice"):
        ffa.ffa_block_slices([2], [[1, 1]], 100, 100, 128, 64)
    with pytest.raises(ffa.FfaError, match="key block 2"):
        ffa.ffa_block_slices([1], [[2]], 100, 100, 128, 64)
    assert ffa.ffa_block_slices([], [], 0, 0)[0].shape == (0, 2)
