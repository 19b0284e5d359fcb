"""The host planner against the oracle's tile set: exact equality.

The planner (C++, via ffa_plan_host) and oracle.tile_set share no code: the
oracle materialises each slice's cells and counts them per tile, the planner
works from slice arithmetic.
"""
import numpy as np
import pytest

import workloads as W
from _lib import ensure_built, ffa
from oracle import ffa_oracle as O


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_built()


def _plan_set(Tq, Tk, qr, kr, ty, bm, bn, transpose=False):
    row_ptr, ent, order = ffa.ffa_plan_host(Tq, Tk, qr, kr, ty, bm, bn, transpose)
    out = set()
    for t in range(len(row_ptr) - 1):
        for e in range(row_ptr[t], row_ptr[t + 1]):
            other, r, kind = ent[e]
            out.add((int(t), int(other), int(r), int(kind)) if not transpose
                    else (int(other), int(t), int(r), int(kind)))
    return out, row_ptr, ent, order


def _check_structure(row_ptr, ent, order, qr, kr):
    n = len(row_ptr) - 1
    assert row_ptr[0] == 0 and np.all(np.diff(row_ptr) >= 0) and row_ptr[-1] == len(ent)
    counts = np.diff(row_ptr)
    # order: a permutation; tiles grouped by the smallest slice start row in
    # their list (empty tiles form one group), each group contiguous, groups
    # by descending longest list, inside a group by descending count, then index
    assert sorted(order.tolist()) == list(range(n))
    key = [min((int(qr[e[1]][0]) for e in ent[row_ptr[t]:row_ptr[t + 1]]), default=None) for t in range(n)]
    seq = [key[t] for t in order]
    starts = [i for i in range(n) if i == 0 or seq[i] != seq[i - 1]]
    assert len(starts) == len(set(seq)), "groups must be contiguous"
    heads = [counts[order[i]] for i in starts]
    assert heads == sorted(heads, reverse=True)
    for a, b in zip(order[:-1], order[1:]):
        if key[a] == key[b]:
            assert (counts[a], -a) >= (counts[b], -b)
    # within a tile: sorted by the other tile, then by slice bounds
    for t in range(n):
        keys = [(int(e[0]), *qr[e[1]].tolist(), *kr[e[1]].tolist()) for e in ent[row_ptr[t]:row_ptr[t + 1]]]
        assert keys == sorted(keys)


@pytest.mark.parametrize("transpose", [False, True])
def test_random_slices_match_oracle(transpose):
    rng = np.random.default_rng(100 + transpose)
    for trial in range(80):
        Tq, Tk = int(rng.integers(1, 300)), int(rng.integers(1, 300))
        qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=6, n_dummies=int(rng.integers(0, 4)))
        bm, bn = [(128, 64), (64, 64), (16, 32), (32, 16), (64, 128)][trial % 5]
        got, row_ptr, ent, order = _plan_set(Tq, Tk, qr, kr, ty, bm, bn, transpose)
        assert got == O.tile_set(qr, kr, ty, Tq, Tk, bm, bn)
        _check_structure(row_ptr, ent, order, qr, kr)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_configs_match_oracle(n):
    w = W.config(n)
    qr, kr, ty = w.slices()
    # (128, 64): the forward's and the dQ pass's q-tile lists; (64, 128,
    # transposed): the dK/dV pass's key-tile lists, as the kernels use them
    for bm, bn, tr in [(128, 64, False), (64, 64, True), (64, 128, True)]:
        got, *_ = _plan_set(w.Tq, w.Tk, qr, kr, ty, bm, bn, tr)
        assert got == O.tile_set(qr, kr, ty, w.Tq, w.Tk, bm, bn)


def test_padding_and_permutation_do_not_change_the_device_order():
    """Dummies anywhere and any slice order give the same per-tile entry sequence."""
    w = W.config(5)
    qr, kr, ty = w.slices(padded=False)
    ref_rp, ref_e, ref_o = ffa.ffa_plan_host(w.Tq, w.Tk, qr, kr, ty, 128, 64)
    rng = np.random.default_rng(7)
    perm = rng.permutation(len(ty))
    pq, pk, pt = qr[perm], kr[perm], ty[perm]
    pq, pk, pt = W.pad_slices(pq, pk, pt, len(ty) + 9)
    # move a few dummies to the front
    pq, pk, pt = np.roll(pq, 4, axis=0), np.roll(pk, 4, axis=0), np.roll(pt, 4)
    rp, e, o = ffa.ffa_plan_host(w.Tq, w.Tk, pq, pk, pt, 128, 64)
    assert np.array_equal(rp, ref_rp) and np.array_equal(o, ref_o)
    assert np.array_equal(e[:, [0, 2]], ref_e[:, [0, 2]])
    # same slices, named by their new positions
    assert np.array_equal(qr[ref_e[:, 1]], pq[e[:, 1]]) and np.array_equal(kr[ref_e[:, 1]], pk[e[:, 1]])


def test_entry_counts_closed_form():
    w = W.config(4)
    rp, e, o = ffa.ffa_plan_host(w.Tq, w.Tk, *w.slices(), 128, 64)
    assert (e[:, 2] == 0).sum() == 8 * sum(2 * t for t in range(64))
    assert (e[:, 2] == 1).sum() == 8 * 128
    # q tile t of each document lists 2t + 2 k tiles
    counts = np.diff(rp)
    assert np.array_equal(np.sort(counts), np.sort(np.tile(2 * np.arange(64) + 2, 8)))


def test_empty_inputs():
    rp, e, o = ffa.ffa_plan_host(100, 100, np.zeros((3, 2)), np.zeros((3, 2)), np.zeros(3), 64, 64)
    assert len(e) == 0 and np.all(rp == 0) and len(o) == 2
    rp, e, o = ffa.ffa_plan_host(0, 0, np.zeros((0, 2)), np.zeros((0, 2)), np.zeros(0), 64, 64)
    assert len(e) == 0


def test_planner_errors():
    with pytest.raises(ffa.FfaError, match="k range"):
        ffa.ffa_plan_host(10, 10, [[0, 5]], [[3, 2]], [0], 64, 64)
    with pytest.raises(ffa.FfaError, match="tile sizes"):
        ffa.ffa_plan_host(10, 10, [[0, 5]], [[0, 2]], [0], 0, 64)
