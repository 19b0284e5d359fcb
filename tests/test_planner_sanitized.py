"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

planner.cpp is built on its own with g++ (no GPU code) into the driver
tests/native/planner_driver.cpp, with -fsanitize=address,undefined and no
recovery, so any out-of-bounds access, use after free, leak, signed overflow
or bad shift ends the run with a report.  The driver is fed random slice
lists (valid and invalid: start > end, ranges past the axis, negative and
int32-extreme values, unknown types), the five workload slice lists, several
tile shapes in both orientations, overlapping pairs for the disjointness
check, and BlockMask-style block lists (valid and invalid).  The plans it
prints are compared with the oracle's tile set, so the run checks results as
well as memory safety.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads as W
from oracle import ffa_oracle as O
from range_masked_attention_amd import _build

I32_MAX = 2**31 - 1


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("asan") / "planner_driver")
    try:
        _build.build_planner_sanitized(out)
    except RuntimeError as e:
        if "asan" in str(e).lower() or "sanitizer" in str(e).lower():
            pytest.skip(f"sanitizer runtime not available: {e}")
        raise
    return out


def _run(driver, lines):
    env = dict(os.environ)
    # the sanitizer runtime must come first unless something else is preloaded
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([driver], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=300)
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.returncode, r.stderr[-4000:])
    return r.stdout.splitlines()


def _plan_line(Tq, Tk, bm, bn, tr, qr, kr, ty):
    qr, kr, ty = np.asarray(qr).reshape(-1, 2), np.asarray(kr).reshape(-1, 2), np.asarray(ty).reshape(-1)
    body = " ".join(f"{int(a)} {int(b)} {int(c)} {int(d)} {int(t)}" for (a, b), (c, d), t in zip(qr, kr, ty))
    return f"plan {Tq} {Tk} {bm} {bn} {int(tr)} {len(ty)} {body}".strip()


def _parse(out):
    """Split the driver's answers into (status, payload lines) per request."""
    res, i = [], 0
    while i < len(out):
        head = out[i].split(" ", 1)
        if head[0] == "ok" and len(head) == 2 and head[1].isdigit():
            n = int(head[1])
            res.append(("ok", out[i + 1:i + 1 + n]))
            i += 1 + n
        else:
            res.append((head[0], [head[1] if len(head) > 1 else ""]))
            i += 1
    return res


def _bad_slices(rng, Tq, Tk):
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=4, n_dummies=1)
    qr, kr, ty = qr.astype(np.int64), kr.astype(np.int64), ty.astype(np.int64)
    r = int(rng.integers(0, len(ty)))
    kind = int(rng.integers(0, 7))
    if kind == 0:
        qr[r] = (qr[r][1] + 1, qr[r][0])          # start > end
    elif kind == 1:
        kr[r] = (0, Tk + 1 + int(rng.integers(0, 5)))  # past the axis
    elif kind == 2:
        qr[r] = (-1 - int(rng.integers(0, 3)), 2)  # negative
    elif kind == 3:
        ty[r] = int(rng.choice([2, -1, I32_MAX]))  # unknown type
    elif kind == 4:
        kr[r] = (I32_MAX - 1, I32_MAX)             # int32-extreme values
    elif kind == 5:
        qr[r] = (-(2**31), -(2**31) + 1)
    else:
        kr[r] = (Tk, Tk + 1)
    return qr, kr, ty


def test_random_and_bad_slice_lists(driver):
    rng = np.random.default_rng(2024)
    lines, expect = [], []
    shapes = [(128, 64), (64, 128), (64, 64), (1, 1), (7, 3), (16, 32)]
    for trial in range(240):
        Tq, Tk = int(rng.integers(0, 260)), int(rng.integers(0, 260))
        bm, bn = shapes[trial % len(shapes)]
        tr = bool(trial % 2)
        if trial % 3 == 2 and Tq > 0 and Tk > 0:
            qr, kr, ty = _bad_slices(rng, Tq, Tk)
            lines.append(_plan_line(Tq, Tk, bm, bn, tr, qr, kr, ty))
            expect.append(None)
            continue
        if Tq == 0 or Tk == 0:
            qr, kr, ty = np.zeros((2, 2), np.int64), np.zeros((2, 2), np.int64), np.zeros(2, np.int64)
        else:
            qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=6, n_dummies=int(rng.integers(0, 3)))
        lines.append(_plan_line(Tq, Tk, bm, bn, tr, qr, kr, ty))
        expect.append(O.tile_set(qr, kr, ty, Tq, Tk, bm, bn))
    # tile sizes the planner must refuse, and the workload slice lists
    lines.append(_plan_line(10, 10, 0, 64, False, [[0, 5]], [[0, 5]], [0]))
    expect.append(None)
    for n in (1, 2, 3, 5):
        w = W.config(n)
        for bm, bn, tr in ((128, 64, False), (64, 128, True)):
            lines.append(_plan_line(w.Tq, w.Tk, bm, bn, tr, *w.slices()))
            expect.append(O.tile_set(*w.slices(), w.Tq, w.Tk, bm, bn))
    res = _parse(_run(driver, lines))
    assert len(res) == len(expect)
    for (status, payload), want, line in zip(res, expect, lines):
        if want is None:
            assert status == "error", line[:200]
            continue
        assert status == "ok", (payload, line[:200])
        tr = line.split()[5] == "1"
        got = set()
        for p in payload:
            t, o, r, kind = (int(x) for x in p.split())
            got.add((o, t, r, kind) if tr else (t, o, r, kind))
        assert got == want, line[:200]


def test_disjointness_check(driver):
    lines = [
        "disjoint 100 100 2 0 50 0 50 0 50 100 50 100 1",     # disjoint rectangles
        "disjoint 100 100 2 0 50 0 50 0 40 60 0 100 0",       # rectangles share cells
        "disjoint 100 100 2 0 50 0 50 1 0 50 40 100 0",       # causal slice reaches a FULL one
        "disjoint 100 100 2 0 100 0 100 1 0 50 60 100 0",     # causal triangle vs. the region above it
        "disjoint 100 100 3 0 0 0 0 0 0 100 0 100 1 5 5 0 100 0",  # dummies never overlap
    ]
    res = [s for s, _ in _parse(_run(driver, lines))]
    assert res == ["ok", "overlap", "overlap", "ok", "ok"]


def test_block_lists(driver):
    rng = np.random.default_rng(77)
    lines, expect = [], []
    for trial in range(60):
        T = int(rng.integers(1, 300))
        bq, bk = int(rng.choice([16, 32, 64])), int(rng.choice([16, 32, 64]))
        nqb, nkb = -(-T // bq), -(-T // bk)
        width = nkb
        num = rng.integers(0, nkb + 1, nqb)
        idx = np.zeros((nqb, width), np.int64)
        for b in range(nqb):
            idx[b, :num[b]] = rng.permutation(nkb)[:num[b]]
        bad = trial % 4 == 3
        if bad:
            b = int(rng.integers(0, nqb))
            choice = int(rng.integers(0, 3))
            if choice == 0:
                num[b] = width + 1                        # count past the width
            elif choice == 1 and num[b] > 0:
                idx[b, 0] = nkb                           # index past the axis
            elif num[b] > 1:
                idx[b, 1] = idx[b, 0]                     # a block listed twice
            else:
                num[b] = -1
        lines.append(f"block {T} {T} {bq} {bk} {width} {nqb} " + " ".join(str(int(x)) for x in num) + " " +
                     " ".join(str(int(x)) for x in idx.reshape(-1)))
        expect.append(None if bad else O.block_visibility(num, idx, bq, bk, T, T))
    res = _parse(_run(driver, lines))
    assert len(res) == len(expect)
    for (status, payload), want, line in zip(res, expect, lines):
        if want is None:
            assert status == "error", line[:200]
            continue
        assert status == "ok"
        T = int(line.split()[1])
        qr = [[int(x) for x in p.split()[:2]] for p in payload]
        kr = [[int(x) for x in p.split()[2:]] for p in payload]
        sl = O.normalise_slices(np.array(qr).reshape(-1, 2), np.array(kr).reshape(-1, 2),
                                np.zeros(len(qr), np.int64), T, T)
        M = O.visibility(sl, np.arange(T), np.arange(T))
        assert M.max(initial=0) <= 1 and np.array_equal(M > 0, want), line[:200]
