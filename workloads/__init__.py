"""Seeded synthetic workloads for range-masked attention.

This module only *describes* inputs: token counts, head counts, head size, the
slice lists (q_ranges, k_ranges, attn_type_map) and seeded random tensors.  It
contains none of the attention arithmetic, so both the CPU oracle (tests) and
the HIP path (tests, bench) can draw identical bits from it.

Slice conventions follow the MagiAttention issue "Using dummy/padded attention
slices with flex_flash_attn_func for torch.compile static shapes": ranges are
int32 ``[start, end)`` rows, type 0 = FULL and 1 = CAUSAL (reporter's repro
script), and padding rows use ``start == end`` (maintainer reply, padding
mechanism).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

FULL = 0
CAUSAL = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    Tq: int
    Tk: int
    hq: int
    hkv: int
    d: int
    q_ranges: Tuple[Tuple[int, int], ...]
    k_ranges: Tuple[Tuple[int, int], ...]
    types: Tuple[int, ...]
    softcap: float = 0.0
    backward: bool = False
    r_max: Optional[int] = None  # pad the slice list to this many rows

    @property
    def scale(self) -> float:
        # default softmax scale 1/sqrt(head_dim)
        return 1.0 / math.sqrt(self.d)

    def slices(self, padded: bool = True):
        """(q_ranges [R,2], k_ranges [R,2], types [R]) as int32 numpy arrays."""
        qr = np.asarray(self.q_ranges, dtype=np.int32).reshape(-1, 2)
        kr = np.asarray(self.k_ranges, dtype=np.int32).reshape(-1, 2)
        ty = np.asarray(self.types, dtype=np.int32).reshape(-1)
        if padded and self.r_max is not None:
            qr, kr, ty = pad_slices(qr, kr, ty, self.r_max)
        return qr, kr, ty


def pad_slices(q_ranges, k_ranges, types, r_max: int, fill: int = 0, fill_type: int = FULL):
    """Pad a slice list to ``r_max`` rows with ``[fill, fill]`` dummy slices.

    This is the static-shape padding from the MagiAttention issue on dummy
    slices (the reporter's ``make_padded_ranges`` idea and the padded call of
    the repro script: zero rows and type 0).
    """
    q_ranges = np.asarray(q_ranges, dtype=np.int32).reshape(-1, 2)
    k_ranges = np.asarray(k_ranges, dtype=np.int32).reshape(-1, 2)
    types = np.asarray(types, dtype=np.int32).reshape(-1)
    n = q_ranges.shape[0]
    if n > r_max:
        raise ValueError(f"{n} slices exceed r_max={r_max}")
    qp = np.full((r_max, 2), fill, dtype=np.int32)
    kp = np.full((r_max, 2), fill, dtype=np.int32)
    tp = np.full((r_max,), fill_type, dtype=np.int32)
    qp[:n], kp[:n], tp[:n] = q_ranges, k_ranges, types
    return qp, kp, tp


def doc_lengths(total: int = 16384, lo: int = 256, hi: int = 4096, seed: int = 0) -> List[int]:
    """Document lengths uniform in [lo, hi], drawn until they cover ``total``.

    The last document is truncated so the lengths sum to ``total`` exactly.
    """
    rng = np.random.default_rng(seed)
    out, s = [], 0
    while s < total:
        x = int(rng.integers(lo, hi + 1))
        x = min(x, total - s)
        out.append(x)
        s += x
    return out


def _tiny() -> Workload:
    return Workload("tiny", 256, 256, 2, 1, 64,
                    ((0, 128), (128, 256)), ((0, 128), (0, 256)), (FULL, CAUSAL),
                    r_max=4)


def _pages() -> Workload:
    # the repro script's shapes: 2048 tokens, 8 q heads, 2 kv heads, head_dim 64,
    # two real slices padded to 20 rows
    return Workload("pages_shaped", 2048, 2048, 8, 2, 64,
                    ((0, 1024), (1024, 2048)), ((0, 1024), (0, 2048)), (FULL, CAUSAL),
                    backward=True, r_max=20)


def _docs() -> Workload:
    lens = doc_lengths()
    qr, s = [], 0
    for n in lens:
        qr.append((s, s + n))
        s += n
    return Workload("packed_docs", 16384, 16384, 16, 16, 128,
                    tuple(qr), tuple(qr), tuple([CAUSAL] * len(qr)), r_max=64)


def _long() -> Workload:
    qr = tuple((8192 * b, 8192 * (b + 1)) for b in range(8))
    return Workload("long_packed", 65536, 65536, 32, 8, 128, qr, qr, (CAUSAL,) * 8,
                    backward=True)


def _mixed() -> Workload:
    qr, kr, ty = [], [], []
    blk, T = 1024, 32768
    for b in range(T // blk):
        s, e = b * blk, (b + 1) * blk
        if b == 0:
            qr.append((s, e)); kr.append((0, e)); ty.append(CAUSAL)
            continue
        qr.append((s, e)); kr.append((0, 512)); ty.append(FULL)           # global sink
        qr.append((s, e)); kr.append((max(512, e - 4096), e)); ty.append(CAUSAL)  # window
    return Workload("mixed_flex", T, T, 32, 4, 128, tuple(qr), tuple(kr), tuple(ty),
                    softcap=50.0, backward=True)


CONFIGS = {1: _tiny(), 2: _pages(), 3: _docs(), 4: _long(), 5: _mixed()}


def config(n: int) -> Workload:
    return CONFIGS[n]


def make_tensors(Tq: int, Tk: int, hq: int, hkv: int, d: int, seed: int = 0,
                 with_dout: bool = True):
    """Seeded bf16 q, k, v (and dO), drawn on the CPU in that order.

    ``torch.randn`` in float32 from ``torch.Generator().manual_seed(seed)``,
    then rounded to bfloat16, so every consumer sees the same bits.
    """
    import torch
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((Tq, hq, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((Tk, hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((Tk, hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    if not with_dout:
        return q, k, v, None
    do = torch.randn((Tq, hq, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, do


def workload_tensors(w: Workload, seed: int = 0, with_dout: Optional[bool] = None):
    if with_dout is None:
        with_dout = w.backward
    return make_tensors(w.Tq, w.Tk, w.hq, w.hkv, w.d, seed=seed, with_dout=with_dout)


def random_slices(rng: np.random.Generator, Tq: int, Tk: int, max_slices: int = 6,
                  p_causal: float = 0.5, n_dummies: int = 0):
    """A random set of non-overlapping slices for property tests.

    The q axis is cut into disjoint row bands; each band gets up to two
    disjoint k intervals (so no (i, j) cell is covered twice).  Dummy
    ``[x, x]`` rows are inserted at random positions.
    """
    n_bands = int(rng.integers(1, max_slices + 1))
    cuts = np.sort(rng.choice(np.arange(1, Tq), size=min(n_bands - 1, Tq - 1), replace=False)) \
        if Tq > 1 else np.array([], dtype=int)
    bounds = [0] + [int(c) for c in cuts] + [Tq]
    qr, kr, ty = [], [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if rng.random() < 0.15:
            continue  # leave this band with no slice: its rows see nothing
        n_k = min(int(rng.integers(1, 3)), (Tk + 1) // 2)
        if n_k == 0:
            continue
        ks = np.sort(rng.choice(np.arange(0, Tk + 1), size=2 * n_k, replace=False))
        for t in range(n_k):
            k0, k1 = int(ks[2 * t]), int(ks[2 * t + 1])
            qr.append((a, b)); kr.append((k0, k1))
            ty.append(CAUSAL if rng.random() < p_causal else FULL)
    for _ in range(n_dummies):
        pos = int(rng.integers(0, len(qr) + 1))
        x = int(rng.integers(0, min(Tq, Tk) + 1))
        if rng.random() < 0.5:
            qd, kd = (x, x), (int(rng.integers(0, Tk // 2 + 1)), Tk)
        else:
            qd, kd = (0, Tq), (x, x)
        qr.insert(pos, qd); kr.insert(pos, kd); ty.insert(pos, int(rng.integers(0, 2)))
    return (np.asarray(qr, dtype=np.int32).reshape(-1, 2),
            np.asarray(kr, dtype=np.int32).reshape(-1, 2),
            np.asarray(ty, dtype=np.int32).reshape(-1))
