"""Plain fp64 CPU oracle for range-masked ("flex") attention.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
bench's CPU-baseline leg may import this module.  The library never calls it
and shares no code with it.

Everything here is written for clarity, not speed: the mask is materialised
as an explicit integer matrix, scores are formed with a dense matmul over the
keys a block of rows can see, and softmax is taken per row in float64.
Inputs are bf16 values upcast exactly to float64.

What is computed, and where the pages define it:

* Slices.  ``q_ranges[r] = [qs, qe)``, ``k_ranges[r] = [ks, ke)``,
  ``attn_type_map[r]`` 0 = FULL, 1 = CAUSAL (MagiAttention issue "Using
  dummy/padded attention slices with flex_flash_attn_func for torch.compile
  static shapes", reporter's repro script).  A slice whose q range or k range
  is empty has zero area and is ignored (same issue, maintainer reply,
  padding mechanism: "a rectangle in the attention map").
* CAUSAL alignment.  The pages do not spell it out; the repro script's slice
  ``q=[1024,2048) x k=[0,2048)`` is ordinary causal attention over the whole
  prefix only if the causal diagonal is anchored at the bottom-right corner of
  the slice rectangle.  So cell (i, j) of a CAUSAL slice is visible iff
  ``j - ke <= i - qe``.
* Scores: ``u = scale * q . k``; optional softcap ``s = c * tanh(u / c)``
  (softcapping limits logit growth: FlexAttention paper summary, section 2,
  attention variants); masked cells are -inf after the cap.
* Optional distance bias (ALiBi): the pages list ALiBi as a variant that
  adds a bias depending on the distance between query and key positions
  (FlexAttention paper summary, section 2, attention variants; section 3.1,
  a position-dependent score bias) and give no formula.  Read here as the
  linear form ``s += slope[h] * (j - i)`` with one slope per q head, i and j
  the token indices along the q and k axes, added after the softcap and
  before the mask.  With slope > 0 on a causal mask (j <= i) it is the usual
  ALiBi penalty ``-slope * (i - j)``.
* Output and log-sum-exp per row (natural log).  A row that sees no key gets
  out = 0 and lse = -inf.
* GQA: q head h reads kv head ``h // (hq // hkv)`` (repro script: 8 q heads,
  2 kv heads).
* Tile lists: for each (q-tile, k-tile) pair and each slice, the tile is
  listed if the slice makes at least one of its cells visible; it is FULL if
  the slice makes every cell of the whole BM x BN tile visible and PARTIAL
  otherwise (FlexAttention paper summary, section 4, block sparsity and the
  full-block optimisation).
"""
from __future__ import annotations

import numpy as np

FULL = 0
CAUSAL = 1


# --------------------------------------------------------------------------
# slices and the visibility matrix
# --------------------------------------------------------------------------
def normalise_slices(q_ranges, k_ranges, types, Tq: int, Tk: int):
    """Validate a slice list and return the non-empty slices.

    Returns a list of ``(r, qs, qe, ks, ke, type)`` with ``r`` the slice's
    position in the caller's list.  Raises ``ValueError`` for ``start > end``,
    ranges outside the token axis and unknown types.  Empty slices (``start
    == end`` on either axis) are dropped: they cover no cell.
    """
    q_ranges = np.asarray(q_ranges, dtype=np.int64).reshape(-1, 2)
    k_ranges = np.asarray(k_ranges, dtype=np.int64).reshape(-1, 2)
    types = np.asarray(types, dtype=np.int64).reshape(-1)
    if not (q_ranges.shape[0] == k_ranges.shape[0] == types.shape[0]):
        raise ValueError("q_ranges, k_ranges and attn_type_map disagree in length")
    out = []
    for r in range(q_ranges.shape[0]):
        qs, qe = int(q_ranges[r, 0]), int(q_ranges[r, 1])
        ks, ke = int(k_ranges[r, 0]), int(k_ranges[r, 1])
        t = int(types[r])
        if not (0 <= qs <= qe <= Tq) or not (0 <= ks <= ke <= Tk):
            raise ValueError(f"slice {r}: range out of bounds or start > end")
        if t not in (FULL, CAUSAL):
            raise ValueError(f"slice {r}: unknown attention type {t}")
        if qs == qe or ks == ke:
            continue
        out.append((r, qs, qe, ks, ke, t))
    return out


def slice_cells(sl, rows, cols):
    """Boolean matrix: which cells (rows x cols) slice ``sl`` makes visible."""
    _, qs, qe, ks, ke, t = sl
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    cell = ((rows >= qs) & (rows < qe))[:, None] & ((cols >= ks) & (cols < ke))[None, :]
    if t == CAUSAL:
        cell &= (cols[None, :] - ke) <= (rows[:, None] - qe)
    return cell


def visibility(slices, rows, cols):
    """Multiplicity matrix M[len(rows), len(cols)]: how many slices cover each cell."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    M = np.zeros((len(rows), len(cols)), dtype=np.int32)
    for sl in slices:
        _, qs, qe, ks, ke, _t = sl
        # a slice whose rectangle misses these rows or these columns adds
        # nothing; skipping it only saves the work of adding zeros
        if not (np.any((rows >= qs) & (rows < qe)) and np.any((cols >= ks) & (cols < ke))):
            continue
        M += slice_cells(sl, rows, cols)
    return M


def visible_count(slices, Tq: int, Tk: int, block: int = 1024) -> int:
    """Number of visible (i, j) cells, counted on the materialised mask."""
    n = 0
    for r0 in range(0, Tq, block):
        rows = np.arange(r0, min(Tq, r0 + block))
        n += int((visibility(slices, rows, np.arange(Tk)) > 0).sum())
    return n


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def _row_block_attention(q, k, v, slices, scale, softcap, rows, Tk, alibi_slopes=None, heads=None):
    """Scores, probabilities, output and lse for one block of rows.

    Returns (cols, vis, s, p, out, lse) per q head, where ``cols`` are the key
    columns that any row of the block can see (found on the materialised
    mask), ``s`` the masked scores (-inf where invisible) and ``p`` the
    softmax probabilities.  ``heads`` (a set of q heads, or None for all)
    limits the work to those heads; the others get None.
    """
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    grp = hq // hkv
    M = visibility(slices, rows, np.arange(Tk))
    if M.size and M.max() > 1:
        raise ValueError("slices overlap: a cell is covered more than once")
    vis = M > 0
    cols = np.nonzero(vis.any(axis=0))[0]
    vis = vis[:, cols]
    res = []
    for h in range(hq):
        g = h // grp
        if cols.size == 0 or (heads is not None and h not in heads):
            res.append(None)
            continue
        u = scale * (q[rows, h, :] @ k[cols, g, :].T)
        s = softcap * np.tanh(u / softcap) if softcap > 0 else u
        if alibi_slopes is not None:
            s = s + alibi_slopes[h] * (cols[None, :] - rows[:, None]).astype(np.float64)
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        has = np.isfinite(m)
        p = np.exp(s - np.where(has, m, 0.0)[:, None])
        l = p.sum(axis=1)
        o = (p @ v[cols, g, :]) / np.where(has, l, 1.0)[:, None]
        out = np.where(has[:, None], o, 0.0)
        lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
        p = p / np.where(has, l, 1.0)[:, None]
        res.append((s, p, out, lse, u))
    return cols, vis, res


def _slopes(alibi_slopes, hq):
    if alibi_slopes is None:
        return None
    a = np.asarray(alibi_slopes, dtype=np.float64).reshape(-1)
    if a.size != hq:
        raise ValueError("alibi_slopes needs one slope per q head")
    return a


def _head_sets(hq, hkv, kv_heads):
    """(q heads, kv heads) to compute: every head when kv_heads is None, else
    the listed kv heads and the q heads that read them, in increasing order."""
    grp = hq // hkv
    if kv_heads is None:
        return list(range(hq)), list(range(hkv))
    kvh = sorted(set(int(g) for g in kv_heads))
    if any(g < 0 or g >= hkv for g in kvh):
        raise ValueError("kv_heads out of range")
    return [h for h in range(hq) if h // grp in kvh], kvh


def attention_fwd(q, k, v, q_ranges, k_ranges, types, scale, softcap=0.0,
                  rows=None, block=256, alibi_slopes=None, kv_heads=None):
    """Forward pass: ``out [n, hq, d]`` and ``lse [n, hq]`` for ``rows``.

    ``q`` is [Tq, hq, d], ``k`` and ``v`` are [Tk, hkv, d] (float64 arrays).
    ``rows`` selects which query rows to compute (all rows when None).
    ``alibi_slopes`` ([hq] or None): the distance bias described above.
    ``kv_heads`` (None = all) computes only the q heads that read the listed
    kv heads; the head axis of the results then holds those q heads in
    increasing order.  Every head is computed independently, so this only
    leaves work out.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, hq, d = q.shape
    Tk = k.shape[0]
    if hq % k.shape[1] != 0:
        raise ValueError("hq must be a multiple of hkv")
    if softcap < 0:
        raise ValueError("softcap must be >= 0")
    slices = normalise_slices(q_ranges, k_ranges, types, Tq, Tk)
    slopes = _slopes(alibi_slopes, hq)
    qheads, _ = _head_sets(hq, k.shape[1], kv_heads)
    hpos = {h: i for i, h in enumerate(qheads)}
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, len(qheads), d))
    lse = np.full((rows.size, len(qheads)), -np.inf)
    for b0 in range(0, rows.size, block):
        rb = rows[b0:b0 + block]
        _, _, res = _row_block_attention(q, k, v, slices, scale, softcap, rb, Tk, slopes, set(qheads))
        for h, r in enumerate(res):
            if r is None:
                continue
            out[b0:b0 + rb.size, hpos[h], :] = r[2]
            lse[b0:b0 + rb.size, hpos[h]] = r[3]
    return out, lse


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def attention_bwd(q, k, v, dout, q_ranges, k_ranges, types, scale, softcap=0.0,
                  rows=None, keys=None, block=256, magnitudes=False, alibi_slopes=None,
                  kv_heads=None):
    """Gradients of ``sum(dout * out)``: dq at ``rows``, dk and dv at ``keys``.

    Chain rule through the forward above, in the usual flash-attention form:
    ``P = softmax(s)``, ``dV = P^T dO``, ``dP = dO V^T``,
    ``D = rowsum(dO * out)``, ``dS = P * (dP - D)``, the softcap derivative
    ``1 - tanh^2(u / c)``, ``dQ = scale * dU K``, ``dK = scale * dU^T Q``.  The
    distance bias is a constant added to the scores: it changes P and nothing
    else in these formulas.
    GQA: dk and dv of a kv head sum over the q heads that read it.
    Returns (dq [len(rows), hq, d], dk [len(keys), hkv, d], dv [len(keys), hkv, d]).
    ``kv_heads`` (None = all) computes only the listed kv heads and the q
    heads that read them (every one of them, so dk and dv of a listed kv head
    are complete); the head axes then hold those heads in increasing order.

    With ``magnitudes=True`` it also returns, per gradient element, the scale
    of the rounding error an implementation in rounded arithmetic can carry:
    the sum of the absolute values of the terms that add up to it, where the
    row term D is taken as uncertain by A_i = sum_d |dO_id| (|out_id| +
    (P|V|)_id) (D is formed from a rounded copy of out):
      dq: scale (|dU| + P A) |K|,  dk: scale (|dU| + P A)^T |Q|,  dv: P^T |dO|.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    Tq, hq, d = q.shape
    Tk, hkv, _ = k.shape
    grp = hq // hkv
    slices = normalise_slices(q_ranges, k_ranges, types, Tq, Tk)
    slopes = _slopes(alibi_slopes, hq)
    qheads, kvheads = _head_sets(hq, hkv, kv_heads)
    hpos = {h: i for i, h in enumerate(qheads)}
    gpos = {g: i for i, g in enumerate(kvheads)}
    rows = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(Tk) if keys is None else np.asarray(keys, dtype=np.int64)

    # rows whose gradient terms we need: the requested dq rows, plus every row
    # that sees one of the requested keys (for dk, dv)
    key_pos = np.full(Tk, -1, dtype=np.int64)
    key_pos[keys] = np.arange(keys.size)
    sees_key = np.zeros(Tq, dtype=bool)
    for r0 in range(0, Tq, 1024):
        rb = np.arange(r0, min(Tq, r0 + 1024))
        sees_key[rb] = (visibility(slices, rb, keys) > 0).any(axis=1)
    want_dq = np.zeros(Tq, dtype=bool)
    want_dq[rows] = True
    dq_pos = np.full(Tq, -1, dtype=np.int64)
    dq_pos[rows] = np.arange(rows.size)
    work = np.nonzero(sees_key | want_dq)[0]

    dq = np.zeros((rows.size, len(qheads), d))
    dk = np.zeros((keys.size, len(kvheads), d))
    dv = np.zeros((keys.size, len(kvheads), d))
    if magnitudes:
        dq_m, dk_m, dv_m = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for b0 in range(0, work.size, block):
        rb = work[b0:b0 + block]
        cols, vis, res = _row_block_attention(q, k, v, slices, scale, softcap, rb, Tk, slopes, set(qheads))
        if cols.size == 0:
            continue
        kp = key_pos[cols]
        kmask = kp >= 0
        dq_rows = dq_pos[rb]
        dq_mask = dq_rows >= 0
        for h in qheads:
            g = h // grp
            hi, gi = hpos[h], gpos[g]
            s, p, out, lse, u = res[h]
            do = dout[rb, h, :]
            D = (do * out).sum(axis=1)
            dP = do @ v[cols, g, :].T
            dS = p * (dP - D[:, None])
            if softcap > 0:
                dU = dS * (1.0 - np.tanh(u / softcap) ** 2)
            else:
                dU = dS
            if dq_mask.any():
                dq[dq_rows[dq_mask], hi, :] += scale * (dU[dq_mask] @ k[cols, g, :])
            if kmask.any():
                dv[kp[kmask], gi, :] += p[:, kmask].T @ do
                dk[kp[kmask], gi, :] += scale * (dU[:, kmask].T @ q[rb, h, :])
            if magnitudes:
                A = (np.abs(do) * (np.abs(out) + p @ np.abs(v[cols, g, :]))).sum(axis=1)
                dU_abs = np.abs(dU) + p * A[:, None]
                if dq_mask.any():
                    dq_m[dq_rows[dq_mask], hi, :] += scale * (dU_abs[dq_mask] @ np.abs(k[cols, g, :]))
                if kmask.any():
                    dv_m[kp[kmask], gi, :] += p[:, kmask].T @ np.abs(do)
                    dk_m[kp[kmask], gi, :] += scale * (dU_abs[:, kmask].T @ np.abs(q[rb, h, :]))
    if magnitudes:
        return dq, dk, dv, (dq_m, dk_m, dv_m)
    return dq, dk, dv


# --------------------------------------------------------------------------
# block lists (BlockMask-style masks)
# --------------------------------------------------------------------------
def block_visibility(kv_num_blocks, kv_indices, block_q: int, block_k: int, Tq: int, Tk: int):
    """Boolean [Tq, Tk]: cell (i, j) is visible iff k block j // block_k is
    among the first kv_num_blocks[b] entries of kv_indices[b], b = i // block_q.

    FlexAttention paper summary, section 4 (block sparsity): the BlockMask
    keeps, per query block, the number of non-masked key blocks and their
    indices, which need not be contiguous.  Here every listed block is fully
    visible (no per-cell mask function runs inside a block).
    """
    num = np.asarray(kv_num_blocks, dtype=np.int64).reshape(-1)
    idx = np.asarray(kv_indices, dtype=np.int64).reshape(num.size, -1)
    n_qb = -(-Tq // block_q)
    n_kb = -(-Tk // block_k)
    if num.size != n_qb:
        raise ValueError("kv_num_blocks needs one count per query block")
    vis = np.zeros((Tq, Tk), dtype=bool)
    for b in range(n_qb):
        if not 0 <= num[b] <= idx.shape[1]:
            raise ValueError(f"query block {b}: count out of range")
        listed = idx[b, :num[b]]
        if np.any(listed < 0) or np.any(listed >= n_kb):
            raise ValueError(f"query block {b}: key block index out of range")
        if np.unique(listed).size != listed.size:
            raise ValueError(f"query block {b}: key block listed twice")
        for kb in listed:
            vis[b * block_q:(b + 1) * block_q, kb * block_k:(kb + 1) * block_k] = True
    return vis


def block_slices_plain(kv_num_blocks, kv_indices, block_q: int, block_k: int, Tq: int, Tk: int):
    """The same block list as one FULL slice per listed block (no merging):
    (q_ranges, k_ranges, types) for the slice-based functions above."""
    num = np.asarray(kv_num_blocks, dtype=np.int64).reshape(-1)
    idx = np.asarray(kv_indices, dtype=np.int64).reshape(num.size, -1)
    qr, kr = [], []
    for b in range(num.size):
        for kb in idx[b, :num[b]]:
            qr.append((b * block_q, min(Tq, (b + 1) * block_q)))
            kr.append((int(kb) * block_k, min(Tk, (int(kb) + 1) * block_k)))
    n = len(qr)
    return (np.array(qr, dtype=np.int64).reshape(n, 2), np.array(kr, dtype=np.int64).reshape(n, 2),
            np.zeros(n, dtype=np.int64))


def attention_fwd_masked(q, k, v, vis, scale, softcap=0.0):
    """Forward pass under an explicit boolean mask ``vis`` [Tq, Tk]: the same
    scores, softcap and softmax as ``attention_fwd``, every row at once."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, hq, d = q.shape
    grp = hq // k.shape[1]
    out = np.zeros((Tq, hq, d))
    lse = np.full((Tq, hq), -np.inf)
    has = vis.any(axis=1)
    for h in range(hq):
        g = h // grp
        u = scale * (q[:, h, :] @ k[:, g, :].T)
        s = softcap * np.tanh(u / softcap) if softcap > 0 else u
        s = np.where(vis, s, -np.inf)
        m = np.where(has, s.max(axis=1), 0.0)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        out[:, h, :] = np.where(has[:, None], (p @ v[:, g, :]) / np.where(has, l, 1.0)[:, None], 0.0)
        lse[:, h] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return out, lse


# --------------------------------------------------------------------------
# tile lists
# --------------------------------------------------------------------------
def tile_set(q_ranges, k_ranges, types, Tq: int, Tk: int, BM: int, BN: int):
    """The set of ``(q_tile, k_tile, r, kind)`` a block-sparse kernel must visit.

    ``kind`` is FULL (0) when slice r makes every cell of the whole BM x BN
    tile visible, else PARTIAL (1).  Computed by materialising each slice's
    cells over the tiles its rectangle touches and counting per tile.
    """
    slices = normalise_slices(q_ranges, k_ranges, types, Tq, Tk)
    out = set()
    for sl in slices:
        r, qs, qe, ks, ke, t = sl
        qt0, qt1 = qs // BM, (qe - 1) // BM + 1
        kt0, kt1 = ks // BN, (ke - 1) // BN + 1
        cols = np.arange(kt0 * BN, kt1 * BN)
        for qt in range(qt0, qt1):
            rows = np.arange(qt * BM, (qt + 1) * BM)
            cells = slice_cells(sl, rows, cols)  # rows past Tq / cols past Tk never match
            counts = cells.reshape(BM, kt1 - kt0, BN).sum(axis=(0, 2))
            for i, c in enumerate(counts):
                if c == 0:
                    continue
                kind = 0 if c == BM * BN else 1
                out.add((qt, kt0 + i, r, kind))
    return out
