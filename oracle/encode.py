"""Dense visibility -> canonical compressed encodings and tile tables (oracle).

Test infrastructure only.  Every result here is derived from the dense boolean
mask, element by element, so that it can serve as the exact expected value for
the GPU encoder and tile classifier.

Canonical interval encoding (the FlashMask per-key-column row intervals, whose
lower/upper-triangle start/end naming the FlashMask rebuttal page relies on):
for column j let M_j = {i : not vis(i, j)}, split into maximal runs of
consecutive rows, ascending.
    no run          -> UT = [0, 0),  LT = [Sq, Sq)
    one run [a, b)  -> a == 0: UT = [0, b), LT = [Sq, Sq)
                       a >  0: UT = [0, 0), LT = [a, b)
    two runs        -> UT = first, LT = second
    more runs       -> not representable (NotRepresentable)
Stored int32 [4][Skv] in the order UTS, UTE, LTS, LTE.

Tile state of tile (qt, kt) at bm x bn, over rows [qt*bm, min(.., Sq)) and
columns [kt*bn, min(.., Skv)): SKIP (0) if nothing is visible, FULL (2) if all
is, else PARTIAL (1).  This is the skip / full / partial distinction the
FlashMask rebuttal draws (fully masked blocks need no computation) at the
kernel's "tiling block size".

Canonical bitmap encoding: 64 x 64 blocks, state recomputed from the bits,
PARTIAL blocks store 64 row words (bit c = column c of the block, bits outside
the matrix cleared) in a pool ordered row-major over (b, h, bi, bj); index -1
for blocks that are not PARTIAL.

Canonical selected-key lists: per query the valid entries (0 <= e < nblk),
distinct, ascending, padded with -1, and their count.
"""

import numpy as np

from .masks import BLOCK, FULL, PARTIAL, SKIP

FULL_BIT = np.int64(1) << 31


class NotRepresentable(ValueError):
    """A column has more than two masked runs."""


def masked_runs(col_masked):
    """Maximal runs [a, b) of True in a 1-D boolean array, ascending."""
    m = np.concatenate(([False], np.asarray(col_masked, dtype=bool), [False]))
    d = np.diff(m.astype(np.int8))
    starts = np.nonzero(d == 1)[0]
    ends = np.nonzero(d == -1)[0]
    return list(zip(starts.tolist(), ends.tolist()))


def canonical_from_runs(runs, sq):
    """(UTS, UTE, LTS, LTE) of one column from its ascending masked runs."""
    if not runs:
        return (0, 0, sq, sq)
    if len(runs) == 1:
        a, b = runs[0]
        return (0, b, sq, sq) if a == 0 else (0, 0, a, b)
    if len(runs) == 2:
        return (runs[0][0], runs[0][1], runs[1][0], runs[1][1])
    raise NotRepresentable(f"{len(runs)} masked runs")


def intervals_from_dense(vis, cols=None):
    """Canonical (UTS, UTE, LTS, LTE) int32 [4][len(cols)] of a dense mask [Sq, Skv].

    Column by column: split the masked rows into runs, then apply the rule above.
    """
    vis = np.asarray(vis, dtype=bool)
    sq, skv = vis.shape
    cols = range(skv) if cols is None else cols
    out = []
    for j in cols:
        try:
            out.append(canonical_from_runs(masked_runs(~vis[:, j]), sq))
        except NotRepresentable as e:
            raise NotRepresentable(f"column {j}: {e}") from None
    return np.array(out, dtype=np.int32).reshape(-1, 4).T.copy()


def intervals_from_dense_fast(vis):
    """intervals_from_dense for every column at once (for large masks)."""
    vis = np.asarray(vis, dtype=bool)
    sq, skv = vis.shape
    pad = np.zeros((1, skv), dtype=np.int8)
    d = np.diff(np.concatenate((pad, (~vis).view(np.int8), pad), axis=0), axis=0)
    up, down = d == 1, d == -1
    nruns = up.sum(axis=0)
    if (nruns > 2).any():
        j = int(np.nonzero(nruns > 2)[0][0])
        raise NotRepresentable(f"column {j}: {int(nruns[j])} masked runs")
    # d has Sq+1 rows: a run [a, b) gives d[a] = +1 and d[b] = -1.
    s1, e1 = up.argmax(axis=0), down.argmax(axis=0)            # first run
    last_up = sq - up[::-1].argmax(axis=0)                      # last run start
    last_down = sq - down[::-1].argmax(axis=0)                  # last run end
    out = np.empty((4, skv), dtype=np.int64)
    zero = nruns == 0
    one = nruns == 1
    two = nruns == 2
    out[:, zero] = np.array([0, 0, sq, sq])[:, None]
    a0 = one & (s1 == 0)
    an = one & (s1 != 0)
    out[0, a0], out[1, a0], out[2, a0], out[3, a0] = 0, e1[a0], sq, sq
    out[0, an], out[1, an], out[2, an], out[3, an] = 0, 0, s1[an], e1[an]
    out[0, two], out[1, two] = s1[two], e1[two]
    out[2, two], out[3, two] = last_up[two], last_down[two]
    return out.astype(np.int32)


def dense_from_intervals(iv, sq):
    """Visibility [Sq, Skv] of an interval encoding (masked iff in UT or LT)."""
    iv = np.asarray(iv, dtype=np.int64)
    r = np.arange(sq, dtype=np.int64)[:, None]
    masked = ((iv[0] <= r) & (r < iv[1])) | ((iv[2] <= r) & (r < iv[3]))
    return ~masked


def tile_states(vis, bm, bn):
    """Exact tile states uint8 [nqt][nkt] of a dense mask at tile size bm x bn."""
    vis = np.asarray(vis, dtype=bool)
    sq, skv = vis.shape
    nqt, nkt = -(-sq // bm), -(-skv // bn)
    out = np.zeros((nqt, nkt), dtype=np.uint8)
    for qt in range(nqt):
        band = vis[qt * bm: min(sq, (qt + 1) * bm)]
        for kt in range(nkt):
            t = band[:, kt * bn: min(skv, (kt + 1) * bn)]
            if t.all():
                out[qt, kt] = FULL
            elif t.any():
                out[qt, kt] = PARTIAL
    return out


def tile_states_fast(vis, bm, bn):
    """Same as tile_states, via padded reshapes (for large masks)."""
    vis = np.asarray(vis, dtype=bool)
    sq, skv = vis.shape
    nqt, nkt = -(-sq // bm), -(-skv // bn)
    anyv = np.zeros((nqt * bm, nkt * bn), dtype=bool)
    anyv[:sq, :skv] = vis
    allv = np.ones((nqt * bm, nkt * bn), dtype=bool)
    allv[:sq, :skv] = vis
    a = anyv.reshape(nqt, bm, nkt, bn).any(axis=(1, 3))
    f = allv.reshape(nqt, bm, nkt, bn).all(axis=(1, 3))
    out = np.where(f, FULL, np.where(a, PARTIAL, SKIP)).astype(np.uint8)
    return out


def tile_lists(states):
    """Per tile row: the non-SKIP kt ascending (FULL ones flagged with bit 31).

    Returns (lists int32 [nqt][nkt] padded with 0, counts int32 [nqt]).
    """
    states = np.asarray(states)
    nqt, nkt = states.shape
    lists = np.zeros((nqt, nkt), dtype=np.int64)
    counts = np.zeros(nqt, dtype=np.int32)
    for qt in range(nqt):
        ks = np.nonzero(states[qt] != SKIP)[0]
        vals = ks.astype(np.int64) | np.where(states[qt, ks] == FULL, FULL_BIT, 0)
        lists[qt, : ks.size] = vals
        counts[qt] = ks.size
    return lists.astype(np.uint32).view(np.int32), counts


def tile_order(counts, slice_rows=None):
    """Tile-row indices by decreasing count, ties by increasing index, within
    each slice of `slice_rows` consecutive rows (one mask slice of the table),
    the slices in turn; one slice of all rows if slice_rows is None.  (The
    pages fix no order of tile rows; any order computes the same result.)"""
    counts = np.asarray(counts, dtype=np.int64).ravel()
    n = counts.size
    step = n if not slice_rows else int(slice_rows)
    out = []
    for lo in range(0, n, max(step, 1)):
        idx = np.arange(lo, min(lo + step, n))
        out.append(idx[np.lexsort((idx, -counts[idx]))])
    return (np.concatenate(out) if out else np.zeros(0, np.int64)).astype(np.int32)


def bitmap_from_dense(vis, blk=BLOCK):
    """Canonical block bitmap of one dense mask: (state, index, words list)."""
    vis = np.asarray(vis, dtype=bool)
    sq, skv = vis.shape
    nbq, nbk = -(-sq // blk), -(-skv // blk)
    state = np.zeros((nbq, nbk), dtype=np.uint8)
    index = np.full((nbq, nbk), -1, dtype=np.int32)
    pool = []
    weights = np.uint64(1) << np.arange(blk, dtype=np.uint64)
    for bi in range(nbq):
        for bj in range(nbk):
            t = vis[bi * blk: min(sq, (bi + 1) * blk), bj * blk: min(skv, (bj + 1) * blk)]
            if t.all():
                state[bi, bj] = FULL
            elif t.any():
                state[bi, bj] = PARTIAL
                words = np.zeros(blk, dtype=np.uint64)
                words[: t.shape[0]] = (t * weights[: t.shape[1]]).sum(axis=1, dtype=np.uint64)
                index[bi, bj] = len(pool)
                pool.append(words)
    return state, index, pool


def canonical_lists(sel, nblk):
    """Canonical selected-key lists: valid, distinct, ascending, -1 padded."""
    sel = np.asarray(sel)
    n = sel.shape[-1]
    flat = sel.reshape(-1, n)
    lists = np.full(flat.shape, -1, dtype=np.int32)
    counts = np.zeros(flat.shape[0], dtype=np.int32)
    for q in range(flat.shape[0]):
        vals = sorted({int(e) for e in flat[q] if 0 <= e < nblk})
        lists[q, : len(vals)] = vals
        counts[q] = len(vals)
    return lists.reshape(sel.shape), counts.reshape(sel.shape[:-1])
